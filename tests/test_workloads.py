"""The seeded input generators (workloads.py) produce the routing and
activations their recipe states: distinct experts per row, the masking
rate, Zipf popularity, group-limited choices, weights that sum to one where
renormalised, N(0,1) activations rounded to bf16, and rounds that partition
the tokens.  CPU only."""
import numpy as np
import pytest
import torch

import workloads as W


def _distinct_valid(idx, E):
    for row in idx:
        v = row[row >= 0]
        assert len(np.unique(v)) == len(v)
        assert v.min(initial=0) >= 0 and v.max(initial=0) < E


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_prefill", "ll_decode_fp8", "long_seq_int8"])
def test_uniform_routing(name):
    w = W.WORKLOADS[name]
    n = min(w.num_tokens, 8192)
    idx, wts = W.routing(w, n)
    assert idx.shape == (n, w.num_topk) and idx.dtype == np.int32
    assert wts.shape == (n, w.num_topk) and wts.dtype == np.float32
    _distinct_valid(idx, w.num_experts)
    assert (idx >= 0).all()
    # renormalised softmax weights
    assert np.allclose(wts.sum(axis=1), 1.0, atol=1e-5) and (wts > 0).all()
    # uniform: every expert's share within 5 sigma of K/E
    cnt = np.bincount(idx.ravel(), minlength=w.num_experts)
    mean = n * w.num_topk / w.num_experts
    assert np.abs(cnt - mean).max() < 5 * np.sqrt(mean)


def test_zipf_masked_routing():
    w = W.WORKLOADS["deepseek_v3_prefill"]
    idx, wts = W.routing(w)
    _distinct_valid(idx, w.num_experts)
    masked = (idx < 0).mean()
    assert abs(masked - w.mask_prob) < 0.005
    assert (wts[idx < 0] == 0).all()
    live = (idx >= 0).any(axis=1)
    assert np.allclose(wts[live].sum(axis=1), 1.0, atol=1e-5)
    # popularity falls with the expert id (Zipf over the un-permuted ids)
    cnt = np.bincount(idx[idx >= 0], minlength=w.num_experts)
    assert cnt[0] == cnt.max()
    assert cnt[0] > cnt[15] > cnt[255]
    # the hottest expert takes about 7.2k of the 8192 rows (close to every
    # token: Gumbel top-8 of a (e+1)^-1.2 popularity)
    assert 6500 < cnt[0] < 7800


def test_permuted_zipf_routing():
    """The permuted variant: the same popularity law over a seeded
    permutation of the experts, so sorted counts match the un-permuted
    workload's closely while the hot experts spread over the ranks."""
    w = W.WORKLOADS["deepseek_v3_prefill_permuted"]
    idx, wts = W.routing(w)
    _distinct_valid(idx, w.num_experts)
    assert abs((idx < 0).mean() - w.mask_prob) < 0.005
    cnt = np.bincount(idx[idx >= 0], minlength=w.num_experts)
    ref_idx, _ = W.routing(W.WORKLOADS["deepseek_v3_prefill"])
    ref = np.bincount(ref_idx[ref_idx >= 0], minlength=w.num_experts)
    srt, rsrt = np.sort(cnt)[::-1], np.sort(ref)[::-1]
    assert np.abs(srt - rsrt).max() < 0.05 * rsrt[0] + 5 * np.sqrt(rsrt[0])
    assert cnt.argmax() != 0                       # the hottest expert moved
    nle = w.num_experts // w.num_ranks
    per_rank = cnt.reshape(w.num_ranks, nle).sum(axis=1)
    ref_rank = ref.reshape(w.num_ranks, nle).sum(axis=1)
    assert per_rank.max() < ref_rank.max()         # rank 0 no longer takes the hot block


def test_softmax_topk_routing_raw_weights():
    w = W.WORKLOADS["tiny"]
    idx, wts = W.routing(w)
    _distinct_valid(idx, w.num_experts)
    # raw top-2 softmax probabilities: decreasing along k, summing below 1
    assert (wts[:, 0] >= wts[:, 1]).all()
    assert (wts.sum(axis=1) < 1.0).all() and (wts > 0).all()


def test_group_limited_routing():
    w = W.WORKLOADS["deepseek_v3_group_limited"]
    idx, wts = W.routing(w, 4096)
    _distinct_valid(idx, w.num_experts)
    per_group = w.num_experts // w.expert_groups
    groups = idx // per_group
    for row in groups:
        g, c = np.unique(row, return_counts=True)
        assert len(g) == w.topk_groups
        assert (c == w.num_topk // w.topk_groups).all()
    assert np.allclose(wts.sum(axis=1), 1.0, atol=1e-5)
    assert (np.diff(wts, axis=1) <= 0).all()   # listed by affinity, highest first


def test_activations_bf16_normal():
    x = W.activations(4096, 512, 7)
    assert x.dtype == torch.bfloat16 and x.shape == (4096, 512)
    v = x.float()
    assert abs(v.mean().item()) < 0.01 and abs(v.std().item() - 1.0) < 0.01
    assert torch.equal(x, W.activations(4096, 512, 7))          # seeded
    assert not torch.equal(x, W.activations(4096, 512, 8))


@pytest.mark.parametrize("n,r", [(32768, 4), (10, 3), (7, 7), (5, 8), (0, 4)])
def test_round_ranges_partition(n, r):
    rr = W.round_ranges(n, r)
    assert rr[0][0] == 0 and rr[-1][1] == n
    for (a, b), (c, d) in zip(rr, rr[1:]):
        assert b == c and a < b
    assert len(rr) <= max(r, 1)
