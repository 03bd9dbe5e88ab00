"""Seeded synthetic inputs for the MoE token shuffle.

Holds only input generation (a router stand-in and random activations); none
of the shuffle's own arithmetic.  Both the HIP path's tests/benchmark and the
CPU oracle take their inputs from here.

The five workloads follow the shapes named for this path: a tiny correctness
case, a Qwen3-30B-A3B-shaped prefill, a low-latency decode batch with FP8
group quantisation, a DeepSeek-V3-shaped prefill with Zipf expert popularity,
masked entries and 128-row expert alignment, and a long-sequence prefill run
as four 8192-token rounds with per-token int8 quantisation.  The model names
stand for shapes only; no weights or datasets are involved.
"""
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

QUANT_NONE, QUANT_FP8, QUANT_INT8, QUANT_MXFP4 = 0, 1, 2, 3
SCALE_FP32, SCALE_POW2, SCALE_UE8M0 = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    num_ranks: int
    num_topk: int
    expert_alignment: int = 1
    quant: int = QUANT_NONE
    quant_group: int = 0          # elements per scale; 0 = not quantised
    mask_prob: float = 0.0
    routing: str = "uniform"      # uniform | softmax_topk | zipf | zipf_permuted | group_limited
    weights: str = "softmax"      # softmax (renormalised over chosen k) | raw (the router's own)
    zipf_s: float = 1.2
    rounds: int = 1
    seed: int = 0
    ranks_per_node: int = 8
    expert_capacity: int = 0      # >0: fixed-capacity receive layout
    num_sources: int = 1          # >1: the batch stacks this many source ranks
    scale_mode: int = SCALE_FP32  # FP8 / int8 scale format
    combine_quant: int = QUANT_NONE   # expert outputs arrive as FP8 / int8 codes
    combine_group: int = 0        # elements per expert-output scale
    non_expand: bool = False      # one receive row per (token, rank) instead of per (token, k)
    expert_groups: int = 32       # group_limited routing: expert groups ...
    topk_groups: int = 4          # ... of which each token uses this many

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 128, 256, 16, 4, 2, routing="softmax_topk", weights="raw",
                     seed=1001),
    "qwen3_30b_a3b_prefill": Workload("qwen3_30b_a3b_prefill", 4096, 2048, 128, 16, 8,
                                      seed=1002),
    "ll_decode_fp8": Workload("ll_decode_fp8", 128, 7168, 256, 16, 8, quant=QUANT_FP8,
                              quant_group=128, seed=1003),
    "deepseek_v3_prefill": Workload("deepseek_v3_prefill", 8192, 7168, 256, 16, 8,
                                    expert_alignment=128, mask_prob=0.05, routing="zipf",
                                    seed=1004),
    "long_seq_int8": Workload("long_seq_int8", 32768, 4096, 64, 8, 6, quant=QUANT_INT8,
                              quant_group=4096, rounds=4, seed=1005),
    # the same shape with the Zipf popularity spread over the experts by a
    # seeded permutation, so the hot experts no longer sit on rank 0
    "deepseek_v3_prefill_permuted": Workload("deepseek_v3_prefill_permuted", 8192, 7168, 256, 16,
                                             8, expert_alignment=128, mask_prob=0.05,
                                             routing="zipf_permuted", seed=1007),
    # DeepSeek-V3 gating (256 experts in 32 groups, top-4 groups, top-2 per
    # group) with the non-expand dispatch that sends a token once per rank
    "deepseek_v3_group_limited": Workload("deepseek_v3_group_limited", 8192, 7168, 256, 16, 8,
                                          routing="group_limited", weights="raw",
                                          non_expand=True, seed=1006),
}


def _softmax(z, axis=-1):
    with np.errstate(invalid="ignore", divide="ignore"):
        z = z - z.max(axis=axis, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=axis, keepdims=True)


def _group_limited(logits, n_groups, topk_groups, K):
    """Group-limited gating ("DeepEP V1 vs V2 深度对比分析" §8.1: experts in
    groups, each token picks its top groups, then the top experts inside
    each picked group).  Readings where the page is silent: affinity =
    sigmoid(logit); a group's score is the sum of its best K/topk_groups
    affinities (the ones it would contribute); ties go to the lower id; the
    chosen experts are listed by affinity, highest first; weights are their
    affinities normalised to sum 1."""
    N, E = logits.shape
    per = K // topk_groups
    aff = 1.0 / (1.0 + np.exp(-logits))
    g = aff.reshape(N, n_groups, E // n_groups)
    top_in_group = -np.sort(-g, axis=2)[:, :, :per]
    gscore = top_in_group.sum(axis=2)
    gsel = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_groups]
    allowed = np.zeros((N, n_groups), bool)
    np.put_along_axis(allowed, gsel, True, axis=1)
    masked = np.where(np.repeat(allowed, E // n_groups, axis=1), aff, -np.inf)
    # the best `per` experts of every group, then the K best of those (all
    # from the allowed groups, `per` from each)
    order = np.argsort(-masked.reshape(N, n_groups, E // n_groups), axis=2, kind="stable")[:, :, :per]
    base = (np.arange(n_groups) * (E // n_groups))[None, :, None]
    cand = (order + base).reshape(N, -1)                 # [N, n_groups*per]
    cand_aff = np.take_along_axis(masked, cand, axis=1)
    pick = np.argsort(-cand_aff, axis=1, kind="stable")[:, :K]
    idx = np.take_along_axis(cand, pick, axis=1)
    w = np.take_along_axis(aff, idx, axis=1)
    return idx, w / w.sum(axis=1, keepdims=True)


def routing(w: Workload, num_tokens: Optional[int] = None):
    """Returns (topk_idx int32 [N,K], topk_weights float32 [N,K])."""
    N = w.num_tokens if num_tokens is None else num_tokens
    E, K = w.num_experts, w.num_topk
    rng = np.random.Generator(np.random.PCG64(w.seed))
    if w.routing == "softmax_topk":
        p = _softmax(rng.standard_normal((N, E)))
        idx = np.argsort(-p, axis=1, kind="stable")[:, :K]
        wts = np.take_along_axis(p, idx, axis=1)
    elif w.routing == "uniform":
        idx = np.argsort(rng.random((N, E)), axis=1, kind="stable")[:, :K]
        wts = None
    elif w.routing == "group_limited":
        idx, wts = _group_limited(rng.standard_normal((N, E)), w.expert_groups, w.topk_groups, K)
    elif w.routing in ("zipf", "zipf_permuted"):
        # p_e proportional to (rank_e + 1)^-s; rank_e = e, or a seeded
        # permutation of the experts
        rank = rng.permutation(E) if w.routing == "zipf_permuted" else np.arange(E)
        logp = -w.zipf_s * np.log(rank.astype(np.float64) + 1.0)
        gumbel = -np.log(-np.log(rng.random((N, E))))
        idx = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :K]
        wts = None
    else:
        raise ValueError(w.routing)
    idx = idx.astype(np.int32)
    if w.mask_prob > 0:
        idx[rng.random((N, K)) < w.mask_prob] = -1
    if wts is None or w.weights == "softmax":
        logits = rng.standard_normal((N, K))
        logits[idx < 0] = -np.inf
        wts = _softmax(logits)
        wts[~np.isfinite(wts)] = 0.0
    return np.ascontiguousarray(idx), np.ascontiguousarray(wts.astype(np.float32))


def activations(rows: int, hidden: int, seed: int, device="cpu"):
    """bf16 [rows, hidden] drawn N(0,1) in fp32 by torch's seeded generator on
    `device`, rounded to bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((rows, hidden), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def x_seed(w: Workload) -> int:
    return w.seed * 10 + 1


def y_seed(w: Workload) -> int:
    return w.seed * 10 + 2


def round_ranges(num_tokens: int, rounds: int):
    """Token ranges [begin, end) of `rounds` equal rounds (the last takes the
    remainder)."""
    per = max(-(-num_tokens // rounds), 1)
    return [(b, min(b + per, num_tokens)) for b in range(0, num_tokens, per)] or [(0, 0)]
