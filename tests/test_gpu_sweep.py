"""GPU parity over seeded random configurations.

Each case draws a configuration the ABI accepts (ranks, experts per rank,
top-k, hidden size, alignment, masking, repeated experts, per-node grouping,
fixed capacity, stacked sources, non-expand, dispatch and combine
quantisation) and runs it through one pipeline: the separate calls, the
one-call layout + dispatch, or the merged calls over a sequence of batches;
the separate calls may split the batch into token rounds on one handle.
Every output is held to the same bars as the hand-picked cases (layout,
slots and bf16 rows bit-exact, codes within one step with scales exact,
combine within one bf16 ulp plus the fp32 chain bound).  Sizes stay small
enough for the oracle yet reach every layout path: the one-block layout,
count + finish, and count + scan + slots.
"""
import os

import numpy as np
import pytest

import workloads as W
from shuffle_check import run_and_check, run_overlap_sequence

PIPELINES = ("serial", "fused", "merged")
# EP_SWEEP_CASES widens the sweep (the draws are a pure function of the case
# number, so a wider run repeats the default cases first)
NUM_CASES = int(os.environ.get("EP_SWEEP_CASES", "60"))


def _draw(i):
    """The i-th configuration: a Workload, the pipeline, the batch sizes and
    whether rows repeat experts.  Pure function of i."""
    rng = np.random.Generator(np.random.PCG64(9100 + i))
    pipeline = PIPELINES[i % 3]
    R = int(rng.choice([1, 2, 4, 8, 12, 16, 32, 64, 256, 1024]))
    nle = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    while R * nle > 1024:
        nle //= 2
    nle = max(nle, 1)
    E = R * nle
    K = int(rng.integers(1, min(16, E) + 1))
    quant = int(rng.choice([W.QUANT_NONE] * 3 + [W.QUANT_FP8, W.QUANT_INT8, W.QUANT_MXFP4]))
    if quant == W.QUANT_MXFP4:
        H, group = 32 * int(rng.integers(1, 33)), 32
    elif quant:
        if rng.random() < 0.5:
            H = 128 * int(rng.integers(1, 17))
            group = 128
        else:
            H = 8 * int(rng.integers(1, 257))
            group = H                                   # one scale per row
    else:
        H, group = 8 * int(rng.integers(1, 257)), 0
    sm = W.SCALE_FP32
    if quant in (W.QUANT_FP8, W.QUANT_INT8):
        sm = int(rng.choice([W.SCALE_FP32, W.SCALE_POW2, W.SCALE_UE8M0]))
    A = int(rng.choice([1, 1, 2, 3, 4, 16, 128]))
    mask = float(rng.choice([0.0, 0.0, 0.05, 0.3]))
    rpn = int(rng.choice([0, 1, 3, 8]))
    routing = "zipf" if rng.random() < 0.3 else "uniform"
    # the one-block layout, count + finish and count + scan + slots
    N = int(rng.choice([int(rng.integers(0, 1025)), int(rng.integers(1025, 4097)),
                        int(rng.integers(4097, 12001))]))
    # keep the oracle's receive buffer modest (N*K rows of H elements)
    while N * max(K, 1) * H > 24_000_000 and N > 1:
        N //= 2
    cap = 0
    non_expand = False
    sources = 1
    cq, cg = W.QUANT_NONE, 0
    extra = rng.random()
    if extra < 0.15 and A == 1:
        cap = int(rng.integers(1, max(2, 2 * N * K // E) + 1))   # some experts overflow
    elif extra < 0.35:
        non_expand = True
    elif extra < 0.5:
        sources = int(rng.choice([2, 3, 4, 16]))
        N = max(sources, N - N % sources)
    elif extra < 0.65 and pipeline != "merged":
        cq = int(rng.choice([W.QUANT_FP8, W.QUANT_INT8]))
        cg = 128 if (H % 128 == 0 and rng.random() < 0.5) else H
        if cg == H and H > 8192:
            cq, cg = W.QUANT_NONE, 0
    dup = pipeline != "merged" and K > 1 and rng.random() < 0.3
    sizes = None
    if pipeline == "merged":
        m = int(rng.integers(2, 4))
        sizes = [N] + [int(rng.integers(0, N + 1)) for _ in range(m - 1)]
        sizes = [s - s % sources for s in sizes]
    # token rounds over one handle (the separate calls only)
    rounds = int(rng.choice([1, 1, 2, 3, 4])) if pipeline == "serial" else 1
    w = W.Workload("sweep", N, H, E, R, K, expert_alignment=A, quant=quant, quant_group=group,
                   mask_prob=mask, seed=5000 + i, ranks_per_node=rpn, routing=routing,
                   expert_capacity=cap, num_sources=sources, scale_mode=sm,
                   combine_quant=cq, combine_group=cg, non_expand=non_expand, rounds=rounds)
    return w, pipeline, sizes, dup


def _with_repeats(w, rng):
    """Routing with some rows that list one expert more than once."""
    idx, wts = W.routing(w)
    if idx.shape[0] == 0:
        return idx, wts
    rows = rng.random(idx.shape[0]) < 0.2
    cols = rng.integers(1, w.num_topk, size=idx.shape[0])
    r = np.nonzero(rows)[0]
    idx[r, cols[r]] = idx[r, 0]
    return np.ascontiguousarray(idx), wts


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(NUM_CASES))
def test_random_config(i):
    w, pipeline, sizes, dup = _draw(i)
    print(f"[sweep] case {i} {pipeline} N={w.num_tokens} H={w.hidden} E={w.num_experts} "
          f"R={w.num_ranks} K={w.num_topk} A={w.expert_alignment} quant={w.quant}/"
          f"{w.quant_group}/{w.scale_mode} mask={w.mask_prob} rpn={w.ranks_per_node} "
          f"{w.routing} cap={w.expert_capacity} rounds={w.rounds} P={w.num_sources} ne={int(w.non_expand)} "
          f"cq={w.combine_quant}/{w.combine_group} dup={dup} sizes={sizes}", flush=True)
    if pipeline == "merged":
        run_overlap_sequence(w, sizes, [5000 + 10 * i + j for j in range(len(sizes))])
        return
    idx = wts = None
    if dup:
        idx, wts = _with_repeats(w, np.random.default_rng(i))
    run_and_check(w, idx=idx, wts=wts, fused=(pipeline == "fused"))


def test_draws_cover_the_paths():
    """The draws reach every pipeline, layout size class and option."""
    ws = [_draw(i) for i in range(NUM_CASES)]
    assert {p for _, p, _, _ in ws} == set(PIPELINES)
    ns = [w.num_tokens for w, _, _, _ in ws]
    assert min(ns) <= 1024 and any(1024 < n <= 4096 for n in ns) and max(ns) > 4096
    assert any(w.quant == W.QUANT_MXFP4 for w, _, _, _ in ws)
    assert any(w.quant in (W.QUANT_FP8, W.QUANT_INT8) for w, _, _, _ in ws)
    assert any(w.non_expand for w, _, _, _ in ws)
    assert any(w.num_sources > 1 for w, _, _, _ in ws)
    assert any(w.combine_quant for w, _, _, _ in ws)
    assert any(w.expert_capacity for w, _, _, _ in ws)
    assert any(d for _, _, _, d in ws)
    assert any(w.rounds > 1 for w, _, _, _ in ws)
