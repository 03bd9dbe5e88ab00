"""Property-based pins of the oracle (hypothesis): random small routings,
including masked entries and experts repeated inside a row, against
brute-force definitions written here from the pages' quantities:

- the routing layout ("DeepEP V1 vs V2 深度对比分析" §2.1 get_dispatch_layout:
  pairs per expert, distinct tokens per rank and per node, is_token_in_rank);
- the receive slots (§3.1 EPHandle: aligned per-expert prefix, rows of an
  expert in (token, k) order, padding rows last; §8.4 deterministic order),
  the fixed-capacity form (§6 low-latency buffer) and the non-expand form
  (§3.1 do_expand: one row per token and rank);
- dispatch as a row copy, and the combine as the weighted sum of the
  gathered rows rounded once to bf16 ("A2_DEEPEP.md" API table), over
  token rounds ("Ant moving home").

The definitions are loops over (t, k) pairs and exact rationals; none of
them calls the oracle's own arithmetic."""
from fractions import Fraction

import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def routings(draw, max_tokens=9):
    R = draw(st.integers(1, 4))
    nle = draw(st.integers(1, 3))
    E = R * nle
    K = draw(st.integers(1, 4))
    N = draw(st.integers(0, max_tokens))
    # ids in [-1, E): -1 masks the entry; an expert may repeat in a row
    flat = draw(st.lists(st.integers(-1, E - 1), min_size=N * K, max_size=N * K))
    idx = np.array(flat, np.int32).reshape(N, K)
    return idx, E, R


def _pairs(idx):
    N, K = idx.shape
    return [(t, k, int(idx[t, k])) for t in range(N) for k in range(K) if idx[t, k] >= 0]


def _aligned(c, A):
    return -(-c // A) * A


@SETTINGS
@given(routings(), st.integers(0, 4))
def test_layout_counts_by_definition(r, rpn):
    idx, E, R = r
    N = idx.shape[0]
    nle = E // R
    rpn = min(rpn, R)
    lay = oracle.layout(idx, E, R, rpn)
    per_expert = [sum(1 for _, _, e in _pairs(idx) if e == x) for x in range(E)]
    ranks_of = [{e // nle for e in idx[t] if e >= 0} for t in range(N)]
    per_rank = [sum(1 for t in range(N) if r_ in ranks_of[t]) for r_ in range(R)]
    in_rank = [[1 if r_ in ranks_of[t] else 0 for r_ in range(R)] for t in range(N)]
    assert lay["num_tokens_per_expert"].tolist() == per_expert
    assert lay["num_tokens_per_rank"].tolist() == per_rank
    assert lay["is_token_in_rank"].reshape(N, R).tolist() == in_rank
    if rpn > 0:
        nodes = -(-R // rpn)
        per_node = [sum(1 for t in range(N) if any(r_ // rpn == n for r_ in ranks_of[t]))
                    for n in range(nodes)]
        assert lay["num_tokens_per_rdma_rank"].tolist() == per_node
    else:
        assert lay["num_tokens_per_rdma_rank"] is None


@SETTINGS
@given(routings(), st.integers(1, 4))
def test_slots_by_definition(r, A):
    idx, E, R = r
    nle = E // R
    s = oracle.slots(idx, E, R, A)
    pairs = _pairs(idx)
    cnt = [sum(1 for _, _, e in pairs if e == x) for x in range(E)]
    start = [sum(_aligned(cnt[x], A) for x in range(e)) for e in range(E + 1)]
    assert s["psum_expert"].tolist() == start
    assert s["num_unaligned"].tolist() == cnt
    assert s["psum_rank"].tolist() == [start[r_ * nle] for r_ in range(R + 1)]
    assert s["S"] == start[E]
    want_slot = np.full(idx.shape, -1, np.int64)
    meta = [(-1, -1)] * start[E]
    for e in range(E):
        mine = sorted((t, k) for t, k, x in pairs if x == e)   # (t, k) order
        for pos, (t, k) in enumerate(mine):
            want_slot[t, k] = start[e] + pos
            meta[start[e] + pos] = (t, k)
    assert s["slot_idx"].tolist() == want_slot.tolist()
    assert [tuple(m) for m in s["src_meta"].tolist()] == meta


@SETTINGS
@given(routings(), st.integers(1, 4))
def test_fixed_capacity_slots_by_definition(r, cap):
    idx, E, R = r
    s = oracle.slots_fixed(idx, E, R, cap)
    pairs = _pairs(idx)
    want_slot = np.full(idx.shape, -1, np.int64)
    meta = [(-1, -1)] * (E * cap)
    dropped = 0
    for e in range(E):
        for pos, (t, k) in enumerate(sorted((t, k) for t, k, x in pairs if x == e)):
            if pos < cap:
                want_slot[t, k] = e * cap + pos
                meta[e * cap + pos] = (t, k)
            else:
                dropped += 1
    assert s["dropped"] == dropped
    assert s["psum_expert"].tolist() == [e * cap for e in range(E + 1)]
    assert s["slot_idx"].tolist() == want_slot.tolist()
    assert [tuple(m) for m in s["src_meta"].tolist()] == meta
    cnt = [sum(1 for _, _, x in pairs if x == e) for e in range(E)]
    nle = E // R
    filled = [min(c, cap) for c in cnt]
    assert oracle.recv_list_fixed(s["num_unaligned"], E, R, cap, False).tolist() == filled
    prefix = [sum(filled[(e // nle) * nle:e + 1]) for e in range(E)]
    assert oracle.recv_list_fixed(s["num_unaligned"], E, R, cap, True).tolist() == prefix


@SETTINGS
@given(routings())
def test_nonexpand_slots_by_definition(r):
    idx, E, R = r
    N, K = idx.shape
    nle = E // R
    s = oracle.slots_nonexpand(idx, E, R)
    # one row per (token, rank), rank-major then token order; the row belongs
    # to the token's first entry on that rank
    rows = [(r_, t) for r_ in range(R) for t in range(N)
            if any(e >= 0 and e // nle == r_ for e in idx[t])]
    assert s["S"] == len(rows)
    assert s["psum_rank"].tolist() == [sum(1 for q, _ in rows if q < r_) for r_ in range(R + 1)]
    want = np.full((N, K), -1, np.int64)
    meta = []
    for row, (r_, t) in enumerate(rows):
        k = min(k for k in range(K) if idx[t, k] >= 0 and idx[t, k] // nle == r_)
        want[t, k] = row
        meta.append((t, k))
    assert s["slot_idx"].tolist() == want.tolist()
    assert [tuple(m) for m in s["src_meta"].tolist()] == meta


def _bf16_value(b):
    return Fraction(float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]))


def _nearest_bf16(q):
    """The bf16 bit pattern nearest to the rational q, ties to an even
    significand, by comparing exact candidates: the truncations of the two
    fp32 neighbours of q."""
    if q == 0:
        return 0
    f = np.float32(float(q))
    cands = set()
    for g in (f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))):
        hi = int(np.array([g], np.float32).view(np.uint32)[0]) >> 16
        for d in (-1, 0, 1):
            b = (hi + d) & 0xFFFF
            if (b & 0x7F80) != 0x7F80:   # finite
                cands.add(b)
    best = min(cands, key=lambda b: (abs(_bf16_value(b) - q), b & 1))
    return best


@SETTINGS
@given(routings(max_tokens=6), st.integers(0, 2 ** 32 - 1), st.integers(1, 3))
def test_dispatch_and_combine_by_definition(r, seed, A):
    idx, E, R = r
    N, K = idx.shape
    H = 8
    rng = np.random.default_rng(seed)
    s = oracle.slots(idx, E, R, A)
    # finite bf16 rows, and fp32 weights
    x = (rng.integers(0, 2 ** 16, (N, H)) & 0xBFFF).astype(np.uint16)
    recv, _ = oracle.dispatch(x, s["slot_idx"], max(s["S"], 1))
    for t, k, _ in _pairs(idx):
        assert recv[s["slot_idx"][t, k]].tolist() == x[t].tolist()
    y = (rng.integers(0, 2 ** 16, (max(s["S"], 1), H)) & 0xBFFF).astype(np.uint16)
    w = rng.standard_normal((N, K)).astype(np.float32)
    out = oracle.combine(y, w, s["slot_idx"])
    for t in range(N):
        for h in range(H):
            q = sum((Fraction(float(w[t, k])) * _bf16_value(y[s["slot_idx"][t, k], h])
                     for k in range(K) if idx[t, k] >= 0), Fraction(0))
            got = int(out[t, h])
            want = _nearest_bf16(q)
            # +0 and -0 are the same sum
            assert got == want or (q == 0 and got in (0, 0x8000)), (t, h, got, want)
    # token rounds give the one-shot result bit for bit
    if N:
        b = int(rng.integers(0, N + 1))
        parts = np.zeros_like(out)
        oracle.combine(y, w, s["slot_idx"], t_begin=0, t_end=b, out=parts)
        oracle.combine(y, w, s["slot_idx"], t_begin=b, t_end=N, out=parts)
        assert np.array_equal(parts, out)
