"""Pins of the oracle's routing layout and slot assignment.

Against: a hand-worked example (tests/golden), numpy library routines
(bincount, any-reductions, stable argsort), invariants that hold for every
input (counts sum to N*K minus masked entries; slots are a bijection onto the
non-padding rows; segments follow token order; the receive total stays under
the non-layered buffer bound of 'A2_DEEPEP.md'), and exhaustive enumeration
of tiny routings.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_worked_example.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def test_worked_example_layout_and_slots():
    g = _gold()
    idx = np.array(g["topk_idx"], np.int32)
    E, R, A = g["num_experts"], g["num_ranks"], g["expert_alignment"]
    lay = oracle.layout(idx, E, R, ranks_per_node=1)
    assert lay["num_tokens_per_expert"].tolist() == g["num_tokens_per_expert"]
    assert lay["num_tokens_per_rank"].tolist() == g["num_tokens_per_rank"]
    assert lay["is_token_in_rank"].tolist() == g["is_token_in_rank"]
    assert lay["num_tokens_per_rdma_rank"].tolist() == g["num_tokens_per_rdma_rank_ranks_per_node_1"]
    lay2 = oracle.layout(idx, E, R, ranks_per_node=2)
    assert lay2["num_tokens_per_rdma_rank"].tolist() == g["num_tokens_per_rdma_rank_ranks_per_node_2"]
    s = oracle.slots(idx, E, R, A)
    assert s["S"] == g["S"]
    assert s["psum_expert"].tolist() == g["psum_expert"]
    assert s["psum_rank"].tolist() == g["psum_rank"]
    assert s["num_unaligned"].tolist() == g["num_unaligned"]
    assert s["slot_idx"].tolist() == g["slot_idx"]
    assert s["src_meta"].tolist() == g["src_meta"]
    assert oracle.recv_list(s["psum_expert"], E, R, False).tolist() == g["recv_list_counts"]
    assert oracle.recv_list(s["psum_expert"], E, R, True).tolist() == g["recv_list_prefix"]


def _random_routing(rng, N, K, E, mask_p=0.1, dup_p=0.1):
    idx = rng.integers(0, E, size=(N, K)).astype(np.int32)
    # some rows with repeated experts, some masked entries
    dup = rng.random((N, K)) < dup_p
    idx[dup] = idx[:, :1].repeat(K, 1)[dup]
    idx[rng.random((N, K)) < mask_p] = -1
    return idx


def _numpy_layout(idx, E, R, rpn):
    nle = E // R
    valid = idx >= 0
    per_expert = np.bincount(idx[valid], minlength=E)
    ranks = np.where(valid, idx // nle, -1)
    in_rank = np.stack([(ranks == r).any(axis=1) for r in range(R)], axis=1)
    per_rank = in_rank.sum(axis=0)
    nodes = -(-R // rpn)
    per_node = np.array([in_rank[:, n * rpn:(n + 1) * rpn].any(axis=1).sum() for n in range(nodes)])
    return per_expert, per_rank, in_rank.astype(np.uint8), per_node


@pytest.mark.parametrize("N,K,E,R,rpn", [(1, 1, 1, 1, 1), (37, 3, 12, 4, 2), (300, 8, 64, 16, 8),
                                          (513, 6, 64, 8, 3), (1000, 2, 16, 4, 4)])
def test_layout_matches_numpy(N, K, E, R, rpn):
    rng = np.random.default_rng(N * 131 + K)
    idx = _random_routing(rng, N, K, E)
    lay = oracle.layout(idx, E, R, rpn)
    pe, pr, ir, pn = _numpy_layout(idx, E, R, rpn)
    assert np.array_equal(lay["num_tokens_per_expert"], pe)
    assert np.array_equal(lay["num_tokens_per_rank"], pr)
    assert np.array_equal(lay["is_token_in_rank"], ir)
    assert np.array_equal(lay["num_tokens_per_rdma_rank"], pn)
    # counts sum to N*K minus masked entries
    assert lay["num_tokens_per_expert"].sum() == N * K - (idx == -1).sum()


def _argsort_slots(idx, E, A):
    """Slot of each pair from numpy's stable sort of the flattened pairs by
    expert (masked pairs sort last)."""
    N, K = idx.shape
    key = np.where(idx >= 0, idx, E).ravel()
    order = np.argsort(key, kind="stable")
    cnt = np.bincount(key, minlength=E + 1)[:E]
    aligned = -(-cnt // A) * A
    psum = np.concatenate([[0], np.cumsum(aligned)])
    starts = np.concatenate([[0], np.cumsum(cnt)])
    slot = np.full(N * K, -1, np.int64)
    for e in range(E):
        pairs = order[starts[e]:starts[e] + cnt[e]]
        slot[pairs] = psum[e] + np.arange(cnt[e])
    return slot.reshape(N, K), psum


def _check_slot_invariants(idx, s, E, R, A):
    N, K = idx.shape
    psum, S = s["psum_expert"], s["S"]
    slot, meta = s["slot_idx"], s["src_meta"]
    cnt = s["num_unaligned"]
    V = int((idx >= 0).sum())
    assert S == psum[-1]
    assert np.all(psum % A == 0)
    assert 0 <= S - V <= E * (A - 1)
    assert np.all(np.diff(psum) >= cnt)
    assert s["psum_rank"].tolist() == [int(psum[r * (E // R)]) for r in range(R + 1)]
    # bijection valid pairs <-> non-padding rows, meta is the inverse map
    valid = idx >= 0
    assert np.all(slot[~valid] == -1)
    sv = slot[valid]
    assert len(np.unique(sv)) == V
    ts, ks = np.nonzero(valid)
    assert np.array_equal(meta[sv, 0], ts) and np.array_equal(meta[sv, 1], ks)
    assert (meta[:, 0] >= 0).sum() == V
    for e in range(E):
        seg = meta[psum[e]:psum[e + 1]]
        real = seg[:cnt[e]]
        assert np.all(seg[cnt[e]:] == -1)                     # padding at the end
        assert np.all(idx[real[:, 0], real[:, 1]] == e)       # rows hold expert e
        key = real[:, 0].astype(np.int64) * K + real[:, 1]
        assert np.all(np.diff(key) > 0)                       # (t, k) order


@pytest.mark.parametrize("N,K,E,R,A", [(1, 1, 1, 1, 1), (50, 4, 8, 2, 1), (200, 8, 32, 4, 4),
                                        (333, 6, 64, 8, 128), (777, 2, 16, 16, 3)])
def test_slots_match_stable_argsort(N, K, E, R, A):
    rng = np.random.default_rng(N + 7 * A)
    idx = _random_routing(rng, N, K, E)
    s = oracle.slots(idx, E, R, A)
    ref_slot, ref_psum = _argsort_slots(idx, E, A)
    assert np.array_equal(s["slot_idx"], ref_slot)
    assert np.array_equal(s["psum_expert"], ref_psum)
    _check_slot_invariants(idx, s, E, R, A)


def test_slots_exhaustive_tiny():
    """Every routing of 3 tokens x 2 choices over {-1,0,1,2,3}, E=4, R=2,
    with alignment 1 and 3."""
    E, R = 4, 2
    for A in (1, 3):
        for flat in itertools.product(range(-1, E), repeat=6):
            idx = np.array(flat, np.int32).reshape(3, 2)
            s = oracle.slots(idx, E, R, A)
            ref_slot, _ = _argsort_slots(idx, E, A)
            assert np.array_equal(s["slot_idx"], ref_slot), flat
            _check_slot_invariants(idx, s, E, R, A)


def test_layout_exhaustive_tiny():
    E, R = 4, 2
    for flat in itertools.product(range(-1, E), repeat=6):
        idx = np.array(flat, np.int32).reshape(3, 2)
        lay = oracle.layout(idx, E, R, 1)
        pe, pr, ir, pn = _numpy_layout(idx, E, R, 1)
        assert np.array_equal(lay["num_tokens_per_expert"], pe)
        assert np.array_equal(lay["num_tokens_per_rank"], pr)
        assert np.array_equal(lay["is_token_in_rank"], ir)
        # K=1-like identity: per-rank count >= largest expert count on it
        for r in range(R):
            assert lay["num_tokens_per_rank"][r] <= 3


def test_invalid_ids_rejected():
    idx = np.array([[0, 4]], np.int32)
    with pytest.raises(ValueError):
        oracle.layout(idx, 4, 2)
    with pytest.raises(ValueError):
        oracle.slots(np.array([[-2, 0]], np.int32), 4, 2)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_receive_bound_on_workloads(name):
    """S * hidden * 2B stays within bs * ep_world_size * min(nle, topk) *
    hidden * 2B, the core term of the non-layered HCCL_BUFFSIZE minimum of
    'A2_DEEPEP.md' (bs = tokens per rank, here the whole batch)."""
    w = W.WORKLOADS[name]
    idx, _ = W.routing(w)
    s = oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment)
    nle = w.num_experts // w.num_ranks
    bound = w.num_tokens * w.num_ranks * min(nle, w.num_topk)
    assert s["S"] * w.hidden * 2 <= bound * w.hidden * 2
    lay = oracle.layout(idx, w.num_experts, w.num_ranks)
    assert lay["num_tokens_per_expert"].sum() == w.num_tokens * w.num_topk - (idx == -1).sum()
    _check_slot_invariants(idx, s, w.num_experts, w.num_ranks, w.expert_alignment)


def _argsort_slots_fixed(idx, E, cap):
    """Fixed-capacity slots from numpy's stable sort: position of each pair
    among its expert's pairs; kept while the position is below cap."""
    N, K = idx.shape
    key = np.where(idx >= 0, idx, E).ravel()
    order = np.argsort(key, kind="stable")
    cnt = np.bincount(key, minlength=E + 1)[:E]
    starts = np.concatenate([[0], np.cumsum(cnt)])
    slot = np.full(N * K, -1, np.int64)
    for e in range(E):
        pairs = order[starts[e]:starts[e] + cnt[e]]
        pos = np.arange(cnt[e])
        keep = pos < cap
        slot[pairs[keep]] = e * cap + pos[keep]
    return slot.reshape(N, K), cnt


def _check_fixed(idx, s, E, R, cap):
    ref_slot, cnt = _argsort_slots_fixed(idx, E, cap)
    assert np.array_equal(s["slot_idx"], ref_slot)
    assert np.array_equal(s["num_unaligned"], cnt)
    assert s["dropped"] == int(np.maximum(cnt - cap, 0).sum())
    assert s["psum_expert"].tolist() == [e * cap for e in range(E + 1)]
    assert s["psum_rank"].tolist() == [r * (E // R) * cap for r in range(R + 1)]
    meta = s["src_meta"]
    used = ref_slot[ref_slot >= 0]
    ts, ks = np.nonzero(ref_slot >= 0)
    assert np.array_equal(meta[used, 0], ts) and np.array_equal(meta[used, 1], ks)
    assert (meta[:, 0] >= 0).sum() == used.size
    for e in range(E):
        seg = meta[e * cap:(e + 1) * cap]
        assert np.all(seg[min(cnt[e], cap):] == -1)


@pytest.mark.parametrize("N,K,E,R,cap", [(1, 1, 1, 1, 1), (64, 8, 32, 4, 64), (200, 4, 16, 4, 10),
                                          (300, 6, 64, 8, 300), (128, 8, 256, 16, 128)])
def test_slots_fixed_match_stable_argsort(N, K, E, R, cap):
    rng = np.random.default_rng(N * 3 + cap)
    idx = _random_routing(rng, N, K, E)
    _check_fixed(idx, oracle.slots_fixed(idx, E, R, cap), E, R, cap)


def test_slots_fixed_exhaustive_tiny():
    E, R = 4, 2
    for cap in (1, 2, 6):
        for flat in itertools.product(range(-1, E), repeat=6):
            idx = np.array(flat, np.int32).reshape(3, 2)
            _check_fixed(idx, oracle.slots_fixed(idx, E, R, cap), E, R, cap)


def test_slots_fixed_relates_to_packed_layout():
    """With enough capacity every pair keeps its position inside the expert,
    so fixed slot - e*cap == packed slot - psum[e] (A = 1)."""
    rng = np.random.default_rng(8)
    idx = _random_routing(rng, 500, 8, 64, dup_p=0.0)
    f = oracle.slots_fixed(idx, 64, 8, 500)
    p = oracle.slots(idx, 64, 8, 1)
    e = np.where(idx >= 0, idx, 0)
    valid = idx >= 0
    assert f["dropped"] == 0
    assert np.array_equal((f["slot_idx"] - e * 500)[valid], (p["slot_idx"] - p["psum_expert"][e])[valid])


def test_worked_example_fixed_capacity():
    """The hand-worked fixed-capacity layouts (capacity 1: three pairs
    dropped; capacity 2: none) and their host lists."""
    g = _gold()
    idx = np.array(g["topk_idx"], np.int32)
    E, R = g["num_experts"], g["num_ranks"]
    for cap_s, want in g["fixed_capacity"].items():
        cap = int(cap_s)
        s = oracle.slots_fixed(idx, E, R, cap)
        assert s["dropped"] == want["dropped"]
        assert s["psum_expert"].tolist() == want["psum_expert"]
        assert s["psum_rank"].tolist() == want["psum_rank"]
        assert s["slot_idx"].tolist() == want["slot_idx"]
        assert s["src_meta"].tolist() == want["src_meta"]
        assert s["num_unaligned"].tolist() == g["num_unaligned"]
        for prefix, key in ((False, "recv_list_counts"), (True, "recv_list_prefix")):
            got = oracle.recv_list_fixed(s["num_unaligned"], E, R, cap, prefix)
            assert got.tolist() == want[key], (cap, key)


@pytest.mark.parametrize("N,K,E,R,cap", [(1, 1, 1, 1, 1), (200, 4, 16, 4, 10), (300, 6, 64, 8, 40),
                                          (128, 8, 256, 16, 3), (64, 8, 32, 1, 64)])
def test_recv_list_fixed_counts_filled_rows(N, K, E, R, cap):
    """The fixed-capacity host list read off the layout itself: the rows of
    each expert's segment that hold a pair (src_meta t >= 0), and for the
    prefix form the filled rows of the rank's partition up to and including
    the expert."""
    rng = np.random.default_rng(N + 7 * cap)
    idx = _random_routing(rng, N, K, E)
    s = oracle.slots_fixed(idx, E, R, cap)
    filled = (s["src_meta"][:, 0] >= 0).reshape(E, cap).sum(axis=1)
    counts = oracle.recv_list_fixed(s["num_unaligned"], E, R, cap, False)
    assert np.array_equal(counts, filled)
    pref = oracle.recv_list_fixed(s["num_unaligned"], E, R, cap, True)
    nle = E // R
    for e in range(E):
        first = (e // nle) * nle
        rows = s["src_meta"][first * cap:(e + 1) * cap, 0]
        assert pref[e] == (rows >= 0).sum(), e
    # every rank's last entry is the pairs its partition holds
    for r in range(R):
        part = s["src_meta"][s["psum_rank"][r]:s["psum_rank"][r + 1], 0]
        assert pref[(r + 1) * nle - 1] == (part >= 0).sum()


def test_recv_list_fixed_with_room_is_packed_list():
    """With room for every pair the fixed-capacity list equals the packed
    layout's list at alignment 1 (both forms)."""
    rng = np.random.default_rng(9)
    idx = _random_routing(rng, 300, 8, 64)
    f = oracle.slots_fixed(idx, 64, 8, 300 * 8)
    p = oracle.slots(idx, 64, 8, 1)
    for prefix in (False, True):
        assert np.array_equal(oracle.recv_list_fixed(f["num_unaligned"], 64, 8, 300 * 8, prefix),
                              oracle.recv_list(p["psum_expert"], 64, 8, prefix))


# ---- several source ranks stacked in one batch ----------------------------

def test_worked_example_multi_source():
    g = _gold()
    idx = np.array(g["topk_idx"], np.int32)
    E, R = g["num_experts"], g["num_ranks"]
    for P, want in g["multi_source"].items():
        got = oracle.source_counts(idx, E, R, int(P))
        assert got["psum_source_rank"].tolist() == want["psum_source_rank"]
        assert got["expert_source_base"].tolist() == want["expert_source_base"]


def _numpy_source_counts(idx, E, R, P):
    """Library-routine form: np.add.at over (source, expert) and a reshape of
    the token x rank membership into (source, token, rank)."""
    N, K = idx.shape
    Ns = N // P
    src = np.repeat(np.arange(N) // Ns, K)
    flat = idx.ravel()
    ok = flat >= 0
    cnt = np.zeros((P, E), np.int64)
    np.add.at(cnt, (src[ok], flat[ok]), 1)
    base = np.vstack([np.zeros((1, E), np.int64), np.cumsum(cnt, axis=0)[:-1]])
    member = np.zeros((N, R), bool)
    rows = np.repeat(np.arange(N), K)
    member[rows[ok], flat[ok] // (E // R)] = True
    per = member.reshape(P, Ns, R).sum(axis=1)          # [P, R]
    psr = np.hstack([np.zeros((R, 1), np.int64), np.cumsum(per.T, axis=1)])
    return psr, base


@pytest.mark.parametrize("N,K,E,R,P", [(1, 1, 1, 1, 1), (40, 3, 12, 4, 4), (300, 8, 64, 16, 3),
                                       (256, 8, 256, 16, 16), (64, 2, 8, 8, 64), (90, 6, 64, 8, 1)])
def test_source_counts_match_numpy(N, K, E, R, P):
    rng = np.random.default_rng(N * 31 + P)
    idx = _random_routing(rng, N, K, E)
    got = oracle.source_counts(idx, E, R, P)
    psr, base = _numpy_source_counts(idx, E, R, P)
    assert np.array_equal(got["psum_source_rank"], psr)
    assert np.array_equal(got["expert_source_base"], base)


@pytest.mark.parametrize("A", [1, 4])
def test_source_bases_place_each_sources_rows(A):
    """With the slots of the stacked batch, the rows of expert e coming from
    source p are contiguous and start at psum_expert[e] + base[p, e]; the
    last prefix entry of each rank is num_tokens_per_rank."""
    rng = np.random.default_rng(77 + A)
    N, K, E, R, P = 240, 6, 32, 8, 6
    idx = _random_routing(rng, N, K, E)
    sc = oracle.source_counts(idx, E, R, P)
    s = oracle.slots(idx, E, R, A)
    lay = oracle.layout(idx, E, R)
    assert np.array_equal(sc["psum_source_rank"][:, -1], lay["num_tokens_per_rank"])
    Ns = N // P
    for p in range(P):
        part = idx[p * Ns:(p + 1) * Ns]
        slots = s["slot_idx"][p * Ns:(p + 1) * Ns]
        for e in range(E):
            rows = np.sort(slots[part == e])
            if rows.size == 0:
                continue
            start = s["psum_expert"][e] + sc["expert_source_base"][p, e]
            assert np.array_equal(rows, np.arange(start, start + rows.size))


def test_source_counts_degenerate_and_invalid():
    rng = np.random.default_rng(5)
    idx = _random_routing(rng, 50, 4, 16)
    one = oracle.source_counts(idx, 16, 4, 1)
    lay = oracle.layout(idx, 16, 4)
    assert np.array_equal(one["psum_source_rank"][:, 1], lay["num_tokens_per_rank"])
    assert not one["expert_source_base"].any()
    # one token per source: the per-source rank counts are is_token_in_rank
    per_tok = oracle.source_counts(idx, 16, 4, 50)
    assert np.array_equal(np.diff(per_tok["psum_source_rank"], axis=1),
                          lay["is_token_in_rank"].T.astype(np.int32))
    with pytest.raises(ValueError):
        oracle.source_counts(idx, 16, 4, 3)          # 50 tokens do not split into 3
    bad = idx.copy()
    bad[3, 1] = 16
    with pytest.raises(ValueError):
        oracle.source_counts(bad, 16, 4, 2)


# ---- non-expand layout ----------------------------------------------------

def test_worked_example_non_expand():
    g = _gold()
    idx = np.array(g["topk_idx"], np.int32)
    E, R = g["num_experts"], g["num_ranks"]
    want = g["non_expand"]
    s = oracle.slots_nonexpand(idx, E, R)
    assert s["S"] == want["S"]
    assert s["psum_rank"].tolist() == want["psum_rank"]
    assert s["slot_idx"].tolist() == want["slot_idx"]
    assert s["src_meta"].tolist() == want["src_meta"]
    ri, rw = oracle.recv_topk(idx, np.array(g["topk_weights"], np.float32), s["src_meta"], E, R)
    assert ri.tolist() == want["recv_topk_idx"]
    assert rw.tolist() == want["recv_topk_weights"]


def _numpy_nonexpand(idx, E, R):
    """Rows from the token x rank membership: a column cumsum gives each
    token's ordinal inside its rank; the first k of a row on a rank owns it."""
    N, K = idx.shape
    nle = E // R
    member = np.zeros((N, R), np.int64)
    rk = np.where(idx >= 0, idx // nle, -1)
    for k in range(K):
        ok = rk[:, k] >= 0
        member[np.nonzero(ok)[0], rk[ok, k]] = 1
    per = member.sum(axis=0)
    psum = np.concatenate([[0], np.cumsum(per)])
    ordinal = np.cumsum(member, axis=0) - member          # earlier tokens on the rank
    slot = np.full((N, K), -1, np.int64)
    for k in range(K):
        first = rk[:, k] >= 0
        for q in range(k):
            first &= rk[:, q] != rk[:, k]
        t = np.nonzero(first)[0]
        slot[t, k] = psum[rk[t, k]] + ordinal[t, rk[t, k]]
    return psum, slot


@pytest.mark.parametrize("N,K,E,R", [(1, 1, 1, 1), (60, 4, 16, 4), (300, 8, 64, 16),
                                     (200, 8, 256, 16), (90, 6, 12, 12), (50, 3, 8, 1)])
def test_nonexpand_matches_numpy(N, K, E, R):
    rng = np.random.default_rng(N + 7 * R)
    idx = _random_routing(rng, N, K, E)
    s = oracle.slots_nonexpand(idx, E, R)
    psum, slot = _numpy_nonexpand(idx, E, R)
    assert np.array_equal(s["psum_rank"], psum)
    assert np.array_equal(s["slot_idx"], slot)
    lay = oracle.layout(idx, E, R)
    assert np.array_equal(np.diff(s["psum_rank"]), lay["num_tokens_per_rank"])
    # src_meta inverts the slots
    meta = s["src_meta"]
    assert np.array_equal(s["slot_idx"][meta[:, 0], meta[:, 1]], np.arange(s["S"]))


def test_nonexpand_is_expand_layout_of_rank_ids():
    """The non-expand rows are the expand layout (alignment 1) of the derived
    routing whose entries are rank ids, repeats of a rank in a row masked,
    with one expert per rank."""
    rng = np.random.default_rng(3)
    N, K, E, R = 400, 8, 64, 8
    idx = _random_routing(rng, N, K, E)
    rk = np.where(idx >= 0, idx // (E // R), -1).astype(np.int32)
    for k in range(K):
        for q in range(k):
            rk[:, k] = np.where((rk[:, k] >= 0) & (rk[:, q] == rk[:, k]), -1, rk[:, k])
    ex = oracle.slots(rk, R, R, 1)
    ne = oracle.slots_nonexpand(idx, E, R)
    assert ex["S"] == ne["S"]
    assert np.array_equal(ex["psum_expert"], ne["psum_rank"])
    assert np.array_equal(ex["slot_idx"], ne["slot_idx"])
    assert np.array_equal(ex["src_meta"], ne["src_meta"])


def test_recv_topk_matches_numpy():
    rng = np.random.default_rng(12)
    N, K, E, R = 150, 8, 32, 4
    idx = _random_routing(rng, N, K, E)
    w = rng.random((N, K)).astype(np.float32)
    s = oracle.slots_nonexpand(idx, E, R)
    ri, rw = oracle.recv_topk(idx, w, s["src_meta"], E, R)
    t = s["src_meta"][:, 0]
    r = idx[t, s["src_meta"][:, 1]] // (E // R)
    on = (idx[t] >= 0) & (idx[t] // (E // R) == r[:, None])
    assert np.array_equal(ri, np.where(on, idx[t] - (r * (E // R))[:, None], -1))
    assert np.array_equal(rw, np.where(on, w[t], 0))
    # every valid entry of a token appears in exactly one of its rows
    cnt = np.zeros((N, K), np.int64)
    np.add.at(cnt, t, on.astype(np.int64))
    assert np.array_equal(cnt, (idx >= 0).astype(np.int64))


def test_group_limited_generator_brute_force():
    """The group-limited router against a per-token loop: top groups by the
    sum of their best two sigmoid affinities, then the best two experts of
    each chosen group, listed by affinity; weights normalised."""
    rng = np.random.default_rng(8)
    N, E, G, TG, K = 40, 64, 8, 4, 8
    logits = rng.standard_normal((N, E))
    idx, w = W._group_limited(logits, G, TG, K)
    aff = 1 / (1 + np.exp(-logits))
    per = K // TG
    for t in range(N):
        score = [sum(sorted(aff[t, g * 8:(g + 1) * 8], reverse=True)[:per]) for g in range(G)]
        groups = sorted(range(G), key=lambda g: (-score[g], g))[:TG]
        chosen = []
        for g in groups:
            ex = sorted(range(g * 8, (g + 1) * 8), key=lambda e: (-aff[t, e], e))[:per]
            chosen += ex
        chosen = sorted(chosen, key=lambda e: -aff[t, e])
        assert sorted(idx[t].tolist()) == sorted(chosen)
        assert np.allclose(aff[t, idx[t]], sorted(aff[t, idx[t]], reverse=True))
        assert abs(w[t].sum() - 1) < 1e-12
