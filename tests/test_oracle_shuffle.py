"""Pins of the oracle's dispatch (plain and quantised) and combine.

Dispatch: row copies checked by numpy fancy indexing; FP8/int8 scales by
their closed form in numpy float32; codes by torch's float8_e4m3fn converter
and numpy's rint applied to the fp32 quotient; dequantisation error bounds.
Combine: the hand-worked example, exact rational sums (fractions.Fraction)
rounded to nearest-even bf16, K=1 identity, linearity, and the identity
round trip (dispatch, identity experts, combine with weights summing to 1
returns x bit for bit).  Rounds: per-range calls equal the one-shot result.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_worked_example.json")


def _bf16_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _x(N, H, seed):
    return _bf16_bits(W.activations(N, H, seed))


def _setup(N, K, E, R, A, H, seed, mask_p=0.0):
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((N, K)) < mask_p] = -1
    s = oracle.slots(idx, E, R, A)
    return idx, s, _x(N, H, seed)


def test_dispatch_copies_rows():
    idx, s, x = _setup(300, 6, 32, 4, 8, 96, 5, mask_p=0.1)
    recv, _ = oracle.dispatch(x, s["slot_idx"], s["S"])
    meta = s["src_meta"]
    real = meta[:, 0] >= 0
    assert np.array_equal(recv[real], x[meta[real, 0]])
    assert np.all(recv[~real] == 0)      # padding rows untouched


@pytest.mark.parametrize("quant,group,H", [(oracle.QUANT_FP8, 128, 512),
                                          (oracle.QUANT_INT8, 128, 384),
                                          (oracle.QUANT_INT8, 256, 256)])
def test_quantised_dispatch_pins(quant, group, H):
    idx, s, x = _setup(200, 4, 16, 4, 1, H, 9, mask_p=0.05)
    # include an all-zero group and a tiny group to exercise the floor
    x[3, :group] = 0
    x[4, :group] = oracle.bf16_from_f32(np.full(group, 1e-6, np.float32))
    recv, sc = oracle.dispatch(x, s["slot_idx"], s["S"], quant=quant, group=group)
    G = H // group
    xf = oracle.f32_from_bf16(x).reshape(-1, G, group)
    qmax = np.float32(448.0 if quant == oracle.QUANT_FP8 else 127.0)
    amax = np.maximum(np.abs(xf).max(axis=2), np.float32(1e-4)).astype(np.float32)
    scale = (amax / qmax).astype(np.float32)                   # closed form, fp32
    q = (xf / scale[:, :, None]).astype(np.float32)             # fp32 quotient
    if quant == oracle.QUANT_FP8:
        codes = torch.from_numpy(q.reshape(-1, H)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        dq = oracle.f32_from_e4m3fn(codes).reshape(-1, G, group)
    else:
        codes = np.clip(np.rint(q), -127, 127).astype(np.int8).reshape(-1, H)
        dq = codes.astype(np.float32).reshape(-1, G, group)
    meta = s["src_meta"]
    real = meta[:, 0] >= 0
    t_of = meta[real, 0]
    assert np.array_equal(sc[real].view(np.uint32), scale[t_of].view(np.uint32))
    assert np.array_equal(recv[real].view(np.uint8), codes[t_of].view(np.uint8))
    # error bound: |code*scale - x| <= half a step of the format at q, times scale
    # (fp64 here; the slack 2^-10 covers the fp32 rounding of the quotient)
    sc64 = scale[:, :, None].astype(np.float64)
    err = np.abs(dq.astype(np.float64) * sc64 - xf.astype(np.float64))
    if quant == oracle.QUANT_FP8:
        step = np.exp2(np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6))) - 3)
        assert np.all(err <= 0.5 * step * sc64 * (1 + 2.0 ** -10))
    else:
        assert np.all(err <= 0.5 * sc64 * (1 + 2.0 ** -10))
    # the group's largest magnitude maps to the top code
    top = np.abs(dq).max(axis=2)
    big = np.abs(xf).max(axis=2) > 1e-4
    assert np.all(top[big] == qmax)
    # all-zero group: zero codes, scale = 1e-4f / qmax
    assert np.all(dq[3, 0] == 0) and scale[3, 0] == np.float32(np.float32(1e-4) / qmax)


def test_int8_ties_to_even():
    # x/scale lands exactly on k + 0.5: build a group whose amax is 127 so
    # scale = 1 and x itself is the quotient
    H = 128
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 127.0
    x[0, 1:7] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5]
    xb = oracle.bf16_from_f32(x).reshape(1, H)
    slot = np.array([[0]], np.int32)
    recv, sc = oracle.dispatch(xb, slot, 1, quant=oracle.QUANT_INT8, group=H)
    assert sc[0, 0] == 1.0
    assert recv[0, :7].tolist() == [127, 0, 2, 2, 0, -2, -2]


def test_worked_example_combine():
    with open(GOLD) as f:
        g = json.load(f)
    slot = np.array(g["slot_idx"], np.int32)
    H = g["combine_hidden"]
    y = np.array([[s + 1, -(s + 1) / 2] for s in range(g["S"])], np.float32)
    out = oracle.combine(oracle.bf16_from_f32(y).reshape(-1, H),
                         np.array(g["topk_weights"], np.float32), slot)
    assert np.array_equal(oracle.f32_from_bf16(out), np.array(g["combine_out"], np.float32))


def _exact_bf16(q: Fraction) -> int:
    """Nearest bf16 (ties to even) of an exact rational, found by comparing
    exactly against the bf16 neighbours of a starting guess."""
    guess = int(_bf16_bits(torch.tensor([float(q)], dtype=torch.float32).to(torch.bfloat16))[0])
    cands = []
    for b in range(guess - 2, guess + 3):
        if 0 <= b <= 0xFFFF and (b & 0x7F80) != 0x7F80:
            cands.append(b)
    if guess & 0x7FFF == 0:          # around zero: both signs' small values
        cands += [0x0000, 0x8000, 0x0001, 0x8001]

    def val(b):
        return Fraction(float(oracle.f32_from_bf16(np.array([b], np.uint16))[0]))

    best = min(cands, key=lambda b: (abs(val(b) - q), b % 2, b & 0x8000))
    return best


def test_combine_exact_rational_sums():
    rng = np.random.default_rng(21)
    N, K, H, S = 40, 5, 16, 120
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = _x(S, H, 22)
    # heavy cancellation rows: make k=1 cancel k=0 almost exactly
    slot[:5, 0] = 3
    slot[:5, 1] = 3
    w[:5, 1] = -np.nextafter(w[:5, 0], np.float32(0))
    out = oracle.combine(y, w, slot)
    yv = oracle.f32_from_bf16(y)
    for t in range(N):
        for h in range(H):
            q = sum((Fraction(float(w[t, k])) * Fraction(float(yv[slot[t, k], h]))
                     for k in range(K) if slot[t, k] >= 0), Fraction(0))
            want = _exact_bf16(q)
            got = int(out[t, h])
            if q == 0:
                assert got in (0x0000, 0x8000)
            else:
                assert got == want, (t, h, q, got, want)


def _bf16_of(v):
    return int(_bf16_bits(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16))[0])


def test_combine_exact_beyond_fp64():
    """Sums whose terms span more than fp64's 53 bits: the exact sum, not
    its fp64 rounding, decides.  1 + 2^-8 is the midpoint between the bf16
    neighbours 1 and 1 + 2^-7; a third term of +-2^-120 puts the sum just
    above or below it (an fp64 sum would land on the midpoint and round to
    even, 1.0, in both cases)."""
    S, H = 3, 1
    y = np.array([[_bf16_of(1.0)], [_bf16_of(2.0 ** -8)], [_bf16_of(2.0 ** -120)]], np.uint16)
    slot = np.array([[0, 1, 2], [0, 1, 2], [0, 1, -1]], np.int32)
    w = np.array([[1.0, 1.0, 1.0], [1.0, 1.0, -1.0], [1.0, 1.0, 0.0]], np.float32)
    out = oracle.combine(y, w, slot)
    assert out[:, 0].tolist() == [0x3F81, 0x3F80, 0x3F80]     # up, down, tie to even
    # wide random spans against exact rationals: values down to 2^-133 and
    # weights from 2^-100 to 2^30
    rng = np.random.default_rng(23)
    N, K, H, S = 30, 6, 8, 40
    # any sign and biased exponent 0..127 (subnormals to just below 2), so
    # that no sum leaves bf16's range
    bits = (rng.integers(0, 2 ** 16, size=(S, H)) & 0xBFFF).astype(np.uint16)
    wv = (rng.standard_normal((N, K)) * 2.0 ** rng.integers(-100, 30, size=(N, K))).astype(np.float32)
    sl = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    out = oracle.combine(bits, wv, sl)
    yv = oracle.f32_from_bf16(bits)
    for t in range(N):
        for h in range(H):
            q = sum((Fraction(float(wv[t, k])) * Fraction(float(yv[sl[t, k], h]))
                     for k in range(K) if sl[t, k] >= 0), Fraction(0))
            got = int(out[t, h])
            if q == 0:
                assert got == 0x0000, (t, h)
            else:
                assert got == _exact_bf16(q), (t, h, got)


def test_quantised_combine_exact_beyond_fp64():
    """A weight times an int8 code times an fp32 scale can need 55 bits: the
    quantised combine sums the exact products.  The midpoint case as above,
    and random full-precision weights and scales against exact rationals."""
    codes = np.array([[1], [1]], np.int8)
    sc = np.array([[1.0 + 2.0 ** -8], [2.0 ** -100]], np.float32)
    slot = np.array([[0, 1], [0, -1]], np.int32)
    w = np.ones((2, 2), np.float32)
    out = oracle.combine_q(codes, sc, oracle.QUANT_INT8, 1, w, slot)
    assert out[:, 0].tolist() == [0x3F81, 0x3F80]
    rng = np.random.default_rng(24)
    S, H, N, K = 20, 4, 25, 5
    codes = rng.integers(-127, 128, size=(S, H)).astype(np.int8)
    sc = (rng.random((S, 1)) * 2.0 ** rng.integers(-60, 20, size=(S, 1))).astype(np.float32)
    wv = (rng.standard_normal((N, K)) * 2.0 ** rng.integers(-60, 20, size=(N, K))).astype(np.float32)
    sl = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    out = oracle.combine_q(codes, sc, oracle.QUANT_INT8, H, wv, sl)
    for t in range(N):
        for h in range(H):
            q = sum((Fraction(float(wv[t, k])) * int(codes[sl[t, k], h])
                     * Fraction(float(sc[sl[t, k], 0])) for k in range(K) if sl[t, k] >= 0),
                    Fraction(0))
            got = int(out[t, h])
            if q == 0:
                assert got == 0x0000, (t, h)
            else:
                assert got == _exact_bf16(q), (t, h, got)


def test_combine_identity_linearity_and_masks():
    rng = np.random.default_rng(4)
    N, K, H, S = 64, 4, 64, 200
    y = _x(S, H, 5)
    slot = rng.integers(0, S, size=(N, 1)).astype(np.int32)
    out = oracle.combine(y, np.ones((N, 1), np.float32), slot)
    assert np.array_equal(out, y[slot[:, 0]])                   # K=1, w=1
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.random((N, K)).astype(np.float32)
    o1 = oracle.f32_from_bf16(oracle.combine(y, w, slot))
    o2 = oracle.f32_from_bf16(oracle.combine(y, 2 * w, slot))
    assert np.array_equal(2 * o1, o2)                           # exact scaling
    slot[7, :] = -1
    out = oracle.combine(y, w, slot)
    assert np.all(out[7] == 0)                                  # all masked -> +0


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_round_trip_returns_x(name):
    """dispatch -> identity experts -> combine with weights summing to 1
    gives x back bit for bit (fp32 weights sum to 1 within a few ulp, far
    inside half a bf16 ulp)."""
    w = W.WORKLOADS[name]
    N = min(w.num_tokens, 512)
    H = min(w.hidden, 512)
    idx, _ = W.routing(w, num_tokens=N)
    rng = np.random.default_rng(w.seed)
    logits = rng.standard_normal(idx.shape)
    logits[idx < 0] = -np.inf
    wt = np.exp(logits - logits.max(axis=1, keepdims=True))
    wt = (wt / wt.sum(axis=1, keepdims=True)).astype(np.float32)
    wt[~np.isfinite(wt)] = 0
    s = oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment)
    x = _x(N, H, 99)
    recv, _ = oracle.dispatch(x, s["slot_idx"], s["S"])
    out = oracle.combine(recv, wt, s["slot_idx"])
    live = (idx >= 0).any(axis=1)
    assert np.array_equal(out[live], x[live])
    assert np.all(out[~live] == 0)


def test_rounds_equal_one_shot():
    w = W.WORKLOADS["long_seq_int8"].scaled(num_tokens=1000, hidden=256, quant_group=256)
    idx, wt = W.routing(w)
    s = oracle.slots(idx, w.num_experts, w.num_ranks)
    x = _x(1000, 256, 1)
    r1, s1 = oracle.dispatch(x, s["slot_idx"], s["S"], quant=w.quant, group=w.quant_group)
    r4 = np.zeros_like(r1)
    s4 = np.zeros_like(s1)
    for b, e in W.round_ranges(1000, 4):
        oracle.dispatch(x, s["slot_idx"], s["S"], quant=w.quant, group=w.quant_group,
                        t_begin=b, t_end=e, recv_x=r4, recv_scales=s4)
    assert np.array_equal(r1, r4) and np.array_equal(s1.view(np.uint32), s4.view(np.uint32))
    y = _x(s["S"], 256, 2)
    o1 = oracle.combine(y, wt, s["slot_idx"])
    o4 = np.zeros_like(o1)
    for b, e in W.round_ranges(1000, 4):
        oracle.combine(y, wt, s["slot_idx"], t_begin=b, t_end=e, out=o4)
    assert np.array_equal(o1, o4)


# ---- scale modes, MXFP4 and quantised combine inputs ----------------------

@pytest.mark.parametrize("quant,group,H", [(oracle.QUANT_FP8, 128, 512),
                                          (oracle.QUANT_INT8, 256, 256)])
@pytest.mark.parametrize("scale_mode", [oracle.SCALE_POW2, oracle.SCALE_UE8M0])
def test_power_of_two_scales(quant, group, H, scale_mode):
    """round_scale: the scale is the smallest power of two not below the fp32
    quotient amax/qmax (no code saturates); with UE8M0 it is stored as its
    biased exponent, whose float8_e8m0fnu decode by torch is the scale."""
    idx, s, x = _setup(150, 4, 16, 4, 1, H, 31, mask_p=0.05)
    x[2, :group] = 0
    recv, sc = oracle.dispatch(x, s["slot_idx"], s["S"], quant=quant, group=group,
                               scale_mode=scale_mode)
    G = H // group
    xf = oracle.f32_from_bf16(x).reshape(-1, G, group)
    qmax = np.float32(448.0 if quant == oracle.QUANT_FP8 else 127.0)
    quot = (np.maximum(np.abs(xf).max(axis=2), np.float32(1e-4)) / qmax).astype(np.float32)
    m, e = np.frexp(quot.astype(np.float64))
    scale = np.ldexp(1.0, np.where(m == 0.5, e - 1, e)).astype(np.float32)
    assert np.all(scale >= quot) and np.all(scale / 2 < quot)
    e8 = (np.log2(scale.ravel()).astype(np.int64) + 127).astype(np.uint8)
    q = (xf / scale[:, :, None]).astype(np.float32)          # exact: a power of two
    assert np.all(np.abs(q) <= qmax)
    if quant == oracle.QUANT_FP8:
        codes = torch.from_numpy(q.reshape(-1, H)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    else:
        codes = np.rint(q).astype(np.int8).reshape(-1, H)
    meta = s["src_meta"]
    real = meta[:, 0] >= 0
    t_of = meta[real, 0]
    assert np.array_equal(recv[real].view(np.uint8), codes[t_of].view(np.uint8))
    if scale_mode == oracle.SCALE_UE8M0:
        assert sc.dtype == np.uint8
        assert np.array_equal(sc[real], e8.reshape(-1, G)[t_of])
        dec = torch.from_numpy(sc[real].copy()).view(torch.float8_e8m0fnu).to(torch.float32)
        assert np.array_equal(dec.numpy(), scale[t_of])
    else:
        assert np.array_equal(sc[real].view(np.uint32), scale[t_of].view(np.uint32))


def test_mxfp4_dispatch_pins():
    """MXFP4: per 32 elements, shared exponent floor(log2 amax) - 2 (E8M0
    byte, clamped to [-127, 127], -127 for an all-zero group), codes the
    E2M1 nearest-even of x * 2^-shared, two per byte, low nibble first."""
    H = 256
    idx, s, x = _setup(120, 4, 16, 4, 1, H, 41, mask_p=0.05)
    x[5, :32] = 0
    x[6, 32:64] = oracle.bf16_from_f32(np.full(32, 2.0 ** -130, np.float32))
    x[7, 64:96] = oracle.bf16_from_f32(np.linspace(-6, 6, 32).astype(np.float32))
    recv, sc = oracle.dispatch(x, s["slot_idx"], s["S"], quant=oracle.QUANT_MXFP4)
    assert recv.shape[1] == H // 2 and sc.dtype == np.uint8 and sc.shape[1] == H // 32
    xf = oracle.f32_from_bf16(x).astype(np.float64).reshape(-1, H // 32, 32)
    amax = np.abs(xf).max(axis=2)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    sx = np.where(amax > 0, np.clip(e - 1 - 2, -127, 127), -127)
    q = np.ldexp(xf, -sx[:, :, None]).reshape(len(x), H)
    want = np.array([_e2m1_code(float(v)) for v in q.ravel()], np.uint8).reshape(len(x), H)
    packed = (want[:, 0::2] | (want[:, 1::2] << 4)).astype(np.uint8)
    meta = s["src_meta"]
    real = meta[:, 0] >= 0
    t_of = meta[real, 0]
    assert np.array_equal(sc[real], (sx + 127).astype(np.uint8)[t_of])
    assert np.array_equal(recv[real], packed[t_of])
    assert sx[5, 0] == -127 and sx[6, 1] == -127 and sx[7, 2] == 0
    # amax / 2^shared lies in [4, 8): the largest element codes to 4 or 6
    big = amax > 2.0 ** -120
    mx = np.abs(q.reshape(-1, H // 32, 32)).max(axis=2)
    assert np.all((mx[big] >= 4) & (mx[big] < 8))


def _e2m1_code(v):
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = Fraction(abs(v))
    code = 7 if a > 6 else min(range(8), key=lambda c: (abs(Fraction(mags[c]) - a), c % 2))
    return code | (8 if np.signbit(v) else 0)


@pytest.mark.parametrize("quant", [oracle.QUANT_FP8, oracle.QUANT_INT8])
def test_quantised_combine_reduces_to_bf16_combine(quant):
    """With power-of-two scales every dequantised value code * scale is a
    bf16 number, so combining the codes equals combining those bf16 rows."""
    rng = np.random.default_rng(50 + quant)
    S, H, N, K = 90, 256, 40, 4
    y = _x(S, H, 51)
    codes, sc = oracle.quantize_rows(y, quant, group=128, scale_mode=oracle.SCALE_POW2)
    dec = (oracle.f32_from_e4m3fn(codes.ravel()).reshape(S, H) if quant == oracle.QUANT_FP8
           else codes.astype(np.float32))
    deq = dec * np.repeat(sc, 128, axis=1)
    deq_bits = oracle.bf16_from_f32(deq).reshape(S, H)
    assert np.array_equal(oracle.f32_from_bf16(deq_bits), deq)          # exact in bf16
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    got = oracle.combine_q(codes, sc, quant, 128, w, slot)
    assert np.array_equal(got, oracle.combine(deq_bits, w, slot))


def test_quantised_combine_exact_rational_sums():
    rng = np.random.default_rng(61)
    S, H, N, K = 30, 256, 12, 3
    y = _x(S, H, 62)
    codes, sc = oracle.quantize_rows(y, oracle.QUANT_INT8, group=H)      # fp32 scales
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    out = oracle.combine_q(codes, sc, oracle.QUANT_INT8, H, w, slot)
    for t in range(N):
        for h in range(0, H, 7):
            q = sum((Fraction(float(w[t, k])) * int(codes[slot[t, k], h])
                     * Fraction(float(sc[slot[t, k], 0])) for k in range(K) if slot[t, k] >= 0),
                    Fraction(0))
            got = int(out[t, h])
            if q == 0:
                assert got in (0x0000, 0x8000)
            else:
                assert got == _exact_bf16(q), (t, h)


def test_nonexpand_combine_sums_rank_rows():
    """Non-expand combine: each token's rank rows summed once (unit
    weights), the sum exact before the single bf16 rounding."""
    rng = np.random.default_rng(70)
    N, K, E, R, H = 60, 8, 32, 8, 16
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int32)
    idx[rng.random((N, K)) < 0.1] = -1
    s = oracle.slots_nonexpand(idx, E, R)
    y = _x(s["S"], H, 71)
    out = oracle.combine(y, np.ones((N, K), np.float32), s["slot_idx"])
    yv = oracle.f32_from_bf16(y)
    for t in range(N):
        rows = [r for r in s["slot_idx"][t] if r >= 0]
        assert len(rows) == len({int(a) // (E // R) for a in idx[t] if a >= 0})
        for h in range(H):
            q = sum((Fraction(float(yv[r, h])) for r in rows), Fraction(0))
            got = int(out[t, h])
            assert got in (0, 0x8000) if q == 0 else got == _exact_bf16(q)


# ---- the combine in fp32 (fused multiply-add chain) ------------------------

def _nearest_f32(q: Fraction) -> np.float32:
    """Nearest fp32 of an exact rational (ties to the even significand),
    chosen by exact comparison among the fp32 neighbours of a starting
    guess; the guess float(q) -> fp32 is within one ulp of the answer."""
    g = np.float32(float(q))
    cands = [np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))]

    def key(c):
        return (abs(Fraction(float(c)) - q), int(np.array([c], np.float32).view(np.uint32)[0]) & 1)
    return min(cands, key=key)


def _fma_chain_bits(terms):
    """bf16 bits of acc = +0, acc = fma(w, v, acc) over the (w, v) terms, each
    step the exact w*v + acc rounded once to fp32; bf16 by torch's
    nearest-even conversion."""
    acc = np.float32(0.0)
    for w, v in terms:
        q = Fraction(float(w)) * Fraction(float(v)) + Fraction(float(acc))
        acc = np.float32(0.0) if q == 0 else _nearest_f32(q)
    return int(_bf16_bits(torch.tensor([acc], dtype=torch.float32).to(torch.bfloat16))[0])


def test_combine_fma_is_the_exact_fma_chain():
    rng = np.random.default_rng(23)
    N, K, H, S = 40, 6, 16, 150
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = _x(S, H, 24)
    slot[:6, 0] = 5
    slot[:6, 1] = 5
    slot[:6, 2:] = -1
    w[:6, 1] = -w[:6, 0]                               # exact cancellation to +0
    w[6:10, 1] = -np.nextafter(w[6:10, 0], np.float32(0))
    slot[6:10, 1] = slot[6:10, 0]                      # near-total cancellation
    slot[10] = -1                                      # all masked
    out = oracle.combine_fma(y, w, slot)
    yv = oracle.f32_from_bf16(y)
    for t in range(N):
        for h in range(H):
            terms = [(w[t, k], yv[slot[t, k], h]) for k in range(K) if slot[t, k] >= 0]
            assert int(out[t, h]) == _fma_chain_bits(terms), (t, h)
    assert np.all(out[10] == 0)
    # w*y - w*y: the exact sum is 0, the chain keeps the rounding error of
    # the first product, at most half an fp32 ulp of w*y
    assert np.all(oracle.combine(y, w, slot)[:6] == 0)
    resid = np.abs(oracle.f32_from_bf16(out[:6]).astype(np.float64))
    prod = np.abs(w[:6, :1].astype(np.float64) * yv[5].astype(np.float64))
    assert np.all(resid <= 2.0 ** -24 * prod * (1 + 2.0 ** -7))


def test_combine_fma_against_exact_sum():
    """The fp32 chain and the exact sum round to the same bf16 value or to
    neighbours, except where cancellation leaves the sum far below its
    terms: there the difference stays within K * 2^-24 * sum|w*y| (the fp32
    chain's error bound) plus the two bf16 roundings."""
    rng = np.random.default_rng(25)
    N, K, H, S = 512, 8, 256, 4096
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = _x(S, H, 26)
    f = oracle.f32_from_bf16(oracle.combine_fma(y, w, slot)).astype(np.float64)
    e = oracle.f32_from_bf16(oracle.combine(y, w, slot)).astype(np.float64)
    yv = oracle.f32_from_bf16(y).astype(np.float64)
    mag = np.zeros((N, H))
    for k in range(K):
        live = slot[:, k] >= 0
        mag[live] += np.abs(w[live, k, None].astype(np.float64) * yv[slot[live, k]])
    d = np.abs(f - e)
    assert np.all(d <= 2.0 ** -8 * (np.abs(f) + np.abs(e)) + K * 2.0 ** -24 * mag)
    assert (d > 2.0 ** -7 * np.abs(e)).mean() < 1e-3     # only cancellation elements
    assert (f == e).mean() > 0.99


def test_combine_fma_identities():
    rng = np.random.default_rng(27)
    N, S, H = 64, 200, 64
    y = _x(S, H, 28)
    slot = rng.integers(0, S, size=(N, 1)).astype(np.int32)
    assert np.array_equal(oracle.combine_fma(y, np.ones((N, 1), np.float32), slot), y[slot[:, 0]])
    slot = rng.integers(-1, S, size=(N, 4)).astype(np.int32)
    wt = rng.random((N, 4)).astype(np.float32)
    o1 = oracle.f32_from_bf16(oracle.combine_fma(y, wt, slot))
    o2 = oracle.f32_from_bf16(oracle.combine_fma(y, 2 * wt, slot))
    assert np.array_equal(2 * o1, o2)                   # scaling by 2 is exact in fp32


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_round_trip_returns_x_fp32(name):
    """The identity round trip holds for the fp32 chain too: with weights
    summing to 1 its error (a few fp32 ulps) stays below half a bf16 ulp."""
    w = W.WORKLOADS[name]
    N, H = min(w.num_tokens, 256), min(w.hidden, 256)
    idx, _ = W.routing(w, num_tokens=N)
    rng = np.random.default_rng(w.seed + 1)
    logits = rng.standard_normal(idx.shape)
    logits[idx < 0] = -np.inf
    wt = np.exp(logits - logits.max(axis=1, keepdims=True))
    wt = (wt / wt.sum(axis=1, keepdims=True)).astype(np.float32)
    wt[~np.isfinite(wt)] = 0
    s = oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment)
    x = _x(N, H, 98)
    recv, _ = oracle.dispatch(x, s["slot_idx"], s["S"])
    out = oracle.combine_fma(recv, wt, s["slot_idx"])
    live = (idx >= 0).any(axis=1)
    assert np.array_equal(out[live], x[live]) and np.all(out[~live] == 0)


@pytest.mark.parametrize("quant,group", [(oracle.QUANT_FP8, 128), (oracle.QUANT_INT8, 256)])
def test_combine_q_fma_is_the_exact_fma_chain(quant, group):
    """Quantised inputs: each value is the fp32 product code * scale (one
    rounding), then the fused multiply-add chain."""
    rng = np.random.default_rng(29 + quant)
    S, H, N, K = 40, 256, 10, 4
    y = _x(S, H, 30)
    codes, sc = oracle.quantize_rows(y, quant, group=group)          # fp32 scales
    slot = rng.integers(-1, S, size=(N, K)).astype(np.int32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    out = oracle.combine_q_fma(codes, sc, quant, group, w, slot)
    dec = (oracle.f32_from_e4m3fn(codes.ravel()).reshape(S, H) if quant == oracle.QUANT_FP8
           else codes.astype(np.float32))
    for t in range(N):
        for h in range(0, H, 5):
            terms = []
            for k in range(K):
                s_ = slot[t, k]
                if s_ >= 0:
                    v = _nearest_f32(Fraction(float(dec[s_, h])) * Fraction(float(sc[s_, h // group])))
                    terms.append((w[t, k], v))
            assert int(out[t, h]) == _fma_chain_bits(terms), (t, h)


# ---- the OpenMP build ---------------------------------------------------------

@pytest.mark.parametrize("quant,group,scale_mode", [(oracle.QUANT_NONE, None, 0),
                                                    (oracle.QUANT_FP8, 128, 0),
                                                    (oracle.QUANT_INT8, 256, 0),
                                                    (oracle.QUANT_FP8, 128, oracle.SCALE_UE8M0),
                                                    (oracle.QUANT_MXFP4, 32, 0)])
def test_openmp_build_matches_serial(quant, group, scale_mode):
    """The OpenMP build (per-token loops on several threads) gives the
    serial build's bits for dispatch and every combine form."""
    assert oracle.num_threads(False) == 1 and oracle.num_threads(True) >= 1
    idx, s, x = _setup(700, 6, 64, 8, 4, 256, 33, mask_p=0.05)
    r1, s1 = oracle.dispatch(x, s["slot_idx"], s["S"], quant=quant, group=group,
                             scale_mode=scale_mode)
    r2, s2 = oracle.dispatch(x, s["slot_idx"], s["S"], quant=quant, group=group,
                             scale_mode=scale_mode, parallel=True)
    assert np.array_equal(r1.view(np.uint8), r2.view(np.uint8))
    if s1 is not None:
        assert np.array_equal(s1.view(np.uint8), s2.view(np.uint8))
    rng = np.random.default_rng(34)
    wt = rng.standard_normal(idx.shape).astype(np.float32)
    y = _x(s["S"], 256, 35)
    for fp32 in (False, True):
        assert np.array_equal(oracle.combine(y, wt, s["slot_idx"], fp32=fp32),
                              oracle.combine(y, wt, s["slot_idx"], fp32=fp32, parallel=True))
        if quant in (oracle.QUANT_FP8, oracle.QUANT_INT8) and scale_mode == 0:
            yc, ys = oracle.quantize_rows(y, quant, group=group)
            assert np.array_equal(
                oracle.combine_q(yc, ys, quant, group, wt, s["slot_idx"], fp32=fp32),
                oracle.combine_q(yc, ys, quant, group, wt, s["slot_idx"], fp32=fp32, parallel=True))
