"""Pins of the oracle's number formats against independent converters and the
format definitions.

bf16: torch's float32 -> bfloat16 conversion (round to nearest even) and the
nearest-with-ties-to-even property checked exactly for fp64 inputs.
E4M3FN ('DeepEP V1 vs V2 深度对比分析' §7.4 names float8_e4m3fn): torch's
float8_e4m3fn converter for every in-range value tried, plus the OCP table of
all 256 codes.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_bf16_identity_on_all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.f32_from_bf16(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.bf16_from_f32(vals[fin]), bits[fin])


def test_bf16_from_f32_matches_torch_on_random_bit_patterns():
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    v = pats.view(np.float32)
    # keep finite values whose rounding stays finite
    v = v[np.isfinite(v) & (np.abs(v) < 3.38e38)]
    assert np.array_equal(oracle.bf16_from_f32(v), _torch_bf16_bits(v))


def test_bf16_from_f32_ties_go_to_even():
    # exact midpoints between neighbouring bf16 values
    bits = np.arange(0x0080, 0x7F00, 7, dtype=np.uint32)
    lo = (bits << 16).view(np.float32)
    mid_bits = (bits << 16) | 0x8000
    mid = mid_bits.view(np.float32)
    got = oracle.bf16_from_f32(mid)
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    assert np.array_equal(got, _torch_bf16_bits(mid))
    assert np.array_equal(oracle.bf16_from_f32(-mid), even | 0x8000)
    assert np.array_equal(oracle.bf16_from_f32(lo), bits.astype(np.uint16))


def _bf16_value(b):
    return Fraction(float(oracle.f32_from_bf16(np.array([b], np.uint16))[0]))


def test_bf16_from_f64_is_nearest_ties_even():
    rng = np.random.default_rng(11)
    d = rng.standard_normal(4000) * np.exp2(rng.integers(-120, 120, 4000))
    # add exact midpoints and near-midpoints in fp64
    base = rng.integers(0x0100, 0x7E00, 500).astype(np.uint32)
    lo = (base << 16).view(np.float32).astype(np.float64)
    hi = ((base + 1) << 16).view(np.float32).astype(np.float64)
    mids = (lo + hi) / 2
    d = np.concatenate([d, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), -mids])
    got = oracle.bf16_from_f64(d)
    for v, b in zip(d, got):
        b = int(b)
        q = Fraction(float(v))
        r = _bf16_value(b)
        # neighbours in bf16 (same sign)
        for nb in (b - 1, b + 1):
            if (nb & 0x7FFF) in (0x7F80,) or nb < 0 or nb > 0xFFFF or (nb ^ b) & 0x8000:
                continue
            c = _bf16_value(nb)
            assert abs(r - q) <= abs(c - q), (v, b, nb)
            if abs(r - q) == abs(c - q):
                assert b % 2 == 0, (v, b)


def _torch_e4m3(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3fn_decode_table():
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle.f32_from_e4m3fn(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(dec[nan])) and np.all(np.isnan(ref[nan]))
    assert np.array_equal(dec[~nan], ref[~nan])
    # spot values from the OCP definition
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    assert dec[0x38] == 1.0 and dec[0xB8] == -1.0


def test_e4m3fn_encode_roundtrips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    keep = (codes & 0x7F) != 0x7F
    dec = oracle.f32_from_e4m3fn(codes[keep])
    assert np.array_equal(oracle.e4m3fn_from_f32(dec), codes[keep])


def test_e4m3fn_matches_torch_in_range():
    rng = np.random.default_rng(3)
    # every bf16 value in range, and random fp32 over the whole exponent range
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v1 = oracle.f32_from_bf16(bits)
    v2 = (rng.standard_normal(1 << 18) * np.exp2(rng.integers(-14, 9, 1 << 18))).astype(np.float32)
    v = np.concatenate([v1, v2])
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    assert np.array_equal(oracle.e4m3fn_from_f32(v), _torch_e4m3(v))


def test_e4m3fn_ties_to_even_and_saturation():
    codes = np.arange(0x00, 0x7E, dtype=np.uint8)
    a = oracle.f32_from_e4m3fn(codes).astype(np.float64)
    b = oracle.f32_from_e4m3fn(codes + 1).astype(np.float64)
    mid = ((a + b) / 2).astype(np.float32)          # exact in fp32
    got = oracle.e4m3fn_from_f32(mid)
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(got, even)
    # above the largest finite value: saturate (reading), never NaN
    big = np.array([448.0, 460.0, 464.0, 500.0, 1e6, -1e6], np.float32)
    assert list(oracle.e4m3fn_from_f32(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    # signed zero keeps its sign
    assert list(oracle.e4m3fn_from_f32(np.array([0.0, -0.0], np.float32))) == [0x00, 0x80]


# ---- OCP FP4 E2M1 and E8M0 (OCP Microscaling Formats v1.0; MXFP4 of
# 'DeepEP 通信库使用指南（v2.1）' §1.3.3) --------------------------------------

E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7, from the definition


def test_e2m1_decode_table():
    got = oracle.f32_from_e2m1(np.arange(16, dtype=np.uint8))
    assert got[:8].tolist() == E2M1_MAGNITUDES
    assert got[8:].tolist() == [-m for m in E2M1_MAGNITUDES]
    assert np.signbit(got[8])                                     # -0


def _e2m1_brute(v: float) -> int:
    """Nearest of the eight magnitudes by exact distance, ties to the even
    code, beyond 6 -> 6; sign from the sign bit."""
    a = Fraction(abs(v))
    if a > 6:
        code = 7
    else:
        code = min(range(8), key=lambda c: (abs(Fraction(E2M1_MAGNITUDES[c]) - a), c % 2))
    return code | (8 if np.signbit(v) else 0)


def test_e2m1_nearest_ties_even_and_saturation():
    mags = np.array(E2M1_MAGNITUDES)
    mids = (mags[:-1] + mags[1:]) / 2
    rng = np.random.default_rng(17)
    v = np.concatenate([mags, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                        rng.uniform(0, 9, 3000), [6.5, 7.0, 8.0, 100.0, 1e30]]).astype(np.float32)
    v = np.concatenate([v, -v])
    got = oracle.e2m1_from_f32(v)
    want = np.array([_e2m1_brute(float(a)) for a in v], np.uint8)
    assert np.array_equal(got, want)
    # every code decodes and re-encodes to itself
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.e2m1_from_f32(oracle.f32_from_e2m1(codes)), codes)


def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    got = oracle.f32_from_e8m0(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == np.float32(2.0 ** -127)
