"""The quantised dispatch forms x / scale as one reciprocal per group plus a
fused multiply-add correction per element (Markstein's correction step):
    r = 1/s,  q0 = x*r,  q = copysign(fma(fma(-q0, s, x), r, q0), x).
This checks, in C on the CPU with the same IEEE single-precision operations
(correctly rounded fmaf, no contraction), that q equals the correctly
rounded x / s for the scales the dispatch uses: s = max(amax, 1e-4) / Q with
Q = 448 (E4M3FN) or 127 (int8), amax any positive finite bf16, x any bf16
with |x| <= amax.  Quotients below 1e-20 in magnitude may differ (the
remainder underflows); both then give a zero code of x's sign, which the
check also asserts.  Every amax is covered; x runs over a stride whose
offset moves with amax, so every x residue occurs."""
import os
import shutil
import subprocess

import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float v; memcpy(&v, &u, 4); return v; }
static uint32_t to_bits(float v) { uint32_t u; memcpy(&u, &v, 4); return u; }

int main(int argc, char** argv)
{
    const unsigned stride = (unsigned)atoi(argv[1]);
    const float qmax[2] = {448.0f, 127.0f};
    long long n = 0, differ = 0, bad = 0;
    for (int qi = 0; qi < 2; ++qi)
        for (uint32_t ab = 0; ab < 0x7F80u; ++ab) {      /* every finite bf16 amax >= 0 */
            const float amax = from_bits(ab << 16);
            volatile float q = qmax[qi];
            const float s = fmaxf(amax, 1e-4f) / q;
            const float r = 1.0f / s;
            for (uint32_t xb = ab % stride; xb <= ab; xb += stride)
                for (int neg = 0; neg < 2; ++neg) {
                    const float x = from_bits((xb << 16) | (neg ? 0x80000000u : 0u));
                    const float ref = x / s;
                    const float q0 = x * r;
                    const float rem = fmaf(-q0, s, x);
                    const float got = copysignf(fmaf(rem, r, q0), x);
                    ++n;
                    if (to_bits(got) == to_bits(ref)) continue;
                    ++differ;
                    /* allowed only far below any code's rounding boundary,
                       with the sign of x */
                    if (!(fabsf(ref) < 1e-20f && fabsf(got) < 1e-20f && signbit(got) == signbit(x)))
                        ++bad;
                }
        }
    printf("%lld %lld %lld\n", n, differ, bad);
    return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_correction_rounds_like_division(tmp_path):
    src = tmp_path / "div_check.c"
    exe = tmp_path / "div_check"
    src.write_text(C_SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), str(src), "-lm"],
                   check=True)
    r = subprocess.run([str(exe), "13"], capture_output=True, text=True, timeout=300)
    n, differ, bad = map(int, r.stdout.split())
    assert n > 150_000_000
    assert bad == 0, r.stdout
    assert r.returncode == 0
