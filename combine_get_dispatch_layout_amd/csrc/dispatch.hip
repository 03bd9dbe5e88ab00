// Dispatch on gfx950 (a3): scatter each token's hidden row to its receive
// rows, optionally quantised.
//
// What is computed ("DeepEP V1 vs V2 深度对比分析" §2.1/§2.2, expand form:
// one receive row per (token, k); quantisation modes from Aliyun "DeepEP
// 通信库使用指南（v2.1）" §1.3.1 -- group of 128 or channel = hidden, the
// round_scale and use_ue8m0 flags -- and §1.3.3 (MXFP4, groups of 32);
// "A2_DEEPEP.md" int8 prefill option; FP8 storage type float8_e4m3fn per
// §7.4 of the first page):
//   recv[slot(t,k)] = x[t]                          (bf16, bit copy), or
//   scale = max(amax over the group, 1e-4) / Q,     Q = 448 (E4M3FN) / 127 (int8)
//           (round_scale: the next power of two up; use_ue8m0: stored as
//           its biased exponent byte)
//   code  = round_nearest_even(x / scale)           (fp32 division), or
//   MXFP4 (OCP MX v1.0): per 32 elements the E8M0 exponent
//   floor(log2 amax) - 2 and E2M1 codes of x * 2^-exponent, two per byte.
//
// Design: one wavefront per (token, column chunk).  A chunk is VPL 16-byte
// vectors per lane, lane-contiguous, so each load and store instruction of
// the wave covers 1 KiB of one row.  The row is read once into registers and
// written to each of the token's K rows; slots are wave-uniform scalar loads.
// For 128-element groups a group is exactly 16 lanes x one vector, so the
// group max is a 4-step butterfly inside a 16-lane row; a channel scale is a
// full-wave reduction (the chunk then covers the whole row).  The quotient
// x / scale takes one reciprocal per group and a fused multiply-add
// correction per element, which rounds exactly as the division would.  Padding rows
// are never written.  HBM-bound: no LDS, no MFMA.
#include "scatter.hpp"

// Threads per block.
#ifndef EP_DISPATCH_BLOCK
#define EP_DISPATCH_BLOCK 256
#endif

namespace epk {

namespace {

using namespace scatter;

constexpr int kBlock = EP_DISPATCH_BLOCK;
constexpr int kWavesPerBlock = kBlock / kWave;

template <int QUANT, bool CHANNEL, int VPL, int KMAX, bool ROW_WAIT>
__global__ __launch_bounds__(kBlock) void k_dispatch(DispatchArgs a, int NV, int NC)
{
    dispatch_wave<QUANT, CHANNEL, VPL, KMAX, ROW_WAIT, kWavesPerBlock>(a, NV, NC, blockIdx.x);
}

template <int QUANT, bool CHANNEL, int VPL, bool ROW_WAIT>
hipError_t launch_v(const DispatchArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    const int NC = (NV + kWave * VPL - 1) / (kWave * VPL);
    const int64_t items = (a.t_end - a.t_begin) * NC;
    if (items <= 0) return hipSuccess;
    const int blocks = (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
    if (a.K <= 8)
        launch_k(k_dispatch<QUANT, CHANNEL, VPL, 8, ROW_WAIT>, dim3(blocks), dim3(kBlock), 0, s,
                 ev.start, ev.stop, a, NV, NC);
    else
        launch_k(k_dispatch<QUANT, CHANNEL, VPL, kMaxTopk, ROW_WAIT>, dim3(blocks), dim3(kBlock), 0,
                 s, ev.start, ev.stop, a, NV, NC);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s, LaunchEvents ev)
{
    auto launch = [&](auto q, auto ch, auto vpl, auto rw, int NV) {
        return launch_v<decltype(q)::value, decltype(ch)::value, decltype(vpl)::value,
                        decltype(rw)::value>(a, NV, s, ev);
    };
    return dispatch_shape(a, launch);
}

}  // namespace epk
