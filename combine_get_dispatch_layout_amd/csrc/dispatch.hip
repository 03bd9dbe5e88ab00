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
// full-wave reduction (the chunk then covers the whole row).  Padding rows
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
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int item = blockIdx.x * kWavesPerBlock + wv;
    const int64_t t = a.t_begin + item / NC;
    const int c = item % NC;
    if (t >= a.t_end) return;
    const int vbase = c * (kWave * VPL) + lane;
    u32x4 d[VPL];
    load_chunk<VPL>(a, t, vbase, NV, d);
    // the token's slots as one batch of scalar loads (the slot array carries
    // kMaxTopk words of slack, so reading KMAX words is in bounds; words past
    // K are ignored)
    int sl[KMAX];
    if (a.identity) {   // row quantisation: row t to receive row t
#pragma unroll
        for (int k = 0; k < KMAX; ++k) sl[k] = k == 0 ? (int)t : -1;
    } else {
        const int32_t* srow = a.slot_idx + t * a.K;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) sl[k] = srow[k];
    }
    scatter_chunk<QUANT, CHANNEL, VPL, KMAX, ROW_WAIT>(a, vbase, NV, d, sl, lane);
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


template <int QUANT, bool CHANNEL, int VPL>
hipError_t launch_w(const DispatchArgs& a, int NV, int row_bytes, hipStream_t s, LaunchEvents ev)
{
    return dispatch_row_wait(row_bytes) ? launch_v<QUANT, CHANNEL, VPL, true>(a, NV, s, ev)
                                   : launch_v<QUANT, CHANNEL, VPL, false>(a, NV, s, ev);
}

// Channel scales need the whole row in one wave: smallest VPL with
// 64*VPL >= NV.
template <int QUANT>
hipError_t launch_channel(const DispatchArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    const int rb = a.H;   // one byte per element
    if (NV <= 64) return launch_w<QUANT, true, 1>(a, NV, rb, s, ev);
    if (NV <= 128) return launch_w<QUANT, true, 2>(a, NV, rb, s, ev);
    if (NV <= 256) return launch_w<QUANT, true, 4>(a, NV, rb, s, ev);
    if (NV <= 512) return launch_w<QUANT, true, 8>(a, NV, rb, s, ev);
    return launch_w<QUANT, true, 16>(a, NV, rb, s, ev);
}

// Per-group scales: 1, 2 or 4 vectors per lane (dispatch_quant_vpl).
template <int QUANT>
hipError_t launch_group(const DispatchArgs& a, int NV, int row_bytes, hipStream_t s, LaunchEvents ev)
{
    switch (dispatch_quant_vpl(NV)) {
        case 2: return launch_w<QUANT, false, 2>(a, NV, row_bytes, s, ev);
        case 4: return launch_w<QUANT, false, 4>(a, NV, row_bytes, s, ev);
        default: return launch_w<QUANT, false, 1>(a, NV, row_bytes, s, ev);
    }
}

// Plain scatter: long rows (>= 8 KiB) one 1 KiB piece per wave with row
// waits; shorter rows as few waves per row as possible (up to 4 KiB per
// wave), all stores in flight.
hipError_t launch_plain(const DispatchArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    const int rb = a.H * 2;
    switch (dispatch_plain_vpl(NV, rb)) {
        case 1: return launch_w<0, false, 1>(a, NV, rb, s, ev);
        case 2: return launch_w<0, false, 2>(a, NV, rb, s, ev);
        case 8: return launch_w<0, false, 8>(a, NV, rb, s, ev);
        default: return launch_w<0, false, 4>(a, NV, rb, s, ev);
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s, LaunchEvents ev)
{
    const int NV = a.H / 8;
    const bool channel = a.quant != 0 && a.group == a.H && a.H != 128;
    switch (a.quant) {
        case 0: return launch_plain(a, NV, s, ev);
        case 1:
            return channel ? launch_channel<1>(a, NV, s, ev) : launch_group<1>(a, NV, a.H, s, ev);
        case 2:
            return channel ? launch_channel<2>(a, NV, s, ev) : launch_group<2>(a, NV, a.H, s, ev);
        default:
            return launch_group<3>(a, NV, a.H / 2, s, ev);
    }
}

}  // namespace epk
