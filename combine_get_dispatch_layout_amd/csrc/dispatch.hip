// Dispatch on gfx950 (a3): scatter each token's hidden row to its receive
// rows, optionally quantised.
//
// What is computed ("DeepEP V1 vs V2 深度对比分析" §2.1/§2.2, expand form:
// one receive row per (token, k); quantisation modes from Aliyun "DeepEP
// 通信库使用指南（v2.1）" §1.3.1 -- group of 128 or channel = hidden -- and
// "A2_DEEPEP.md" int8 prefill option; FP8 storage type float8_e4m3fn per
// §7.4 of the first page):
//   recv[slot(t,k)] = x[t]                          (bf16, bit copy), or
//   scale = max(amax over the group, 1e-4) / Q,     Q = 448 (E4M3FN) / 127 (int8)
//   code  = round_nearest_even(x / scale)           (fp32 division)
//
// Design: one wavefront per (token, column chunk).  A chunk is VPL 16-byte
// vectors per lane, lane-contiguous, so each load and store instruction of
// the wave covers 1 KiB of one row.  The row is read once into registers and
// written to each of the token's K rows; slots are wave-uniform scalar loads.
// For 128-element groups a group is exactly 16 lanes x one vector, so the
// group max is a 4-step butterfly inside a 16-lane row; a channel scale is a
// full-wave reduction (the chunk then covers the whole row).  Padding rows
// are never written.  HBM-bound: no LDS, no MFMA.
#include "ep_internal.hpp"

// Launch shape: threads per block and whether loads/stores carry the
// non-temporal hint.  EP_DISPATCH_VPL / EP_DISPATCH_ROW_WAIT > = 0 force the
// per-shape choices made in launch_dispatch (for measurements).
#ifndef EP_DISPATCH_VPL
#define EP_DISPATCH_VPL -1
#endif
#ifndef EP_DISPATCH_BLOCK
#define EP_DISPATCH_BLOCK 256
#endif
#ifndef EP_DISPATCH_NT
#define EP_DISPATCH_NT 1
#endif
// Receive-row stores through per-row buffer resources (1) or plain global
// stores (0).
#ifndef EP_DISPATCH_BUFFER
#define EP_DISPATCH_BUFFER 1
#endif
#ifndef EP_DISPATCH_ROW_WAIT
#define EP_DISPATCH_ROW_WAIT -1
#endif

namespace epk {

namespace {

constexpr int kBlock = EP_DISPATCH_BLOCK;
constexpr int kWavesPerBlock = kBlock / kWave;

template <typename T>
__device__ __forceinline__ T load_stream(const T* p)
{
    if constexpr (EP_DISPATCH_NT) return __builtin_nontemporal_load(p);
    else return *p;
}


// Receive-row stores go through a buffer resource per row (base = the row,
// bound = the row's bytes; the third word is the gfx9 raw-buffer format):
// the row address lives in scalar registers and the lane offset in one
// vector register that never changes, so consecutive stores of a wave need
// no wait between them, and the hardware drops anything outside the row.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStoreAux = EP_DISPATCH_NT ? 2 : 0;   // nt cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(char* row, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(row, 0, bytes, kBufferWord3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int WIDTH>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int m = 1; m < WIDTH; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, WIDTH));
    return v;
}

__device__ __forceinline__ uint32_t pack_int8x4(float a, float b, float c, float d)
{
    const int ia = (int)fminf(fmaxf(rintf(a), -127.0f), 127.0f);
    const int ib = (int)fminf(fmaxf(rintf(b), -127.0f), 127.0f);
    const int ic = (int)fminf(fmaxf(rintf(c), -127.0f), 127.0f);
    const int id = (int)fminf(fmaxf(rintf(d), -127.0f), 127.0f);
    return (uint32_t)(ia & 0xFF) | ((uint32_t)(ib & 0xFF) << 8) | ((uint32_t)(ic & 0xFF) << 16) |
           ((uint32_t)(id & 0xFF) << 24);
}

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// QUANT: 0 none, 1 E4M3FN, 2 int8.  CHANNEL: one scale per row (the chunk
// covers the row), else one per 128 elements.
// ROW_WAIT: wait for each receive row's stores before writing the next row,
// which bounds the writes a wave keeps in flight (faster for long rows).
template <int QUANT, bool CHANNEL, int VPL, int KMAX, bool ROW_WAIT>
__global__ __launch_bounds__(kBlock) void k_dispatch(DispatchArgs a, int NV, int NC)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int item = blockIdx.x * kWavesPerBlock + wv;
    const int64_t t = a.t_begin + item / NC;
    const int c = item % NC;
    if (t >= a.t_end) return;
    const int K = a.K;
    const int vbase = c * (kWave * VPL) + lane;

    const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x) + t * NV;
    u32x4 d[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = vbase + kWave * i;
        d[i] = (v < NV) ? load_stream(xrow + v) : u32x4{0u, 0u, 0u, 0u};
    }
    // the token's slots as one batch of scalar loads (the slot array carries
    // kMaxTopk words of slack, so reading KMAX words is in bounds; words past
    // K are ignored)
    int sl[KMAX];
    const int32_t* srow = a.slot_idx + t * K;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) sl[k] = srow[k];

    if constexpr (QUANT == 0) {
        // Wait for the row once (s_waitcnt vmcnt(0), other counters left
        // alone): the stores below sit in separate branches, and without it
        // each would wait for every earlier store as well.
        __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            const int s = sl[k];
            if (s < 0) continue;
            if (s >= a.capacity) {
                if (lane == 0) atomicOr(a.flags, kFlagCapacity);
                continue;
            }
            char* row = reinterpret_cast<char*>(a.recv) + (int64_t)s * NV * 16;
            if constexpr (EP_DISPATCH_BUFFER) {
                const __amdgpu_buffer_rsrc_t r = row_rsrc(row, NV * 16);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int v = vbase + kWave * i;
                    if (v < NV) __builtin_amdgcn_raw_buffer_store_b128(d[i], r, v * 16, 0, kStoreAux);
                }
                if constexpr (ROW_WAIT) __builtin_amdgcn_s_waitcnt(0x0F70);
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int v = vbase + kWave * i;
                    u32x4* p = reinterpret_cast<u32x4*>(row) + v;
                    if (v < NV) {
                        if constexpr (EP_DISPATCH_NT) __builtin_nontemporal_store(d[i], p);
                        else *p = d[i];
                    }
                }
            }
        }
    } else {
        constexpr float kQ = (QUANT == 1) ? 448.0f : 127.0f;
        float amax[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                m = fmaxf(m, fmaxf(fabsf(bf16_lo(d[i][j])), fabsf(bf16_hi(d[i][j]))));
            amax[i] = m;
        }
        float scale[VPL];
        if constexpr (CHANNEL) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) m = fmaxf(m, amax[i]);
            m = group_max<kWave>(m);
            const float sc = fmaxf(m, 1e-4f) / kQ;
#pragma unroll
            for (int i = 0; i < VPL; ++i) scale[i] = sc;
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i) scale[i] = fmaxf(group_max<16>(amax[i]), 1e-4f) / kQ;
        }
        u32x2 code[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            float q[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                q[2 * j] = bf16_lo(d[i][j]) / scale[i];
                q[2 * j + 1] = bf16_hi(d[i][j]) / scale[i];
            }
            if constexpr (QUANT == 1) {
                code[i] = u32x2{pack_fp8x4(q[0], q[1], q[2], q[3]), pack_fp8x4(q[4], q[5], q[6], q[7])};
            } else {
                code[i] = u32x2{pack_int8x4(q[0], q[1], q[2], q[3]), pack_int8x4(q[4], q[5], q[6], q[7])};
            }
        }
        const int G = CHANNEL ? 1 : NV / 16;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            const int s = sl[k];
            if (s < 0) continue;
            if (s >= a.capacity) {
                if (lane == 0) atomicOr(a.flags, kFlagCapacity);
                continue;
            }
            const __amdgpu_buffer_rsrc_t r =
                row_rsrc(reinterpret_cast<char*>(a.recv) + (int64_t)s * NV * 8, NV * 8);
            float* srow = a.scales + (int64_t)s * G;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = vbase + kWave * i;
                if (v < NV) {
                    __builtin_amdgcn_raw_buffer_store_b64(code[i], r, v * 8, 0, kStoreAux);
                    if constexpr (CHANNEL) {
                        if (v == 0) srow[0] = scale[i];
                    } else {
                        if ((lane & 15) == 0) srow[v / 16] = scale[i];
                    }
                }
            }
            if constexpr (ROW_WAIT) __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    }
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

// Row-wait choice: rows of 8 KiB or more are written one row at a time per
// wave; shorter rows keep all K rows' stores in flight (measured on MI355X:
// 14 KiB rows 187 us vs 205 us, 4 KiB rows 27.3 us vs 29.2 us).
inline bool row_wait_for(int row_bytes)
{
    return EP_DISPATCH_ROW_WAIT >= 0 ? EP_DISPATCH_ROW_WAIT != 0 : row_bytes >= 8192;
}

template <int QUANT, bool CHANNEL, int VPL>
hipError_t launch_w(const DispatchArgs& a, int NV, int row_bytes, hipStream_t s, LaunchEvents ev)
{
    return row_wait_for(row_bytes) ? launch_v<QUANT, CHANNEL, VPL, true>(a, NV, s, ev)
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

// Plain scatter: long rows (>= 8 KiB) one 1 KiB piece per wave with row
// waits; shorter rows as few waves per row as possible (up to 4 KiB per
// wave), all stores in flight.
hipError_t launch_plain(const DispatchArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    const int rb = a.H * 2;
    int vpl = EP_DISPATCH_VPL;
    if (vpl < 0) vpl = rb >= 8192 ? 1 : (NV <= 64 ? 1 : NV <= 128 ? 2 : 4);
    switch (vpl) {
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
            return channel ? launch_channel<1>(a, NV, s, ev)
                           : launch_w<1, false, 1>(a, NV, a.H, s, ev);
        default:
            return channel ? launch_channel<2>(a, NV, s, ev)
                           : launch_w<2, false, 1>(a, NV, a.H, s, ev);
    }
}

}  // namespace epk
