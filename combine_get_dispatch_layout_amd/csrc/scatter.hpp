// Device building blocks of the dispatch scatter (load a row chunk, quantise,
// write it to the token's receive rows), shared by the dispatch kernel
// (dispatch.hip) and the single-launch layout + dispatch (fused.hip).  See
// dispatch.hip for what is computed and its sources.
#pragma once

#include "ep_internal.hpp"

// Whether x loads and receive-row stores carry the non-temporal hint.
#ifndef EP_DISPATCH_NT
#define EP_DISPATCH_NT 1
#endif

// >= 0: force the per-shape choices below (for measurements).
#ifndef EP_DISPATCH_VPL
#define EP_DISPATCH_VPL -1
#endif
#ifndef EP_DISPATCH_ROW_WAIT
#define EP_DISPATCH_ROW_WAIT -1
#endif

namespace epk {

// Row-wait choice: rows of 8 KiB or more are written one row at a time per
// wave; shorter rows keep all K rows' stores in flight (measured on MI355X:
// 14 KiB rows 187 us vs 205 us, 4 KiB rows 27.3 us vs 29.2 us).
inline bool dispatch_row_wait(int row_bytes)
{
    return EP_DISPATCH_ROW_WAIT >= 0 ? EP_DISPATCH_ROW_WAIT != 0 : row_bytes >= 8192;
}

// Vectors per lane of the plain scatter: long rows (>= 8 KiB) one 1 KiB piece
// per wave; shorter rows as few waves per row as possible, up to 4 KiB each.
inline int dispatch_plain_vpl(int NV, int row_bytes)
{
    if (EP_DISPATCH_VPL >= 0) return EP_DISPATCH_VPL;
    return row_bytes >= 8192 ? 1 : (NV <= 64 ? 1 : NV <= 128 ? 2 : 4);
}

namespace scatter {

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

// Loads the wave's chunk of row t: VPL 16-byte vectors per lane starting at
// vector vbase (lane-contiguous), zero past the row end.
template <int VPL>
__device__ __forceinline__ void load_chunk(const DispatchArgs& a, int64_t t, int vbase, int NV,
                                           u32x4 (&d)[VPL])
{
    const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x) + t * NV;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = vbase + kWave * i;
        d[i] = (v < NV) ? load_stream(xrow + v) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Writes the chunk (loaded by load_chunk) to the token's receive rows
// sl[0..K), quantising it first when QUANT != 0.
// QUANT: 0 none, 1 E4M3FN, 2 int8.  CHANNEL: one scale per row (the chunk
// covers the row), else one per 128 elements.
// ROW_WAIT: wait for each receive row's stores before writing the next row,
// which bounds the writes a wave keeps in flight (faster for long rows).
template <int QUANT, bool CHANNEL, int VPL, int KMAX, bool ROW_WAIT>
__device__ __forceinline__ void scatter_chunk(const DispatchArgs& a, int vbase, int NV,
                                              u32x4 (&d)[VPL], const int (&sl)[KMAX], int lane)
{
    const int K = a.K;
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
            const __amdgpu_buffer_rsrc_t r =
                row_rsrc(reinterpret_cast<char*>(a.recv) + (int64_t)s * NV * 16, NV * 16);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = vbase + kWave * i;
                if (v < NV) __builtin_amdgcn_raw_buffer_store_b128(d[i], r, v * 16, 0, kStoreAux);
            }
            if constexpr (ROW_WAIT) __builtin_amdgcn_s_waitcnt(0x0F70);
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

}  // namespace scatter
}  // namespace epk
