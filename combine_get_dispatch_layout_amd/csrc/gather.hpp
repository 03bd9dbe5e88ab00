// Device building blocks of the combine gather-reduce, shared by the combine
// kernel (combine.hip) and the combine launch that also runs the next
// batch's layout (overlap.hip).  See combine.hip for what is computed and its
// sources.
#pragma once

#include "ep_internal.hpp"

// Whether y loads / out stores carry the non-temporal hint.
#ifndef EP_COMBINE_NT
#define EP_COMBINE_NT 1
#endif
#ifndef EP_COMBINE_NT_STORE
#define EP_COMBINE_NT_STORE EP_COMBINE_NT
#endif

namespace epk {
namespace gather {


template <typename T>
__device__ __forceinline__ T load_stream(const T* p)
{
    if constexpr (EP_COMBINE_NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <typename T>
__device__ __forceinline__ void store_stream(T v, T* p)
{
    if constexpr (EP_COMBINE_NT_STORE) __builtin_nontemporal_store(v, p);
    else *p = v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

// Eight dequantised values of one 8-byte vector of codes.
template <int YQ>
__device__ __forceinline__ void decode8(u32x2 c, float (&v)[8])
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if constexpr (YQ == 1) {   // OCP E4M3FN, exact in fp32
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[h], true);
            v[4 * h] = lo[0];
            v[4 * h + 1] = lo[1];
            v[4 * h + 2] = hi[0];
            v[4 * h + 3] = hi[1];
        } else {                   // int8
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * h + j] = (float)((int32_t)(c[h] << (24 - 8 * j)) >> 24);
        }
    }
}

// YQ: expert outputs y as bf16 (0) or as E4M3FN (1) / int8 (2) codes with
// fp32 scales, one per row (YCH) or per 128 elements.
template <int KMAX, int VPL, int YQ, bool YCH, int WPB>
__device__ __forceinline__ void combine_wave(const CombineArgs& a, int NV, int NC, int block)
{
    constexpr int kWavesPerBlock = WPB;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int item = block * kWavesPerBlock + wv;
    const int64_t t = a.t_begin + item / NC;
    const int c = item % NC;
    if (t >= a.t_end) return;
    const int K = a.K;
    const int vbase = c * (kWave * VPL) + lane;

    // one lane-parallel load of the K slots and weights (lane k holds entry
    // k), broadcast to scalars: a single round trip for any K
    const int sv = (lane < K) ? a.slot_idx[t * K + lane] : -1;
    const float wl = (lane < K) ? (a.weights ? a.weights[t * K + lane] : 1.0f) : 0.0f;
    int slot[KMAX];
    float wk[KMAX];
    bool oob = false;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int s = __builtin_amdgcn_readlane(sv, k);
        wk[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k));
        if (s >= a.y_rows) {
            oob = true;
            s = -1;
        }
        slot[k] = s;
    }
    if (oob && lane == 0) atomicOr(a.flags, kFlagYRows);

    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    if constexpr (YQ == 0) {
        const u32x4* y = reinterpret_cast<const u32x4*>(a.y);
        u32x4 yv[KMAX][VPL];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = vbase + kWave * i;
                yv[k][i] = (slot[k] >= 0 && v < NV)
                               ? load_stream(y + (int64_t)slot[k] * NV + v)
                               : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (slot[k] < 0) continue;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wd = yv[k][i][j];
                    acc[i][2 * j] = __builtin_fmaf(wk[k], __uint_as_float(wd << 16), acc[i][2 * j]);
                    acc[i][2 * j + 1] =
                        __builtin_fmaf(wk[k], __uint_as_float(wd & 0xFFFF0000u), acc[i][2 * j + 1]);
                }
        }
    } else {
        // codes: 8 bytes per vector of 8 elements; scale of vector v is
        // y_scales[slot, v / 16] (128-element groups) or y_scales[slot, 0]
        const u32x2* y = reinterpret_cast<const u32x2*>(a.y);
        const int G = YCH ? 1 : NV / 16;
        u32x2 yv[KMAX][VPL];
        float ys[KMAX][VPL];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = vbase + kWave * i;
                const bool live = slot[k] >= 0 && v < NV;
                yv[k][i] = live ? load_stream(y + (int64_t)slot[k] * NV + v) : u32x2{0u, 0u};
                ys[k][i] = live ? a.y_scales[(int64_t)slot[k] * G + (YCH ? 0 : v / 16)] : 0.0f;
            }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (slot[k] < 0) continue;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                float dv[8];
                decode8<YQ>(yv[k][i], dv);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_fmaf(wk[k], dv[j] * ys[k][i], acc[i][j]);
            }
        }
    }

    u32x4* orow = reinterpret_cast<u32x4*>(a.out) + t * NV;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = vbase + kWave * i;
        if (v < NV) {
            u32x4 o;
            o[0] = pack_bf16x2(acc[i][0], acc[i][1]);
            o[1] = pack_bf16x2(acc[i][2], acc[i][3]);
            o[2] = pack_bf16x2(acc[i][4], acc[i][5]);
            o[3] = pack_bf16x2(acc[i][6], acc[i][7]);
            store_stream(o, orow + v);
        }
    }
}

}  // namespace gather
}  // namespace epk
