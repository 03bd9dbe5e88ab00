// Streaming HBM probes (libep_probe.so): plain read, write and copy kernels
// whose achieved bandwidth is the ceiling a data-moving kernel can reach on
// this GPU.  See include/ep_probe.h.
#include "ep_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4 v, u32x4* p)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Each step a thread moves VPL vectors: vector i of the wave's chunk at
// (chunk * 64 * VPL) + i * 64 + lane, so every instruction of a wave covers
// 1 KiB of consecutive memory.
template <int MODE, int VPL, bool NT>
__global__ void k_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t nvec)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int64_t chunk = 64 * VPL;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const u32x4 pat = {(uint32_t)blockIdx.x, 0x9E3779B9u, (uint32_t)threadIdx.x, 0x85EBCA6Bu};
    for (int64_t c = wave * chunk; c < nvec; c += waves * chunk) {
        u32x4 v[VPL];
        if constexpr (MODE != EP_PROBE_WRITE) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) v[i] = ld<NT>(src + c + i * 64 + lane);
        }
        if constexpr (MODE == EP_PROBE_READ) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) acc ^= v[i];
        } else if constexpr (MODE == EP_PROBE_WRITE) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) st<NT>(pat, dst + c + i * 64 + lane);
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i) st<NT>(v[i], dst + c + i * 64 + lane);
        }
    }
    if constexpr (MODE == EP_PROBE_READ) {
        // keeps the loads: a store that the data decides, all but never taken
        if (acc[0] == 0x7FC00001u && acc[1] == 0x7FC00002u) dst[blockIdx.x] = acc;
    }
}

template <int MODE, bool NT>
hipError_t launch_v(int vpl, const u32x4* s, u32x4* d, int64_t nvec, int blocks, int threads,
                    hipStream_t stream)
{
    switch (vpl) {
        case 1: hipLaunchKernelGGL((k_stream<MODE, 1, NT>), dim3(blocks), dim3(threads), 0, stream, s, d, nvec); break;
        case 2: hipLaunchKernelGGL((k_stream<MODE, 2, NT>), dim3(blocks), dim3(threads), 0, stream, s, d, nvec); break;
        case 4: hipLaunchKernelGGL((k_stream<MODE, 4, NT>), dim3(blocks), dim3(threads), 0, stream, s, d, nvec); break;
        default: hipLaunchKernelGGL((k_stream<MODE, 8, NT>), dim3(blocks), dim3(threads), 0, stream, s, d, nvec); break;
    }
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_m(int vpl, bool nt, const u32x4* s, u32x4* d, int64_t nvec, int blocks,
                    int threads, hipStream_t stream)
{
    return nt ? launch_v<MODE, true>(vpl, s, d, nvec, blocks, threads, stream)
              : launch_v<MODE, false>(vpl, s, d, nvec, blocks, threads, stream);
}

// One wave per (token, chunk): KMAX unrolled entries, those past K masked.
template <int MODE, int VPL, int KMAX>
__global__ void k_rows(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                       const int32_t* __restrict__ slot, int64_t N, int K, int NV, int NC)
{
    const int lane = threadIdx.x & 63;
    const int64_t item = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t t = item / NC;
    const int c = (int)(item % NC);
    if (t >= N) return;
    const int vb = c * 64 * VPL + lane;
    int s[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        s[k] = k < K ? __builtin_amdgcn_readfirstlane(slot[t * K + k]) : -1;
    if constexpr (MODE == EP_PROBE_GATHER) {
        u32x4 v[KMAX][VPL];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int vi = vb + 64 * i;
                v[k][i] = (s[k] >= 0 && vi < NV) ? ld<true>(src + (int64_t)s[k] * NV + vi)
                                                 : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            u32x4 a = v[0][i];
#pragma unroll
            for (int k = 1; k < KMAX; ++k) a ^= v[k][i];
            const int vi = vb + 64 * i;
            if (vi < NV) st<true>(a, dst + t * NV + vi);
        }
    } else {
        u32x4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int vi = vb + 64 * i;
            v[i] = vi < NV ? ld<true>(src + t * NV + vi) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (s[k] < 0) continue;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int vi = vb + 64 * i;
                if (vi < NV) st<true>(v[i], dst + (int64_t)s[k] * NV + vi);
            }
        }
    }
}

template <int MODE, int VPL>
hipError_t launch_rows(const u32x4* s, u32x4* d, const int32_t* slot, int64_t N, int K, int NV,
                       int threads, hipStream_t stream)
{
    const int NC = (NV + 64 * VPL - 1) / (64 * VPL);
    const int64_t waves = N * NC;
    const int64_t blocks = (waves * 64 + threads - 1) / threads;
    if (K <= 8)
        hipLaunchKernelGGL((k_rows<MODE, VPL, 8>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                           s, d, slot, N, K, NV, NC);
    else
        hipLaunchKernelGGL((k_rows<MODE, VPL, 16>), dim3((unsigned)blocks), dim3(threads), 0,
                           stream, s, d, slot, N, K, NV, NC);
    return hipGetLastError();
}

}  // namespace

extern "C" int ep_probe_rows(int mode, const void* d_src, void* d_dst, const int32_t* d_slot,
                             int64_t num_tokens, int topk, int64_t row_bytes, int threads,
                             int vec_per_lane, void* stream)
{
    const int vpl = vec_per_lane;
    if ((mode != EP_PROBE_GATHER && mode != EP_PROBE_SCATTER) || num_tokens < 0 || topk < 1 ||
        topk > 16 || row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes / 16 > (1 << 30) ||
        threads < 64 || threads > 1024 || threads % 64 != 0 || !(vpl == 1 || vpl == 2 || vpl == 4) ||
        !d_src || !d_dst || !d_slot)
        return -1;
    if (num_tokens == 0) return 0;
    const int NV = (int)(row_bytes / 16);
    const u32x4* s = static_cast<const u32x4*>(d_src);
    u32x4* d = static_cast<u32x4*>(d_dst);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (mode == EP_PROBE_GATHER) {
        e = vpl == 1 ? launch_rows<EP_PROBE_GATHER, 1>(s, d, d_slot, num_tokens, topk, NV, threads, hs)
          : vpl == 2 ? launch_rows<EP_PROBE_GATHER, 2>(s, d, d_slot, num_tokens, topk, NV, threads, hs)
                     : launch_rows<EP_PROBE_GATHER, 4>(s, d, d_slot, num_tokens, topk, NV, threads, hs);
    } else {
        e = vpl == 1 ? launch_rows<EP_PROBE_SCATTER, 1>(s, d, d_slot, num_tokens, topk, NV, threads, hs)
          : vpl == 2 ? launch_rows<EP_PROBE_SCATTER, 2>(s, d, d_slot, num_tokens, topk, NV, threads, hs)
                     : launch_rows<EP_PROBE_SCATTER, 4>(s, d, d_slot, num_tokens, topk, NV, threads, hs);
    }
    return e == hipSuccess ? 0 : (int)e;
}

extern "C" int ep_probe_stream(int mode, const void* d_src, void* d_dst, int64_t bytes, int blocks,
                               int threads, int vec_per_lane, int nontemporal, void* stream)
{
    const int vpl = vec_per_lane;
    if (mode < EP_PROBE_READ || mode > EP_PROBE_COPY || bytes <= 0 || blocks <= 0 ||
        threads < 64 || threads > 1024 || threads % 64 != 0 ||
        !(vpl == 1 || vpl == 2 || vpl == 4 || vpl == 8) || !d_dst ||
        (mode != EP_PROBE_WRITE && !d_src))
        return -1;
    if (bytes % ((int64_t)16 * 64 * vpl) != 0) return -1;
    const int64_t nvec = bytes / 16;
    const u32x4* s = static_cast<const u32x4*>(d_src);
    u32x4* d = static_cast<u32x4*>(d_dst);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (mode) {
        case EP_PROBE_READ: e = launch_m<EP_PROBE_READ>(vpl, nontemporal, s, d, nvec, blocks, threads, hs); break;
        case EP_PROBE_WRITE: e = launch_m<EP_PROBE_WRITE>(vpl, nontemporal, s, d, nvec, blocks, threads, hs); break;
        default: e = launch_m<EP_PROBE_COPY>(vpl, nontemporal, s, d, nvec, blocks, threads, hs); break;
    }
    return e == hipSuccess ? 0 : (int)e;
}
