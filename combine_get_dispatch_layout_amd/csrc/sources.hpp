// Device bodies of the per-source receive counts (stacked sources), shared
// by their own kernels (sources.hip) and the launches that run the next
// batch's layout beside dispatch and combine (overlap.hip).  See
// sources.hip for what is computed and its sources.
#pragma once

#include "ep_internal.hpp"

namespace epk {
namespace sources {

constexpr int kHistBlock = 256;
constexpr int kScanBlock = 256;
constexpr int kScanBatch = 8;

__host__ __device__ inline int hist_chunks(const SourceArgs& a)
{
    return (int)((a.tokens_per_source + kHistBlock - 1) / kHistBlock);
}
__host__ __device__ inline int scan_blocks(const SourceArgs& a)
{
    return (a.E + a.R + kScanBlock - 1) / kScanBlock;
}
__host__ __device__ inline size_t hist_lds_bytes(const SourceArgs& a) { return (size_t)(a.E + a.R) * 4; }

// Chunk `chunk` (256 tokens) of source p: LDS histogram of the chunk's
// experts and distinct ranks, added with integer atomics into the per-source
// accumulators.  lds: [E + R] ints.
template <int KMAX>
__device__ __forceinline__ void hist_body(const SourceArgs& a, int chunk, int p, int32_t* lds)
{
    int32_t* hist = lds;          // [E]
    int32_t* rc = lds + a.E;      // [R]
    const int tid = threadIdx.x;
    for (int i = tid; i < a.E + a.R; i += kHistBlock) lds[i] = 0;
    const int64_t tl = (int64_t)chunk * kHistBlock + tid;
    int ids[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int v = -1;
        if (k < a.K && tl < a.tokens_per_source) {
            v = a.topk[((int64_t)p * a.tokens_per_source + tl) * a.K + k];
            if (v < 0 || v >= a.E) v = -1;   // bad ids are flagged by the layout kernels
        }
        ids[k] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (ids[k] >= 0) atomicAdd(hist + ids[k], 1);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (ids[k] < 0) continue;
        const int r = ids[k] / a.nle;
        bool first = true;
#pragma unroll
        for (int q = 0; q < k; ++q) first &= (ids[q] < 0 || ids[q] / a.nle != r);
        if (first) atomicAdd(rc + r, 1);
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += kHistBlock)
        if (hist[e] != 0) atomicAdd(a.acc_expert + (int64_t)p * a.E + e, hist[e]);
    for (int r = tid; r < a.R; r += kHistBlock)
        if (rc[r] != 0) atomicAdd(a.acc_rank + (int64_t)p * a.R + r, rc[r]);
}

// Scan block b: one thread per expert or rank column, exclusive prefix over
// sources with loads batched 8 deep; the accumulators are re-zeroed behind
// the reads.
__device__ __forceinline__ void scan_body(const SourceArgs& a, int b)
{
    const int col = b * kScanBlock + threadIdx.x;
    if (col >= a.E + a.R) return;
    const bool is_expert = col < a.E;
    const int c = is_expert ? col : col - a.E;
    const int stride = is_expert ? a.E : a.R;
    int32_t* acc = is_expert ? a.acc_expert : a.acc_rank;
    const int P = a.P;
    int run = 0;
    if (!is_expert) a.psum_source_rank[(int64_t)c * (P + 1)] = 0;
    for (int p0 = 0; p0 < P; p0 += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
            v[j] = p0 + j < P ? acc[(int64_t)(p0 + j) * stride + c] : 0;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
            const int p = p0 + j;
            if (p >= P) break;
            acc[(int64_t)p * stride + c] = 0;
            if (is_expert) {
                a.expert_source_base[(int64_t)p * a.E + c] = run;
                run += v[j];
            } else {
                run += v[j];
                a.psum_source_rank[(int64_t)c * (P + 1) + p + 1] = run;
            }
        }
    }
}

}  // namespace sources
}  // namespace epk
