// Per-source receive counts for a batch of P stacked source ranks.
//
// What is computed ("DeepEP V1 vs V2 深度对比分析" §3.1, the EPHandle field
// psum_num_recv_tokens_per_scaleup_rank; §3.2 lists it among the cached
// arrays).  Source p owns tokens [p*Ns, (p+1)*Ns), Ns = N/P, so the
// (source, token, k) receive order is the (t,k) order the layout kernels
// already give; two arrays are added:
//   psum_source_rank[r][p]   tokens rank r receives from the sources before
//                            p, a token counted once per rank ([R][P+1])
//   expert_source_base[p][e] pairs of expert e from the sources before p:
//                            source p's rows of e start at psum_expert[e] +
//                            this ([P][E])
//
// Two launches, both integer and order-independent (deterministic):
//   k_source_hist  grid (chunks of 256 tokens) x P: LDS histogram of the
//                  chunk's experts and distinct ranks, added with integer
//                  atomics into per-source accumulators [P][E] and [P][R]
//                  (kept at zero between calls);
//   k_source_scan  one thread per expert or rank column: exclusive prefix
//                  over sources, loads batched 8 deep; the accumulators are
//                  re-zeroed behind the reads.
#include "ep_internal.hpp"

namespace epk {

namespace {

constexpr int kHistBlock = 256;
constexpr int kScanBlock = 256;
constexpr int kScanBatch = 8;

template <int KMAX>
__global__ __launch_bounds__(kHistBlock) void k_source_hist(SourceArgs a)
{
    extern __shared__ __align__(16) int32_t lds[];
    int32_t* hist = lds;          // [E]
    int32_t* rc = lds + a.E;      // [R]
    const int tid = threadIdx.x;
    const int p = blockIdx.y;
    for (int i = tid; i < a.E + a.R; i += kHistBlock) lds[i] = 0;
    const int64_t tl = (int64_t)blockIdx.x * kHistBlock + tid;
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

__global__ __launch_bounds__(kScanBlock) void k_source_scan(SourceArgs a)
{
    const int col = blockIdx.x * kScanBlock + threadIdx.x;
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

template <int KMAX>
hipError_t launch_sources_k(const SourceArgs& a, hipStream_t s, LaunchEvents ev)
{
    const int chunks = (int)((a.tokens_per_source + kHistBlock - 1) / kHistBlock);
    const size_t lds = (size_t)(a.E + a.R) * 4;
    if (chunks > 0)
        launch_k(k_source_hist<KMAX>, dim3(chunks, a.P), dim3(kHistBlock), lds, s, ev.start,
                 nullptr, a);
    const int cols = a.E + a.R;
    launch_k(k_source_scan, dim3((cols + kScanBlock - 1) / kScanBlock), dim3(kScanBlock), 0, s,
             chunks > 0 ? nullptr : ev.start, ev.stop, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sources(const SourceArgs& a, hipStream_t s, LaunchEvents ev)
{
    if (a.K <= 2) return launch_sources_k<2>(a, s, ev);
    if (a.K <= 4) return launch_sources_k<4>(a, s, ev);
    if (a.K <= 8) return launch_sources_k<8>(a, s, ev);
    return launch_sources_k<16>(a, s, ev);
}

}  // namespace epk
