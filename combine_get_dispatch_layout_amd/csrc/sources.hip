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
#include "sources.hpp"

namespace epk {

namespace {

using namespace sources;

template <int KMAX>
__global__ __launch_bounds__(kHistBlock) void k_source_hist(SourceArgs a)
{
    extern __shared__ __align__(16) int32_t lds[];
    hist_body<KMAX>(a, blockIdx.x, blockIdx.y, lds);
}

__global__ __launch_bounds__(kScanBlock) void k_source_scan(SourceArgs a)
{
    scan_body(a, blockIdx.x);
}

template <int KMAX>
hipError_t launch_sources_k(const SourceArgs& a, hipStream_t s, LaunchEvents ev)
{
    const int chunks = hist_chunks(a);
    if (chunks > 0)
        launch_k(k_source_hist<KMAX>, dim3(chunks, a.P), dim3(kHistBlock), hist_lds_bytes(a), s,
                 ev.start, nullptr, a);
    launch_k(k_source_scan, dim3(scan_blocks(a)), dim3(kScanBlock), 0, s,
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
