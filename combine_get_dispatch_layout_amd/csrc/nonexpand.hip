// Non-expand dispatch support: one receive row per (token, rank holding one
// of its experts) instead of one per (token, k).
//
// What is computed ("DeepEP V1 vs V2 深度对比分析" §2.1, the V1 normal
// dispatch returning recv_x, recv_topk_idx and recv_topk_weights; §3.1
// EPHandle.do_expand): rank r's rows are [psum_rank[r], psum_rank[r+1]) in
// source-token order; the row of (t, r) belongs to the token's first entry
// k on r, later entries on r get slot -1.  That is exactly the expand layout
// (alignment 1) of a derived routing whose entry k is the rank of expert
// idx[t,k], with repeats of a rank inside a row masked, over R "experts"
// (one per rank).  So the layout kernels run a second time, on that derived
// routing, which they compute from the expert routing as they load it
// (LayoutArgs::derive_src); dispatch and combine run unchanged: a -1 slot is
// skipped, so each (t, r) row is written once and summed once.
//
//   k_recv_topk  one thread per (t,k) owning a row: the row's local expert
//                ids (idx - r*nle where the expert is on r, else -1) and
//                weights (0 where not on r)
#include "ep_internal.hpp"

namespace epk {

namespace {

constexpr int kBlock = 256;

template <int KMAX>
__global__ __launch_bounds__(kBlock) void k_recv_topk(RecvTopkArgs a)
{
    const int64_t i = a.t_begin * a.K + (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= a.t_end * a.K) return;
    const int K = a.K;
    const int64_t t = i / K;
    const int s = a.slot_idx[i];
    if (s < 0) return;
    if (s >= a.capacity) {
        atomicOr(a.flags, kFlagCapacity);
        return;
    }
    const int r = a.topk[i] / a.nle;   // the clone: valid wherever a slot exists
    const int32_t* row = a.topk + t * K;
    for (int q = 0; q < K; ++q) {
        const int e = row[q];
        const bool on = e >= 0 && e / a.nle == r;
        if (a.recv_topk_idx) a.recv_topk_idx[(int64_t)s * K + q] = on ? e - r * a.nle : -1;
        if (a.recv_topk_weights)
            a.recv_topk_weights[(int64_t)s * K + q] = on ? a.weights[t * K + q] : 0.0f;
    }
}

}  // namespace

hipError_t launch_recv_topk(const RecvTopkArgs& a, hipStream_t s, LaunchEvents ev)
{
    if (a.t_end <= a.t_begin) return hipSuccess;
    const int64_t n = (a.t_end - a.t_begin) * a.K;
    const int blocks = (int)((n + kBlock - 1) / kBlock);
    launch_k(k_recv_topk<kMaxTopk>, dim3(blocks), dim3(kBlock), 0, s, ev.start, ev.stop, a);
    return hipGetLastError();
}

}  // namespace epk
