// Routing layout and slot assignment on gfx950 (a1 + a2).
//
// What is computed ("DeepEP V1 vs V2 深度对比分析" §2.1 layout outputs, §3.1
// EPHandle fields, §8.4 deterministic order; "A2_DEEPEP.md" HCCL_BUFFSIZE
// note for num_local_experts = num_experts / ep_world_size):
//   num_tokens_per_expert[e]  pairs (t,k) routed to e
//   is_token_in_rank[t,r]     token t has an expert on rank r (r = e / nle)
//   num_tokens_per_rank[r]    distinct tokens on rank r (per node likewise)
//   psum_expert               exclusive prefix of the per-expert counts
//                             rounded up to expert_alignment
//   slot_idx[t,k]             psum_expert[e] + rank of (t,k) among the pairs
//                             of expert e in (t,k) order
//   src_meta[slot]            (t,k); (-1,-1) on padding rows
//
// All integer work; every count is order-independent, so the result is
// deterministic.  The in-block rank of a pair comes from a per-wave LDS
// table holding, for each expert, the 64-bit mask of lanes whose row
// contains it (ds_or_b64; one table per occurrence level, so a row that
// repeats an expert counts each copy): the rank is the popcount of that mask
// below the lane (mbcnt), plus earlier copies in the lane's own row, plus the
// counts of earlier waves of the block.
//
// The kernels are latency-bound (a few hundred KiB at most), so the paths
// are shaped to keep global round trips and launches few:
//   A (N <= 1024):   k_fused, one block: everything in LDS, one launch.
//   B (C*E small):   k_count (per 256-token block: histogram, in-block
//                    ranks, rank counts) + k_finish (each block reduces the
//                    whole histogram from one batched LDS staging: totals,
//                    its own base, the aligned prefix; writes its slots;
//                    block 0 writes the per-expert arrays; padding rows are
//                    shared out across blocks).
//   C (otherwise):   k_count + k_scan (one block, histogram staged in LDS
//                    bands) + k_slots.
#include "route.hpp"

namespace epk {

namespace {

using namespace route;

constexpr int kScanThreads = 256;
constexpr int kFusedMaxTokens = 1024;
constexpr int kFinishMaxInts = 8192;     // histogram ints k_finish stages
constexpr int kBandInts = 8192;          // LDS band of k_scan

__global__ void k_clear(uint32_t* w, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

// ---- path A: one block does everything ------------------------------------

template <int KMAX, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_fused(LayoutArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    fused_body<KMAX, WAVES>(a, smem);
}

// ---- paths B and C: per-block routing ---------------------------------------

template <int KMAX>
__global__ __launch_bounds__(kLayoutBlock) void k_count(LayoutArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    count_body<KMAX>(a, blockIdx.x, smem);
}

// Path B: every block stages the whole C x E histogram (C*E <=
// kFinishMaxInts) in one batch of independent loads, reduces the columns to
// the totals and to its own base, forms the aligned prefix and finishes its
// tokens' slots.
template <int KMAX>
__global__ __launch_bounds__(kLayoutBlock) void k_finish(LayoutArgs a, int C)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NT = kLayoutBlock;
    const int E = a.E, K = a.K, tid = threadIdx.x, b = blockIdx.x;
    int32_t* tile = reinterpret_cast<int32_t*>(smem);     // [C][E]
    int32_t* tot = tile + C * E;                           // [E]
    int32_t* base = tot + E;                               // [E]
    int32_t* psum = base + E;                              // [E+1]
    int32_t* scratch = psum + E + 1;                       // [2*NT]
    __shared__ int32_t part_pre[NT], part_all[NT];

    // token data and the histogram, all loads independent
    const int64_t t = (int64_t)b * kLayoutBlock + tid;
    const bool tv = t < a.num_tokens;
    int ids[KMAX], lr[KMAX];
    load_row<KMAX>(a.topk_clone + t * K, K, a.row_vec, tv, -1, ids);
    load_row<KMAX>(a.slot_idx + t * K, K, a.row_vec, tv, 0, lr);
    // the histogram as 16-byte vectors (workspace and LDS are 16-byte
    // aligned), then the tail
    const int n = C * E, nv = n / 4;
    const int4* src = reinterpret_cast<const int4*>(a.hist);
    int4* dst = reinterpret_cast<int4*>(tile);
#pragma unroll 8
    for (int i = tid; i < nv; i += NT) dst[i] = src[i];
    for (int i = 4 * nv + tid; i < n; i += NT) tile[i] = a.hist[i];
    __syncthreads();

    const int EPT = E < NT ? E : NT;
    int P = NT / EPT;
    if (P > C) P = C;
    for (int eb = 0; eb < E; eb += EPT) {
        const int e = eb + tid % EPT, p = tid / EPT;
        const bool act = e < E && p < P;
        const int r0 = act ? p * C / P : 0;
        const int r1 = act ? (p + 1) * C / P : 0;
        int pre = 0, all = 0;
        for (int r = r0; r < r1; ++r) {
            const int v = tile[r * E + e];
            all += v;
            pre += (r < b) ? v : 0;
        }
        if (act) {
            part_pre[p * EPT + (e - eb)] = pre;
            part_all[p * EPT + (e - eb)] = all;
        }
        __syncthreads();
        if (act && p == 0) {
            int sp = 0, sa = 0;
            for (int q = 0; q < P; ++q) {
                sp += part_pre[q * EPT + (e - eb)];
                sa += part_all[q * EPT + (e - eb)];
            }
            base[e] = sp;
            tot[e] = sa;
        }
        __syncthreads();
    }
    aligned_prefix<NT>(a, tot, psum, scratch);

    int off[KMAX];
    bool dropped = false;
    int start[KMAX], pos[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        start[k] = psum[safe_id(ids[k])];
        pos[k] = base[safe_id(ids[k])] + lr[k];
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        off[k] = ids[k] >= 0 ? final_slot(a, start[k], pos[k], dropped) : 0;
    flag_dropped<KMAX>(a, dropped);
    store_slots<KMAX>(a, t, ids, off);
    write_padding<NT>(a, tot, psum, b, C);
    if (b == 0) {
        write_expert_arrays<NT>(a, tot, psum);
        flush_rank_totals<NT>(a);
    }
}

// Path C: one block; the histogram is staged in LDS bands, turned into
// per-block bases in place, then the aligned prefix and the per-expert
// arrays.
__global__ __launch_bounds__(kScanThreads) void k_scan(LayoutArgs a, int C)
{
    constexpr int NT = kScanThreads;
    __shared__ int32_t band[kBandInts];
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t psum[kMaxExperts + 1];
    __shared__ int32_t scratch[2 * NT];
    __shared__ int32_t part[NT];
    const int E = a.E, tid = threadIdx.x;
    for (int e = tid; e < E; e += NT) cnt[e] = 0;

    const int TC = kBandInts / E > 0 ? kBandInts / E : 1;
    const int EPT = E < NT ? E : NT;
    const int P = NT / EPT;
    for (int c0 = 0; c0 < C; c0 += TC) {
        const int rows = (C - c0) < TC ? (C - c0) : TC;
        const int n = rows * E;
        const int32_t* src = a.hist + (int64_t)c0 * E;
        __syncthreads();
#pragma unroll 8
        for (int i = tid; i < n; i += NT) band[i] = src[i];
        __syncthreads();
        for (int eb = 0; eb < E; eb += EPT) {
            const int e = eb + tid % EPT, p = tid / EPT;
            const bool act = e < E && p < P;
            const int r0 = act ? p * rows / P : 0;
            const int r1 = act ? (p + 1) * rows / P : 0;
            int sum = 0;
            for (int r = r0; r < r1; ++r) sum += band[r * E + e];
            if (act) part[p * EPT + (e - eb)] = sum;
            __syncthreads();
            int tot = 0;
            if (act) {
                int run = cnt[e];
                for (int q = 0; q < P; ++q) {
                    const int v = part[q * EPT + (e - eb)];
                    if (q < p) run += v;
                    tot += v;
                }
                for (int r = r0; r < r1; ++r) {
                    const int v = band[r * E + e];
                    a.hist[(int64_t)(c0 + r) * E + e] = run;
                    run += v;
                }
            }
            __syncthreads();
            if (act && p == 0) cnt[e] += tot;
        }
    }
    __syncthreads();
    aligned_prefix<NT>(a, cnt, psum, scratch);
    write_expert_arrays<NT>(a, cnt, psum);
    write_padding<NT>(a, cnt, psum, 0, 1);
    flush_rank_totals<NT>(a);
}

template <int KMAX>
__global__ __launch_bounds__(kLayoutBlock) void k_slots(LayoutArgs a)
{
    const int64_t t = (int64_t)blockIdx.x * kLayoutBlock + threadIdx.x;
    if (t >= a.num_tokens) return;
    const int K = a.K;
    const int32_t* base = a.hist + (int64_t)blockIdx.x * a.E;
    int ids[KMAX], lr[KMAX], off[KMAX];
    load_row<KMAX>(a.topk_clone + t * K, K, a.row_vec, true, -1, ids);
    load_row<KMAX>(a.slot_idx + t * K, K, a.row_vec, true, 0, lr);
    bool dropped = false;
    int start[KMAX], pos[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        start[k] = a.psum_expert[safe_id(ids[k])];
        pos[k] = base[safe_id(ids[k])] + lr[k];
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        off[k] = ids[k] >= 0 ? final_slot(a, start[k], pos[k], dropped) : 0;
    flag_dropped<KMAX>(a, dropped);
    store_slots<KMAX>(a, t, ids, off);
}

template <int KMAX>
hipError_t launch_layout_k(const LayoutArgs& a, hipStream_t s, LaunchEvents ev)
{
    const int64_t N = a.num_tokens;
    if (N <= kLayoutBlock && fused_lds_bytes(a, 4) <= kMaxLds) {
        launch_k(k_fused<KMAX, 4>, dim3(1), dim3(4 * kWave), fused_lds_bytes(a, 4), s, ev.start,
                 ev.stop, a);
        return hipGetLastError();
    }
    if (N <= kFusedMaxTokens && fused_lds_bytes(a, 16) <= kMaxLds) {
        launch_k(k_fused<KMAX, 16>, dim3(1), dim3(16 * kWave), fused_lds_bytes(a, 16), s, ev.start,
                 ev.stop, a);
        return hipGetLastError();
    }
    const int C = (int)((N + kLayoutBlock - 1) / kLayoutBlock);
    if (C == 0) {   // empty batch whose fused path did not fit: zero outputs
        launch_k(k_scan, dim3(1), dim3(kScanThreads), 0, s, ev.start, ev.stop, a, 0);
        return hipGetLastError();
    }
    launch_k(k_count<KMAX>, dim3(C), dim3(kLayoutBlock),
             route_lds_bytes(kLayoutBlock / kWave, a.E, a.R, a.nodes), s, ev.start, nullptr, a);
    if ((int64_t)C * a.E <= kFinishMaxInts) {
        const size_t fl = ((size_t)C * a.E + 3 * (size_t)a.E + 1 + 2 * kLayoutBlock) * 4;
        launch_k(k_finish<KMAX>, dim3(C), dim3(kLayoutBlock), fl, s, nullptr, ev.stop, a, C);
    } else {
        launch_k(k_scan, dim3(1), dim3(kScanThreads), 0, s, nullptr, nullptr, a, C);
        launch_k(k_slots<KMAX>, dim3(C), dim3(kLayoutBlock), 0, s, nullptr, ev.stop, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_clear(uint32_t* words, int n, hipStream_t s)
{
    hipLaunchKernelGGL(k_clear, dim3(1), dim3(64), 0, s, words, n);
    return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s, LaunchEvents ev)
{
    if (a.K <= 2) return launch_layout_k<2>(a, s, ev);
    if (a.K <= 4) return launch_layout_k<4>(a, s, ev);
    if (a.K <= 8) return launch_layout_k<8>(a, s, ev);
    return launch_layout_k<16>(a, s, ev);
}

}  // namespace epk
