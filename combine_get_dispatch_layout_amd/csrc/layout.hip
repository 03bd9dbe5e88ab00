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
// Three launches, all integer work and all order-independent, so the result
// is deterministic:
//   k_count  one token per lane, 256 tokens per block.  Per wave, an LDS
//            table holds, for each expert, the 64-bit mask of lanes whose
//            row contains it (ds_or_b64; one table per occurrence level, so a
//            row that repeats an expert counts each copy).  A lane's rank
//            inside the wave is the popcount of that mask below its lane
//            (mbcnt), plus earlier copies in its own row; the block adds
//            the counts of earlier waves.  Writes the block's expert
//            histogram, per-rank/per-node distinct-token counts, the
//            is_token_in_rank row, the topk clone, and the in-block rank.
//   k_scan   one 1024-thread block: column prefix of the block histograms
//            (block bases), aligned per-expert prefix, rank prefix, totals,
//            host list, and the (-1,-1) metadata of padding rows.
//   k_assign one token per lane: slot = psum_expert[e] + block base + rank.
#include "ep_internal.hpp"

namespace epk {

namespace {

// popcount(m & lanes-below-me): mbcnt over the two 32-bit halves.
__device__ __forceinline__ int count_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ void k_clear(uint32_t* w, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

template <int KMAX>
__global__ __launch_bounds__(kLayoutBlock) void k_count(LayoutArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int E = a.E, R = a.R, K = a.K;
    unsigned long long* tab = reinterpret_cast<unsigned long long*>(smem);  // [4][E]
    int32_t* wcnt = reinterpret_cast<int32_t*>(tab + 4 * E);      // [4][E]
    int32_t* rcnt = wcnt + 4 * E;                                  // [R]
    int32_t* ncnt = rcnt + R;                                      // [nodes]

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int64_t t = (int64_t)blockIdx.x * kLayoutBlock + tid;
    const bool tv = t < a.num_tokens;

    for (int i = tid; i < 4 * E; i += kLayoutBlock) wcnt[i] = 0;
    for (int i = tid; i < R; i += kLayoutBlock) rcnt[i] = 0;
    for (int i = tid; i < a.nodes; i += kLayoutBlock) ncnt[i] = 0;

    int ids[KMAX];
    bool bad = false;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int v = -1;
        if (k < K && tv) {
            v = a.topk[t * K + k];
            if (v < -1 || v >= E) {
                bad = true;
                v = -1;
            }
            a.topk_clone[t * K + k] = v;
        }
        ids[k] = v;
    }
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(a.ctrl + kCtrlFlags, kFlagBadId);

    // occ[k]: copies of ids[k] earlier in the same row.
    int occ[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < k; ++q) c += (ids[q] == ids[k]) ? 1 : 0;
        occ[k] = c;
    }

    int rank[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) rank[k] = 0;
    unsigned long long* mytab = tab + w * E;
    int32_t* mycnt = wcnt + w * E;

    for (int j = 0; j < KMAX; ++j) {
        bool have = false;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) have |= (ids[k] >= 0 && occ[k] == j);
        if (!__syncthreads_or(have)) break;
        for (int e = lane; e < E; e += kWave) mytab[e] = 0ull;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (ids[k] >= 0 && occ[k] == j) atomicOr(mytab + ids[k], 1ull << lane);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (ids[k] >= 0) rank[k] += count_below(mytab[ids[k]]);
        for (int e = lane; e < E; e += kWave) mycnt[e] += __popcll(mytab[e]);
        __syncthreads();
    }

    // Block histogram; wcnt[w][e] becomes the count of earlier waves.
    for (int e = tid; e < E; e += kLayoutBlock) {
        const int c0 = wcnt[e], c1 = wcnt[E + e], c2 = wcnt[2 * E + e], c3 = wcnt[3 * E + e];
        wcnt[e] = 0;
        wcnt[E + e] = c0;
        wcnt[2 * E + e] = c0 + c1;
        wcnt[3 * E + e] = c0 + c1 + c2;
        a.hist[(int64_t)blockIdx.x * E + e] = c0 + c1 + c2 + c3;
    }

    // Ranks: count each token once per rank and once per node.
    int rk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) rk[k] = ids[k] >= 0 ? ids[k] / a.nle : -1;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (rk[k] < 0) continue;
        bool first = true;
#pragma unroll
        for (int q = 0; q < k; ++q) first &= (rk[q] != rk[k]);
        if (first) atomicAdd(rcnt + rk[k], 1);
    }
    if (a.nodes > 0) {
        int nd[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) nd[k] = rk[k] >= 0 ? rk[k] / a.ranks_per_node : -1;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (nd[k] < 0) continue;
            bool first = true;
#pragma unroll
            for (int q = 0; q < k; ++q) first &= (nd[q] != nd[k]);
            if (first) atomicAdd(ncnt + nd[k], 1);
        }
    }
    if (a.out_in_rank != nullptr && tv) {
        uint8_t* row = a.out_in_rank + t * R;
        if (a.in_rank_words) {
            uint32_t* roww = reinterpret_cast<uint32_t*>(row);
            for (int q = 0; q < R / 4; ++q) {
                uint32_t word = 0u;
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
                    if (rk[k] >= 0 && (rk[k] >> 2) == q) word |= 1u << ((rk[k] & 3) * 8);
                roww[q] = word;
            }
        } else {
            for (int r = 0; r < R; ++r) {
                uint8_t b = 0;
#pragma unroll
                for (int k = 0; k < KMAX; ++k) b |= (rk[k] == r) ? 1 : 0;
                row[r] = b;
            }
        }
    }
    __syncthreads();

    if (tv) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K)
                a.slot_idx[t * K + k] =
                    ids[k] >= 0 ? rank[k] + occ[k] + wcnt[w * E + ids[k]] : -1;
    }
    for (int r = tid; r < R; r += kLayoutBlock) a.rank_hist[(int64_t)blockIdx.x * R + r] = rcnt[r];
    for (int n = tid; n < a.nodes; n += kLayoutBlock)
        a.node_hist[(int64_t)blockIdx.x * a.nodes + n] = ncnt[n];
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void k_scan(LayoutArgs a, int C)
{
    __shared__ int32_t part[kScanThreads];
    __shared__ int32_t buf[2][kScanThreads];
    const int E = a.E, tid = threadIdx.x;

    // 1. Column prefix of the block histograms: P threads per expert.
    int P = kScanThreads / E;
    if (P > C) P = C;
    if (P < 1) P = 1;
    const int e = tid % E, p = tid / E;
    const bool act = tid < P * E && C > 0;
    const int c0 = act ? (int)((int64_t)p * C / P) : 0;
    const int c1 = act ? (int)((int64_t)(p + 1) * C / P) : 0;
    int sum = 0;
    for (int c = c0; c < c1; ++c) sum += a.hist[(int64_t)c * E + e];
    if (act) part[p * E + e] = sum;
    __syncthreads();
    int total = 0;
    if (act) {
        int run = 0;
        for (int q = 0; q < P; ++q) {
            const int v = part[q * E + e];
            if (q < p) run += v;
            total += v;
        }
        for (int c = c0; c < c1; ++c) {
            const int v = a.hist[(int64_t)c * E + e];
            a.hist[(int64_t)c * E + e] = run;
            run += v;
        }
    }
    // 2. Aligned counts and their inclusive prefix over experts.
    int cnt = 0, aligned = 0;
    if (tid < E) {
        cnt = (C > 0) ? total : 0;
        aligned = ((cnt + a.A - 1) / a.A) * a.A;
        a.num_unaligned[tid] = cnt;
        if (a.out_per_expert) a.out_per_expert[tid] = cnt;
    }
    int cur = 0;
    buf[cur][tid] = (tid < E) ? aligned : 0;
    __syncthreads();
    for (int off = 1; off < E; off <<= 1) {
        const int v = buf[cur][tid] + ((tid >= off) ? buf[cur][tid - off] : 0);
        buf[cur ^ 1][tid] = v;
        cur ^= 1;
        __syncthreads();
    }
    const int32_t* incl = buf[cur];
    if (tid < E) {
        a.psum_expert[tid + 1] = incl[tid];
        const int first = (tid / a.nle) * a.nle;
        const int excl_first = first > 0 ? incl[first - 1] : 0;
        a.recv_list[tid] = a.counts_as_prefix ? incl[tid] - excl_first : aligned;
    }
    if (tid == 0) {
        a.psum_expert[0] = 0;
        a.ctrl[kCtrlNumSlots] = (uint32_t)incl[E - 1];
    }
    for (int r = tid; r <= a.R; r += kScanThreads)
        a.psum_rank[r] = (r * a.nle > 0) ? incl[r * a.nle - 1] : 0;

    // 3. Distinct-token totals per rank and per node.
    for (int r = tid; r < a.R; r += kScanThreads) {
        int s = 0;
        for (int c = 0; c < C; ++c) s += a.rank_hist[(int64_t)c * a.R + r];
        if (a.out_per_rank) a.out_per_rank[r] = s;
    }
    for (int n = tid; n < a.nodes; n += kScanThreads) {
        int s = 0;
        for (int c = 0; c < C; ++c) s += a.node_hist[(int64_t)c * a.nodes + n];
        if (a.out_per_node) a.out_per_node[n] = s;
    }

    // 4. Padding rows at the end of each expert segment.
    if (tid < E) {
        const int beg = incl[tid] - aligned + cnt;
        for (int row = beg; row < incl[tid]; ++row) {
            int2 m;
            m.x = -1;
            m.y = -1;
            reinterpret_cast<int2*>(a.src_meta)[row] = m;
        }
    }
}

template <int KMAX>
__global__ __launch_bounds__(kLayoutBlock) void k_assign(LayoutArgs a)
{
    const int64_t t = (int64_t)blockIdx.x * kLayoutBlock + threadIdx.x;
    if (t >= a.num_tokens) return;
    const int K = a.K, E = a.E;
    const int32_t* base = a.hist + (int64_t)blockIdx.x * E;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k >= K) break;
        const int id = a.topk_clone[t * K + k];
        if (id < 0) continue;
        const int s = a.psum_expert[id] + base[id] + a.slot_idx[t * K + k];
        a.slot_idx[t * K + k] = s;
        int2 m;
        m.x = (int)t;
        m.y = k;
        reinterpret_cast<int2*>(a.src_meta)[s] = m;
    }
}

template <int KMAX>
hipError_t launch_layout_k(const LayoutArgs& a, hipStream_t s)
{
    const int C = (int)((a.num_tokens + kLayoutBlock - 1) / kLayoutBlock);
    if (C > 0) {
        const size_t lds = (size_t)4 * a.E * 8 + (size_t)4 * a.E * 4 + (size_t)a.R * 4 +
                           (size_t)a.nodes * 4;
        hipLaunchKernelGGL(k_count<KMAX>, dim3(C), dim3(kLayoutBlock), lds, s, a);
    }
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, a, C);
    if (C > 0) hipLaunchKernelGGL(k_assign<KMAX>, dim3(C), dim3(kLayoutBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_clear(uint32_t* words, int n, hipStream_t s)
{
    hipLaunchKernelGGL(k_clear, dim3(1), dim3(64), 0, s, words, n);
    return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s)
{
    if (a.K <= 2) return launch_layout_k<2>(a, s);
    if (a.K <= 4) return launch_layout_k<4>(a, s);
    if (a.K <= 8) return launch_layout_k<8>(a, s);
    return launch_layout_k<16>(a, s);
}

}  // namespace epk
