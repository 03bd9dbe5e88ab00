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
#include "ep_internal.hpp"

namespace epk {

namespace {

constexpr int kScanThreads = 256;
constexpr int kFusedMaxTokens = 1024;
constexpr int kFinishMaxInts = 8192;     // histogram ints k_finish stages
constexpr int kBandInts = 8192;          // LDS band of k_scan
constexpr size_t kMaxLds = 65536;

// popcount(m & lanes-below-me): mbcnt over the two 32-bit halves.
__device__ __forceinline__ int count_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int div_by(int n, uint32_t magic)
{
    return magic == 0u ? n : (int)__umulhi((uint32_t)n, magic);
}

__global__ void k_clear(uint32_t* w, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

// LDS of the routing phase for a block of `waves` waves.
struct RouteLds {
    unsigned long long* tab;   // [waves][E] lane masks (free after the phase)
    int32_t* wcnt;             // [waves][E] per-wave counts -> exclusive bases
    int32_t* bhist;            // [E] block totals
    int32_t* rcnt;             // [R] distinct tokens per rank
    int32_t* ncnt;             // [nodes]
};

inline size_t route_lds_bytes(int waves, int E, int R, int nodes)
{
    return (size_t)waves * E * 8 + (size_t)waves * E * 4 + (size_t)E * 4 + (size_t)R * 4 +
           (size_t)nodes * 4;
}

__device__ inline RouteLds carve_route(unsigned char* smem, int waves, int E, int R)
{
    RouteLds L;
    L.tab = reinterpret_cast<unsigned long long*>(smem);
    L.wcnt = reinterpret_cast<int32_t*>(L.tab + waves * E);
    L.bhist = L.wcnt + waves * E;
    L.rcnt = L.bhist + E;
    L.ncnt = L.rcnt + R;
    return L;
}

// Routing phase for the block's tokens t0 .. t0 + WAVES*64 - 1 (one per
// thread).  Leaves the sanitised ids and the in-block rank of every pair in
// registers, the block histogram in L.bhist and the distinct-token counts in
// L.rcnt / L.ncnt; writes the topk clone and the is_token_in_rank rows.
template <int KMAX, int WAVES>
__device__ __forceinline__ void route_block(const LayoutArgs& a, int64_t t0, const RouteLds& L,
                                            int (&ids)[KMAX], int (&lr)[KMAX])
{
    constexpr int NT = WAVES * kWave;
    const int E = a.E, R = a.R, K = a.K;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int64_t t = t0 + tid;
    const bool tv = t < a.num_tokens;

    for (int i = tid; i < WAVES * E; i += NT) L.wcnt[i] = 0;
    for (int i = tid; i < R; i += NT) L.rcnt[i] = 0;
    for (int i = tid; i < a.nodes; i += NT) L.ncnt[i] = 0;

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
    unsigned long long* mytab = L.tab + w * E;
    int32_t* mycnt = L.wcnt + w * E;

    // Each wave owns its table and counts, so the occurrence levels need only
    // wave-level ordering: a wave's LDS operations complete in issue order,
    // and the wavefront fences keep the compiler from reordering them.
    __syncthreads();   // counters zeroed
    for (int j = 0; j < KMAX; ++j) {
        bool have = false;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) have |= (ids[k] >= 0 && occ[k] == j);
        if (__ballot(have) == 0ull) break;
        for (int e = lane; e < E; e += kWave) mytab[e] = 0ull;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (ids[k] >= 0 && occ[k] == j) atomicOr(mytab + ids[k], 1ull << lane);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (ids[k] >= 0) rank[k] += count_below(mytab[ids[k]]);
        for (int e = lane; e < E; e += kWave) mycnt[e] += __popcll(mytab[e]);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    __syncthreads();

    // Block totals; wcnt[w][e] becomes the count of earlier waves.
    for (int e = tid; e < E; e += NT) {
        int run = 0;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) {
            const int v = L.wcnt[q * E + e];
            L.wcnt[q * E + e] = run;
            run += v;
        }
        L.bhist[e] = run;
    }

    // Count each token once per rank and once per node.
    int rk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) rk[k] = ids[k] >= 0 ? div_by(ids[k], a.nle_magic) : -1;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (rk[k] < 0) continue;
        bool first = true;
#pragma unroll
        for (int q = 0; q < k; ++q) first &= (rk[q] != rk[k]);
        if (first) atomicAdd(L.rcnt + rk[k], 1);
    }
    if (a.nodes > 0) {
        int nd[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) nd[k] = rk[k] >= 0 ? div_by(rk[k], a.rpn_magic) : -1;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (nd[k] < 0) continue;
            bool first = true;
#pragma unroll
            for (int q = 0; q < k; ++q) first &= (nd[q] != nd[k]);
            if (first) atomicAdd(L.ncnt + nd[k], 1);
        }
    }
    if (a.out_in_rank != nullptr && tv) {
        uint8_t* row = a.out_in_rank + t * R;
        if (a.in_rank_words && R <= 64) {
            uint64_t m = 0ull;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (rk[k] >= 0) m |= 1ull << rk[k];
            uint32_t* roww = reinterpret_cast<uint32_t*>(row);
            for (int q = 0; q < R / 4; ++q) {
                const uint32_t nib = (uint32_t)(m >> (4 * q));
                roww[q] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
            }
        } else if (a.in_rank_words) {
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
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        lr[k] = ids[k] >= 0 ? rank[k] + occ[k] + L.wcnt[w * E + ids[k]] : -1;
}

// Exclusive prefix of the aligned counts cnt[0..E) into psum[0..E]; NT
// threads, each owning up to kMaxExperts/NT consecutive experts: a
// shuffle scan inside each wave, one barrier, then the wave offsets.
// scratch: NT/64 ints.
template <int NT>
__device__ void aligned_prefix(const LayoutArgs& a, const int32_t* cnt, int32_t* psum,
                               int32_t* scratch)
{
    constexpr int EPT = (kMaxExperts + NT - 1) / NT;
    constexpr int WAVES = NT / kWave;
    const int tid = threadIdx.x, E = a.E, lane = tid & (kWave - 1), w = tid / kWave;
    int al[EPT];
    int own = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * EPT + j;
        const int c = e < E ? cnt[e] : 0;
        al[j] = ((c + a.A - 1) / a.A) * a.A;
        own += al[j];
    }
    int incl = own;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == kWave - 1) scratch[w] = incl;
    __syncthreads();
    int run = incl - own;
    for (int q = 0; q < w; ++q) run += scratch[q];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * EPT + j;
        if (e < E) psum[e] = run;
        run += al[j];
    }
    if (tid == NT - 1) psum[E] = run;
    __syncthreads();
    (void)WAVES;
}

// Per-expert handle arrays and caller outputs from the counts and prefix
// (both in LDS).
template <int NT>
__device__ void write_expert_arrays(const LayoutArgs& a, const int32_t* cnt, const int32_t* psum)
{
    const int tid = threadIdx.x, E = a.E;
    for (int e = tid; e <= E; e += NT) a.psum_expert[e] = psum[e];
    for (int e = tid; e < E; e += NT) {
        a.num_unaligned[e] = cnt[e];
        if (a.out_per_expert) a.out_per_expert[e] = cnt[e];
        const int first = (e / a.nle) * a.nle;
        a.recv_list[e] = a.counts_as_prefix ? psum[e + 1] - psum[first] : psum[e + 1] - psum[e];
    }
    for (int r = tid; r <= a.R; r += NT) a.psum_rank[r] = psum[r * a.nle];
    if (tid == 0) a.ctrl[kCtrlNumSlots] = (uint32_t)psum[E];
}

// (-1,-1) metadata of the padding rows of experts e0, e0+step, ...  At
// most A-1 rows per expert: the (expert, row) pairs are flattened so that
// consecutive threads write consecutive rows.
template <int NT>
__device__ void write_padding(const LayoutArgs& a, const int32_t* cnt, const int32_t* psum, int e0,
                              int step)
{
    if (a.A <= 1 || e0 >= a.E) return;
    const int W = a.A - 1;
    const int ne = (a.E - e0 + step - 1) / step;
    int2 m;
    m.x = -1;
    m.y = -1;
    for (int i = threadIdx.x; i < ne * W; i += NT) {
        const int ei = i / W;
        const int e = e0 + ei * step;
        const int row = psum[e] + cnt[e] + (i - ei * W);
        if (row < psum[e + 1]) reinterpret_cast<int2*>(a.src_meta)[row] = m;
    }
}

template <int KMAX>
__device__ __forceinline__ void store_slots(const LayoutArgs& a, int64_t t, const int (&ids)[KMAX],
                                            const int (&off)[KMAX])
{
    const int K = a.K;
    if (t >= a.num_tokens) return;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k >= K) break;
        const int s = ids[k] >= 0 ? off[k] : -1;
        a.slot_idx[t * K + k] = s;
        if (s >= 0) {
            int2 m;
            m.x = (int)t;
            m.y = k;
            reinterpret_cast<int2*>(a.src_meta)[s] = m;
        }
    }
}

// ---- path A: one block does everything ------------------------------------

template <int KMAX, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void k_fused(LayoutArgs a)
{
    constexpr int NT = WAVES * kWave;
    extern __shared__ __align__(16) unsigned char smem[];
    const RouteLds L = carve_route(smem, WAVES, a.E, a.R);
    int ids[KMAX], lr[KMAX];
    route_block<KMAX, WAVES>(a, 0, L, ids, lr);
    // prefix [E+1] and scan scratch [2*NT] follow the routing LDS
    int32_t* psum = L.ncnt + a.nodes;
    int32_t* scratch = psum + a.E + 1;
    aligned_prefix<NT>(a, L.bhist, psum, scratch);
    int off[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) off[k] = ids[k] >= 0 ? psum[ids[k]] + lr[k] : 0;
    store_slots<KMAX>(a, threadIdx.x, ids, off);
    write_expert_arrays<NT>(a, L.bhist, psum);
    write_padding<NT>(a, L.bhist, psum, 0, 1);
    for (int r = threadIdx.x; r < a.R; r += NT)
        if (a.out_per_rank) a.out_per_rank[r] = L.rcnt[r];
    for (int n = threadIdx.x; n < a.nodes; n += NT)
        if (a.out_per_node) a.out_per_node[n] = L.ncnt[n];
}

// ---- paths B and C: per-block routing ---------------------------------------

// Writes the block histogram, the in-block ranks (into slot_idx, finished by
// the next kernel) and adds the distinct-token counts to the accumulators.
template <int KMAX>
__global__ __launch_bounds__(kLayoutBlock) void k_count(LayoutArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int WAVES = kLayoutBlock / kWave;
    const RouteLds L = carve_route(smem, WAVES, a.E, a.R);
    int ids[KMAX], lr[KMAX];
    const int64_t t0 = (int64_t)blockIdx.x * kLayoutBlock;
    route_block<KMAX, WAVES>(a, t0, L, ids, lr);
    const int tid = threadIdx.x, K = a.K;
    const int64_t t = t0 + tid;
    if (t < a.num_tokens) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K) a.slot_idx[t * K + k] = lr[k];
    }
    for (int e = tid; e < a.E; e += kLayoutBlock) a.hist[(int64_t)blockIdx.x * a.E + e] = L.bhist[e];
    for (int r = tid; r < a.R; r += kLayoutBlock)
        if (L.rcnt[r] != 0) atomicAdd(a.rank_acc + r, L.rcnt[r]);
    for (int n = tid; n < a.nodes; n += kLayoutBlock)
        if (L.ncnt[n] != 0) atomicAdd(a.node_acc + n, L.ncnt[n]);
}

// Distinct-token totals from the accumulators, which are re-zeroed for the
// next call.
template <int NT>
__device__ void flush_rank_totals(const LayoutArgs& a)
{
    for (int r = threadIdx.x; r < a.R; r += NT) {
        const int v = atomicExch(a.rank_acc + r, 0);
        if (a.out_per_rank) a.out_per_rank[r] = v;
    }
    for (int n = threadIdx.x; n < a.nodes; n += NT) {
        const int v = atomicExch(a.node_acc + n, 0);
        if (a.out_per_node) a.out_per_node[n] = v;
    }
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
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        ids[k] = (tv && k < K) ? a.topk_clone[t * K + k] : -1;
        lr[k] = (tv && k < K) ? a.slot_idx[t * K + k] : 0;
    }
    const int n = C * E;
#pragma unroll 8
    for (int i = tid; i < n; i += NT) tile[i] = a.hist[i];
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
#pragma unroll
    for (int k = 0; k < KMAX; ++k) off[k] = ids[k] >= 0 ? psum[ids[k]] + base[ids[k]] + lr[k] : 0;
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
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        ids[k] = (k < K) ? a.topk_clone[t * K + k] : -1;
        lr[k] = (k < K) ? a.slot_idx[t * K + k] : 0;
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        off[k] = ids[k] >= 0 ? a.psum_expert[ids[k]] + base[ids[k]] + lr[k] : 0;
    store_slots<KMAX>(a, t, ids, off);
}

// Path A: the routing LDS of one block of `waves` waves plus the prefix
// [E+1] and the scan scratch [2 * threads].
size_t fused_lds_bytes(const LayoutArgs& a, int waves)
{
    return route_lds_bytes(waves, a.E, a.R, a.nodes) +
           ((size_t)a.E + 1 + 2 * (size_t)waves * kWave) * 4;
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
