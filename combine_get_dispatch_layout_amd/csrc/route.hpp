// Device building blocks of the routing layout, shared by the layout
// kernels (layout.hip), the single-launch layout + dispatch (fused.hip) and
// the launches that run the next batch's layout beside dispatch and combine
// (overlap.hip).  See layout.hip for what is computed and its sources.
#pragma once

#include "ep_internal.hpp"

namespace epk {
namespace route {

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
                                            int (&ids)[KMAX], int (&lr)[KMAX],
                                            bool write_rows = true)
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
            if (write_rows) a.topk_clone[t * K + k] = v;
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
    if (a.out_in_rank != nullptr && tv && write_rows) {
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
    if (a.cap > 0) {   // fixed capacity: expert e starts at e*cap
        for (int e = tid; e <= E; e += NT) psum[e] = e * a.cap;
        __syncthreads();
        return;
    }
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
        if (a.cap > 0) {   // rows filled: min(count, cap), prefix within the rank
            int v = 0;
            for (int q = a.counts_as_prefix ? first : e; q <= e; ++q) v += min(cnt[q], a.cap);
            a.recv_list[e] = v;
        } else {
            a.recv_list[e] = a.counts_as_prefix ? psum[e + 1] - psum[first] : psum[e + 1] - psum[e];
        }
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
    // unused rows per expert: at most A-1 (packed) or cap (fixed capacity)
    const int W = a.cap > 0 ? a.cap : a.A - 1;
    if (W <= 0 || e0 >= a.E) return;
    const int ne = (a.E - e0 + step - 1) / step;
    int2 m;
    m.x = -1;
    m.y = -1;
    for (int i = threadIdx.x; i < ne * W; i += NT) {
        const int ei = i / W;
        const int e = e0 + ei * step;
        const int filled = a.cap > 0 ? min(cnt[e], a.cap) : cnt[e];
        const int row = psum[e] + filled + (i - ei * W);
        if (row < psum[e + 1]) reinterpret_cast<int2*>(a.src_meta)[row] = m;
    }
}

// Receive row of a pair at position `pos` inside expert e's segment that
// starts at `start`; -1 (and the capacity flag) when a fixed-capacity
// segment is full.
__device__ __forceinline__ int final_slot(const LayoutArgs& a, int start, int pos, bool& dropped)
{
    if (a.cap > 0 && pos >= a.cap) {
        dropped = true;
        return -1;
    }
    return start + pos;
}

template <int KMAX>
__device__ __forceinline__ void flag_dropped(const LayoutArgs& a, bool dropped)
{
    if (__ballot(dropped) != 0ull && (threadIdx.x & (kWave - 1)) == 0)
        atomicOr(a.ctrl + kCtrlFlags, kFlagCapacity);
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
        const int s = ids[k] >= 0 ? off[k] : -1;   // off is -1 for a dropped pair
        a.slot_idx[t * K + k] = s;
        if (s >= 0) {
            int2 m;
            m.x = (int)t;
            m.y = k;
            reinterpret_cast<int2*>(a.src_meta)[s] = m;
        }
    }
}


// LDS of the single-block path: routing of `waves` waves plus the prefix
// [E+1] and the scan scratch [2 * threads].
inline size_t fused_lds_bytes(const LayoutArgs& a, int waves)
{
    return route_lds_bytes(waves, a.E, a.R, a.nodes) +
           ((size_t)a.E + 1 + 2 * (size_t)waves * kWave) * 4;
}

// ---- block bodies (used by the layout kernels and by the launches that run
// a layout phase of the next batch beside dispatch or combine) ------------

// Path A: one block of WAVES waves does the whole layout of N <= WAVES*64
// tokens in LDS (fused_lds_bytes).
template <int KMAX, int WAVES>
__device__ __forceinline__ void fused_body(const LayoutArgs& a, unsigned char* smem)
{
    constexpr int NT = WAVES * kWave;
    const RouteLds L = carve_route(smem, WAVES, a.E, a.R);
    int ids[KMAX], lr[KMAX];
    route_block<KMAX, WAVES>(a, 0, L, ids, lr);
    // prefix [E+1] and scan scratch [2*NT] follow the routing LDS
    int32_t* psum = L.ncnt + a.nodes;
    int32_t* scratch = psum + a.E + 1;
    aligned_prefix<NT>(a, L.bhist, psum, scratch);
    int off[KMAX];
    bool dropped = false;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        off[k] = ids[k] >= 0 ? final_slot(a, psum[ids[k]], lr[k], dropped) : 0;
    flag_dropped<KMAX>(a, dropped);
    store_slots<KMAX>(a, threadIdx.x, ids, off);
    write_expert_arrays<NT>(a, L.bhist, psum);
    write_padding<NT>(a, L.bhist, psum, 0, 1);
    for (int r = threadIdx.x; r < a.R; r += NT)
        if (a.out_per_rank) a.out_per_rank[r] = L.rcnt[r];
    for (int n = threadIdx.x; n < a.nodes; n += NT)
        if (a.out_per_node) a.out_per_node[n] = L.ncnt[n];
}

// Paths B and C, first phase, layout block b (tokens [256b, 256b+256)):
// writes the block histogram, the in-block ranks (into slot_idx, finished by
// the second phase) and adds the distinct-token counts to the accumulators.
template <int KMAX>
__device__ __forceinline__ void count_body(const LayoutArgs& a, int b, unsigned char* smem)
{
    constexpr int WAVES = kLayoutBlock / kWave;
    const RouteLds L = carve_route(smem, WAVES, a.E, a.R);
    int ids[KMAX], lr[KMAX];
    const int64_t t0 = (int64_t)b * kLayoutBlock;
    route_block<KMAX, WAVES>(a, t0, L, ids, lr);
    const int tid = threadIdx.x, K = a.K;
    const int64_t t = t0 + tid;
    if (t < a.num_tokens) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K) a.slot_idx[t * K + k] = lr[k];
    }
    for (int e = tid; e < a.E; e += kLayoutBlock) a.hist[(int64_t)b * a.E + e] = L.bhist[e];
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

// LDS of finish_lean: totals, bases [E] each, prefix [E+1], scan scratch
// [2*256] and the column partials [2*256].
inline size_t finish_lean_lds_bytes(const LayoutArgs& a)
{
    return ((size_t)3 * a.E + 1 + 4 * kLayoutBlock) * 4;
}

// Paths B's second phase for layout block b of C, reading the C x E
// histogram straight from memory (a few KiB of LDS, so it can share a launch
// with bandwidth-bound blocks): each column's total and the part before
// block b, split over 256/E threads per column with batched loads; then the
// aligned prefix and block b's final slots; padding rows of experts b, b+C,
// ...; block 0 writes the per-expert arrays and flushes the rank totals.
template <int KMAX>
__device__ __forceinline__ void finish_lean(const LayoutArgs& a, int C, int b, unsigned char* smem)
{
    constexpr int NT = kLayoutBlock;
    constexpr int kBatch = 8;
    const int E = a.E, K = a.K, tid = threadIdx.x;
    int32_t* tot = reinterpret_cast<int32_t*>(smem);   // [E]
    int32_t* base = tot + E;                            // [E]
    int32_t* psum = base + E;                           // [E+1]
    int32_t* scratch = psum + E + 1;                    // [2*NT]
    int32_t* part_pre = scratch + 2 * NT;               // [NT]
    int32_t* part_all = part_pre + NT;                  // [NT]

    const int64_t t = (int64_t)b * kLayoutBlock + tid;
    const bool tv = t < a.num_tokens;
    int ids[KMAX], lr[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        ids[k] = (tv && k < K) ? a.topk_clone[t * K + k] : -1;
        lr[k] = (tv && k < K) ? a.slot_idx[t * K + k] : 0;
    }

    const int EPT = E < NT ? E : NT;
    int P = NT / EPT;
    if (P > C) P = C;
    for (int eb = 0; eb < E; eb += EPT) {
        const int e = eb + tid % EPT, p = tid / EPT;
        const bool act = e < E && p < P;
        const int r0 = act ? p * C / P : 0;
        const int r1 = act ? (p + 1) * C / P : 0;
        int pre = 0, all = 0;
        for (int r = r0; r < r1; r += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) v[j] = r + j < r1 ? a.hist[(int64_t)(r + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                all += v[j];
                pre += (r + j < b) ? v[j] : 0;
            }
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
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        off[k] = ids[k] >= 0 ? final_slot(a, psum[ids[k]], base[ids[k]] + lr[k], dropped) : 0;
    flag_dropped<KMAX>(a, dropped);
    store_slots<KMAX>(a, t, ids, off);
    write_padding<NT>(a, tot, psum, b, C);
    if (b == 0) {
        write_expert_arrays<NT>(a, tot, psum);
        flush_rank_totals<NT>(a);
    }
}

}  // namespace route
}  // namespace epk
