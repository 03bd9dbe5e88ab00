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

// An entry's id when it is valid, else 0: an always-valid index, so that a
// row's K table reads are issued together and waited for once (a read under
// a per-entry branch is waited for before the next one is issued).
__device__ __forceinline__ int safe_id(int id) { return id >= 0 ? id : 0; }

// n / d for the host-computed magic of d (div_magic; 0 for d == 1), as
// arithmetic rather than a branch: umulhi(n, 0) is 0, and n is added back
// only when the magic is 0.
__device__ __forceinline__ int div_by(int n, uint32_t magic)
{
    const int keep = -(int)(magic == 0u);
    return (int)__umulhi((uint32_t)n, magic) + (n & keep);
}

// LDS of the routing phase for a block of `waves` waves.
struct RouteLds {
    unsigned long long* tab;   // [waves][E] lane masks (free after the phase)
    int32_t* wcnt;             // [waves][E] per-wave counts -> exclusive bases
    int32_t* bhist;            // [E] block totals
    int32_t* rcnt;             // [R] distinct tokens per rank
    int32_t* ncnt;             // [nodes]
};

__host__ __device__ inline size_t route_lds_bytes(int waves, int E, int R, int nodes)
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

// K entries of an [N,K] int32 row.  vec: K % 4 == 0 and the row is 16-byte
// aligned, so the row moves as K/4 16-byte vectors.
template <int KMAX>
__device__ __forceinline__ void load_row(const int32_t* p, int K, bool vec, bool valid, int fill,
                                         int (&v)[KMAX])
{
    if constexpr (KMAX >= 4) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < KMAX / 4; ++q) {
                int4 x = make_int4(fill, fill, fill, fill);
                if (valid && 4 * q < K) x = reinterpret_cast<const int4*>(p)[q];
                v[4 * q] = x.x;
                v[4 * q + 1] = x.y;
                v[4 * q + 2] = x.z;
                v[4 * q + 3] = x.w;
            }
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) v[k] = (valid && k < K) ? p[k] : fill;
}

template <int KMAX>
__device__ __forceinline__ void store_row(int32_t* p, int K, bool vec, const int (&v)[KMAX])
{
    if constexpr (KMAX >= 4) {
        if (vec) {
#pragma unroll
            for (int q = 0; q < KMAX / 4; ++q)
                if (4 * q < K)
                    reinterpret_cast<int4*>(p)[q] =
                        make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (k < K) p[k] = v[k];
}

// Inclusive sum over each row of 16 lanes (DPP row shifts; lanes shifted in
// from outside the row read 0).  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t row_incl_sum(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
    return x;
}

// Sum of x over the wave, in every lane (every lane active).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x)
{
    x = row_incl_sum(x);
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 15) +
           (uint32_t)__builtin_amdgcn_readlane((int)x, 31) +
           (uint32_t)__builtin_amdgcn_readlane((int)x, 47) +
           (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Inclusive prefix sum of x over the wave's lanes (every lane active).
__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
    const uint32_t r = row_incl_sum((uint32_t)x);
    const int t0 = __builtin_amdgcn_readlane((int)r, 15);
    const int t1 = __builtin_amdgcn_readlane((int)r, 31);
    const int t2 = __builtin_amdgcn_readlane((int)r, 47);
    const int row = lane >> 4;
    return (int)r + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

// Per-wave counts of the set bits of a 64-bit mask held by every lane, for
// bits [0, n), n <= 64: lane b receives the number of lanes with bit b set.
// Four bits at a time become four byte counters of one word (a wave has 64
// lanes, so a byte never overflows), summed over the wave by DPP.  Every
// lane of the wave must be active.
__device__ __forceinline__ int wave_bit_counts(uint64_t m, int n, int lane)
{
    int mine = 0;
    for (int q = 0; 4 * q < n; ++q) {
        const uint32_t nib = (uint32_t)(m >> (4 * q)) & 15u;
        const uint32_t spread =
            (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
        const uint32_t tot = wave_sum(spread);
        if ((lane >> 2) == q) mine = (int)((tot >> (8 * (lane & 3))) & 0xFFu);
    }
    return mine;
}

// Token t's routing row with ids outside [-1, E) replaced by -1; returns
// whether it had any.
template <int KMAX>
__device__ __forceinline__ bool load_ids(const LayoutArgs& a, int64_t t, bool valid,
                                         int (&ids)[KMAX])
{
    if (a.derive_src != nullptr) {
        // the ranks of the expert routing's row, each rank once (bad expert
        // ids are masked here and flagged by the expert-level layout)
        load_row<KMAX>(a.derive_src + t * a.K, a.K, a.topk_vec, valid, -1, ids);
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            ids[k] = (ids[k] >= 0 && ids[k] < a.derive_E) ? div_by(ids[k], a.derive_magic) : -1;
#pragma unroll
        for (int k = KMAX - 1; k > 0; --k) {
            bool rep = false;
#pragma unroll
            for (int q = 0; q < k; ++q) rep |= ids[q] == ids[k];
            if (rep) ids[k] = -1;
        }
        return false;
    }
    load_row<KMAX>(a.topk + t * a.K, a.K, a.topk_vec, valid, -1, ids);
    bool bad = false;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (ids[k] < -1 || ids[k] >= a.E) {
            bad = true;
            ids[k] = -1;
        }
    }
    return bad;
}

// The token's ranks as a bit mask (R <= 64; 0 otherwise).
template <int KMAX>
__device__ __forceinline__ uint64_t rank_mask(const LayoutArgs& a, const int (&ids)[KMAX])
{
    uint64_t m = 0ull;
    if (a.R <= 64) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)   // selects, not branches
            m |= (ids[k] >= 0 ? 1ull : 0ull) << div_by(safe_id(ids[k]), a.nle_magic);
    }
    return m;
}

// Adds the wave's tokens to the distinct-token counts per rank and node in
// LDS (every lane of the wave calls it).  R <= 64: per-wave counts by
// ballot over the rank masks, one LDS add per rank; otherwise the first
// occurrence of each rank (and node) in a row, by comparison.
template <int KMAX>
__device__ __forceinline__ void add_rank_counts(const LayoutArgs& a, const int (&ids)[KMAX],
                                                uint64_t m, int lane, int32_t* rcnt, int32_t* ncnt)
{
    const int R = a.R;
    if (R <= 64) {
        const int rc = wave_bit_counts(m, R, lane);
        if (lane < R && rc != 0) atomicAdd(rcnt + lane, rc);
        if (a.nodes > 0) {
            const int rpn = a.ranks_per_node;
            const uint64_t gm = rpn >= 64 ? ~0ull : (1ull << rpn) - 1ull;
            uint64_t nm = 0ull;
            for (int n = 0; n < a.nodes; ++n)
                nm |= (((m >> (n * rpn)) & gm) != 0ull ? 1ull : 0ull) << n;
            const int nc = wave_bit_counts(nm, a.nodes, lane);
            if (lane < a.nodes && nc != 0) atomicAdd(ncnt + lane, nc);
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (ids[k] < 0) continue;
        const int rk = div_by(ids[k], a.nle_magic);
        const int nd = a.nodes > 0 ? div_by(rk, a.rpn_magic) : 0;
        bool first = true, nfirst = true;
#pragma unroll
        for (int q = 0; q < k; ++q) {
            if (ids[q] < 0) continue;
            const int rq = div_by(ids[q], a.nle_magic);
            first &= rq != rk;
            if (a.nodes > 0) nfirst &= div_by(rq, a.rpn_magic) != nd;
        }
        if (first) atomicAdd(rcnt + rk, 1);
        if (a.nodes > 0 && nfirst) atomicAdd(ncnt + nd, 1);
    }
}

// One token's is_token_in_rank row (m from rank_mask when R <= 64).
template <int KMAX>
__device__ __forceinline__ void write_in_rank_row(const LayoutArgs& a, const int (&ids)[KMAX],
                                                  uint64_t m, uint8_t* row)
{
    const int R = a.R;
    if (R <= 64) {
        if (a.in_rank_words) {
            // 0/1 bytes from 4 bits of the mask per word; 16-byte stores when
            // the row holds whole, aligned 16-byte pieces
            uint32_t* roww = reinterpret_cast<uint32_t*>(row);
            const bool vec = R % 16 == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
            for (int q = 0; q < R / 4; q += vec ? 4 : 1) {
                uint32_t wd[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t nib = (uint32_t)(m >> (4 * (q + i)));
                    wd[i] = (nib & 1u) | ((nib & 2u) << 7) | ((nib & 4u) << 14) | ((nib & 8u) << 21);
                }
                if (vec) *reinterpret_cast<u32x4*>(roww + q) = u32x4{wd[0], wd[1], wd[2], wd[3]};
                else roww[q] = wd[0];
            }
        } else {
            for (int r = 0; r < R; ++r) row[r] = (uint8_t)((m >> r) & 1ull);
        }
        return;
    }
    if (a.in_rank_words) {
        uint32_t* roww = reinterpret_cast<uint32_t*>(row);
        for (int q = 0; q < R / 4; ++q) {
            uint32_t word = 0u;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (ids[k] < 0) continue;
                const int rk = div_by(ids[k], a.nle_magic);
                if ((rk >> 2) == q) word |= 1u << ((rk & 3) * 8);
            }
            roww[q] = word;
        }
    } else {
        for (int r = 0; r < R; ++r) {
            uint8_t b = 0;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                b |= (ids[k] >= 0 && div_by(ids[k], a.nle_magic) == r) ? 1 : 0;
            row[r] = b;
        }
    }
}

// Routing phase for the block's tokens t0 .. t0 + WAVES*64 - 1 (one per
// thread).  LEAN: the kernel shares its launch with streaming blocks and
// must stay within 64 vector registers, so the per-entry table reads of the
// level loop are not batched.  Leaves the sanitised ids and the in-block rank of every pair in
// registers, the block histogram in L.bhist and the distinct-token counts in
// L.rcnt / L.ncnt; writes the topk clone and the is_token_in_rank rows.
template <int KMAX, int WAVES, bool LEAN = false>
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

    for (int i = tid; i < R; i += NT) L.rcnt[i] = 0;
    for (int i = tid; i < a.nodes; i += NT) L.ncnt[i] = 0;

    const bool bad = load_ids<KMAX>(a, t, tv, ids);
    if (tv && write_rows) store_row<KMAX>(a.topk_clone + t * K, K, a.row_vec, ids);
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(a.ctrl + kCtrlFlags, kFlagBadId);

    // Copies of ids[k] earlier in the same row (its occurrence level), 4 bits
    // each; the in-block rank starts there and lr accumulates the rest.
    static_assert(KMAX <= 16, "occurrence levels are packed 4 bits per entry");
    uint64_t occp = 0ull;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int c = 0;
#pragma unroll
        for (int q = 0; q < k; ++q) c += (ids[q] == ids[k]) ? 1 : 0;
        lr[k] = c;
        occp |= (uint64_t)c << (4 * k);
    }

    unsigned long long* mytab = L.tab + w * E;
    int32_t* mycnt = L.wcnt + w * E;

    // Each wave owns its table and counts, so the occurrence levels need only
    // wave-level ordering: a wave's LDS operations complete in issue order,
    // and the wavefront fences keep the compiler from reordering them.  Level
    // 0 always runs (it writes the wave's counts); later levels only while a
    // row of the wave repeats an expert.
    for (int j = 0; j < KMAX; ++j) {
        if (j > 0) {
            bool have = false;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                have |= (ids[k] >= 0 && (int)((occp >> (4 * k)) & 15ull) == j);
            if (__ballot(have) == 0ull) break;
        }
        for (int e = lane; e < E; e += kWave) mytab[e] = 0ull;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (ids[k] >= 0 && (int)((occp >> (4 * k)) & 15ull) == j)
                atomicOr(mytab + ids[k], 1ull << lane);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if constexpr (LEAN) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (ids[k] >= 0) lr[k] += count_below(mytab[ids[k]]);
        } else {
            unsigned long long mk[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; ++k) mk[k] = mytab[safe_id(ids[k])];
#pragma unroll
            for (int k = 0; k < KMAX; ++k) lr[k] += ids[k] >= 0 ? count_below(mk[k]) : 0;
        }
        // the level's per-expert counts, four table words in flight per lane
        for (int e0 = lane; e0 < E; e0 += 4 * kWave) {
            unsigned long long m[4];
            int c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = e0 + i * kWave;
                if constexpr (LEAN) {
                    m[i] = e < E ? mytab[e] : 0ull;
                    c[i] = (j > 0 && e < E) ? mycnt[e] : 0;
                } else {   // in-range reads, issued unconditionally
                    const int ec = e < E ? e : E - 1;
                    m[i] = mytab[ec];
                    c[i] = mycnt[ec];
                    if (e >= E) m[i] = 0ull;
                    if (j == 0 || e >= E) c[i] = 0;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = e0 + i * kWave;
                if (e < E) mycnt[e] = c[i] + __popcll(m[i]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    __syncthreads();

    // Block totals; wcnt[w][e] becomes the count of earlier waves.
    for (int e = tid; e < E; e += NT) {
        int v[WAVES];   // all reads first, then the writes: one wait
#pragma unroll
        for (int q = 0; q < WAVES; ++q) v[q] = L.wcnt[q * E + e];
        int run = 0;
#pragma unroll
        for (int q = 0; q < WAVES; ++q) {
            L.wcnt[q * E + e] = run;
            run += v[q];
        }
        L.bhist[e] = run;
    }

    // Count each token once per rank and once per node, and write its
    // is_token_in_rank row.
    const uint64_t m = rank_mask<KMAX>(a, ids);
    add_rank_counts<KMAX>(a, ids, m, lane, L.rcnt, L.ncnt);
    if (a.out_in_rank != nullptr && tv && write_rows)
        write_in_rank_row<KMAX>(a, ids, m, a.out_in_rank + t * R);
    __syncthreads();
    int before[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) before[k] = L.wcnt[w * E + safe_id(ids[k])];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) lr[k] = ids[k] >= 0 ? lr[k] + before[k] : -1;
}

// Exclusive prefix of the aligned counts cnt[0..E) into psum[0..E]; NT
// threads, each owning ceil(E/NT) consecutive experts: a shuffle scan
// inside each wave, one barrier, then the wave offsets.
// scratch: NT/64 ints.
template <int NT>
__device__ __forceinline__ void aligned_prefix(const LayoutArgs& a, const int32_t* cnt,
                                               int32_t* psum, int32_t* scratch)
{
    constexpr int EPT = (kMaxExperts + NT - 1) / NT;
    constexpr int WAVES = NT / kWave;
    const int tid = threadIdx.x, E = a.E, lane = tid & (kWave - 1), w = tid / kWave;
    if (a.cap > 0) {   // fixed capacity: expert e starts at e*cap
        for (int e = tid; e <= E; e += NT) psum[e] = e * a.cap;
        __syncthreads();
        return;
    }
    // thread tid owns experts [tid*ept, tid*ept + ept): one each while E <= NT
    const int ept = (E + NT - 1) / NT;
    int al[EPT];
    int own = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * ept + j;
        const int c = (j < ept && e < E) ? cnt[e] : 0;
        al[j] = a.A == 1 ? c : ((c + a.A - 1) / a.A) * a.A;
        own += al[j];
    }
    const int incl = wave_incl_scan(own, lane);
    if (lane == kWave - 1) scratch[w] = incl;
    __syncthreads();
    int run = incl - own;
    for (int q = 0; q < w; ++q) run += scratch[q];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * ept + j;
        if (j < ept && e < E) psum[e] = run;
        run += al[j];
    }
    if (tid == NT - 1) psum[E] = run;
    __syncthreads();
    (void)WAVES;
}

// Per-expert handle arrays and caller outputs from the counts and prefix
// (both in LDS).
template <int NT>
__device__ __forceinline__ void write_expert_arrays(const LayoutArgs& a, const int32_t* cnt,
                                                    const int32_t* psum)
{
    const int tid = threadIdx.x, E = a.E;
    for (int e = tid; e <= E; e += NT) a.psum_expert[e] = psum[e];
    for (int e = tid; e < E; e += NT) {
        a.num_unaligned[e] = cnt[e];
        if (a.out_per_expert) a.out_per_expert[e] = cnt[e];
        const int first = div_by(e, a.nle_magic) * a.nle;   // the rank's first expert
        if (a.cap > 0) {   // rows filled: min(count, cap), prefix within the rank
            int v = 0;
            for (int q = a.counts_as_prefix ? first : e; q <= e; ++q) v += min(cnt[q], a.cap);
            a.recv_list[e] = v;
        } else {
            a.recv_list[e] = a.counts_as_prefix ? psum[e + 1] - psum[first] : psum[e + 1] - psum[e];
        }
    }
    if (a.counts_only) return;   // the rank-level layout writes these
    for (int r = tid; r <= a.R; r += NT) a.psum_rank[r] = psum[r * a.nle];
    if (tid == 0) a.ctrl[kCtrlNumSlots] = (uint32_t)psum[E];
}

// (-1,-1) metadata of the padding rows of experts e0, e0+step, ...  At
// most A-1 rows per expert: the (expert, row) pairs are flattened so that
// consecutive threads write consecutive rows.
template <int NT>
__device__ __forceinline__ void write_padding(const LayoutArgs& a, const int32_t* cnt,
                                              const int32_t* psum, int e0, int step)
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
    int sl[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) sl[k] = ids[k] >= 0 ? off[k] : -1;   // off is -1 when dropped
    store_row<KMAX>(a.slot_idx + t * K, K, a.row_vec, sl);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k >= K) break;
        if (sl[k] >= 0) {
            int2 m;
            m.x = (int)t;
            m.y = k;
            reinterpret_cast<int2*>(a.src_meta)[sl[k]] = m;
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
template <int KMAX, int WAVES, bool LEAN = false>
__device__ __forceinline__ void fused_body(const LayoutArgs& a, unsigned char* smem)
{
    constexpr int NT = WAVES * kWave;
    const RouteLds L = carve_route(smem, WAVES, a.E, a.R);
    int ids[KMAX], lr[KMAX];
    route_block<KMAX, WAVES, LEAN>(a, 0, L, ids, lr);
    // prefix [E+1] and scan scratch [2*NT] follow the routing LDS
    int32_t* psum = L.ncnt + a.nodes;
    int32_t* scratch = psum + a.E + 1;
    aligned_prefix<NT>(a, L.bhist, psum, scratch);
    int off[KMAX];
    bool dropped = false;
    int start[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) start[k] = psum[safe_id(ids[k])];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        off[k] = ids[k] >= 0 ? final_slot(a, start[k], lr[k], dropped) : 0;
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
template <int KMAX, bool LEAN = false>
__device__ __forceinline__ void count_body(const LayoutArgs& a, int b, unsigned char* smem)
{
    constexpr int WAVES = kLayoutBlock / kWave;
    const RouteLds L = carve_route(smem, WAVES, a.E, a.R);
    int ids[KMAX], lr[KMAX];
    const int64_t t0 = (int64_t)b * kLayoutBlock;
    route_block<KMAX, WAVES, LEAN>(a, t0, L, ids, lr);
    const int tid = threadIdx.x, K = a.K;
    const int64_t t = t0 + tid;
    if (t < a.num_tokens && !a.counts_only) store_row<KMAX>(a.slot_idx + t * K, K, a.row_vec, lr);
    for (int e = tid; e < a.E; e += kLayoutBlock) a.hist[(int64_t)b * a.E + e] = L.bhist[e];
    if (a.no_rank_counts) return;
    // this block's copy of the accumulators (spreads the atomics of many
    // blocks over several addresses per rank)
    const int copy = a.acc_copies > 1 ? (b % a.acc_copies) * a.acc_stride : 0;
    for (int r = tid; r < a.R; r += kLayoutBlock)
        if (L.rcnt[r] != 0) atomicAdd(a.rank_acc + copy + r, L.rcnt[r]);
    for (int n = tid; n < a.nodes; n += kLayoutBlock)
        if (L.ncnt[n] != 0) atomicAdd(a.node_acc + copy + n, L.ncnt[n]);
}

// Distinct-token totals from the accumulators (the sum of the acc_copies
// copies in use), which are re-zeroed for the next call.  The additions were
// made by an earlier launch, so plain loads see them; the copies are read at
// once.
//   RankTotals: when every rank and node has a thread of its own
//   (R, nodes <= NT) the loads are issued by rank_totals_load at the start
//   of a block, beside its other loads, so that rank_totals_store at its
//   end waits for nothing; otherwise rank_totals_store reads them itself.
struct RankTotals {
    int r[kAccCopies], n[kAccCopies];
    bool early;
};

template <int NT>
__device__ __forceinline__ void rank_totals_load(const LayoutArgs& a, RankTotals& rt)
{
    const int tid = threadIdx.x;
    rt.early = a.R <= NT && a.nodes <= NT;
    if (!rt.early) return;
#pragma unroll
    for (int c = 0; c < kAccCopies; ++c) {
        const bool used = c < a.acc_copies;
        rt.r[c] = used && tid < a.R ? a.rank_acc[c * a.acc_stride + tid] : 0;
        rt.n[c] = used && tid < a.nodes ? a.node_acc[c * a.acc_stride + tid] : 0;
    }
}

template <int NT>
__device__ __forceinline__ void rank_totals_store(const LayoutArgs& a, const RankTotals& rt)
{
    if (rt.early) {
        const int tid = threadIdx.x;
        int rs = 0, ns = 0;
#pragma unroll
        for (int c = 0; c < kAccCopies; ++c) {
            rs += rt.r[c];
            ns += rt.n[c];
        }
        if (tid < a.R) {
#pragma unroll
            for (int c = 0; c < kAccCopies; ++c)
                if (c < a.acc_copies) a.rank_acc[c * a.acc_stride + tid] = 0;
            if (a.out_per_rank) a.out_per_rank[tid] = rs;
        }
        if (tid < a.nodes) {
#pragma unroll
            for (int c = 0; c < kAccCopies; ++c)
                if (c < a.acc_copies) a.node_acc[c * a.acc_stride + tid] = 0;
            if (a.out_per_node) a.out_per_node[tid] = ns;
        }
        return;
    }
    for (int r = threadIdx.x; r < a.R; r += NT) {
        int v[kAccCopies];
#pragma unroll
        for (int c = 0; c < kAccCopies; ++c) v[c] = c < a.acc_copies ? a.rank_acc[c * a.acc_stride + r] : 0;
        int sum = 0;
#pragma unroll
        for (int c = 0; c < kAccCopies; ++c) {
            sum += v[c];
            if (c < a.acc_copies) a.rank_acc[c * a.acc_stride + r] = 0;
        }
        if (a.out_per_rank) a.out_per_rank[r] = sum;
    }
    for (int n = threadIdx.x; n < a.nodes; n += NT) {
        int v[kAccCopies];
#pragma unroll
        for (int c = 0; c < kAccCopies; ++c) v[c] = c < a.acc_copies ? a.node_acc[c * a.acc_stride + n] : 0;
        int sum = 0;
#pragma unroll
        for (int c = 0; c < kAccCopies; ++c) {
            sum += v[c];
            if (c < a.acc_copies) a.node_acc[c * a.acc_stride + n] = 0;
        }
        if (a.out_per_node) a.out_per_node[n] = sum;
    }
}

template <int NT>
__device__ __forceinline__ void flush_rank_totals(const LayoutArgs& a)
{
    RankTotals rt;
    rt.early = false;
    rank_totals_store<NT>(a, rt);
}

// LDS of finish_lean with NT threads: totals [E], bases [NT/256][E], prefix
// [E+1], scan scratch [2*NT] and the column partials [2*NT].
__host__ __device__ inline size_t finish_lean_lds_bytes(const LayoutArgs& a, int NT)
{
    return ((size_t)(2 + NT / kLayoutBlock) * a.E + 1 + 4 * (size_t)NT) * 4;
}

// Path B's second phase for finish block b of ceil(C / (NT/256)), reading
// the C x E histogram straight from memory (a few KiB of LDS, so it can
// share a launch with bandwidth-bound blocks).  The block finishes the
// NT/256 count blocks cb0 = b*NT/256 ...: each column's total and the part
// before cb0, split over NT/E threads per column with batched loads; the
// base of each later count block adds the histogram rows in between; then
// the aligned prefix and the final slots of the block's NT tokens; padding
// rows of experts b, b + blocks, ...; block 0 writes the per-expert arrays
// and flushes the rank totals.
template <int KMAX, int NT>
__device__ __forceinline__ void finish_lean(const LayoutArgs& a, int C, int b, unsigned char* smem)
{
    constexpr int G = NT / kLayoutBlock;   // count blocks per finish block
    constexpr int kBatch = 8;
    const int E = a.E, K = a.K, tid = threadIdx.x;
    const int cb0 = b * G;
    const int blocks = (C + G - 1) / G;
    int32_t* tot = reinterpret_cast<int32_t*>(smem);   // [E]
    int32_t* base = tot + E;                            // [G][E]
    int32_t* psum = base + G * E;                       // [E+1]
    int32_t* scratch = psum + E + 1;                    // [2*NT]
    int32_t* part_pre = scratch + 2 * NT;               // [NT]
    int32_t* part_all = part_pre + NT;                  // [NT]

    // Column e of the histogram is split over P threads (NT / E of them when
    // E < NT), each summing its rows in batches of kBatch loads.  The first
    // batch of the first columns is issued before anything else, beside the
    // token rows and the rank totals, so that a small histogram costs no
    // round trip of its own.
    const int EPT = E < NT ? E : NT;
    int P = NT / EPT;
    if (P > C) P = C;
    int v0[kBatch];
    {
        const int e = tid % EPT, p = tid / EPT;
        const bool act = e < E && p < P;
        const int r0 = act ? p * C / P : 0;
        const int r1 = act ? (p + 1) * C / P : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            v0[j] = r0 + j < r1 ? a.hist[(int64_t)(r0 + j) * E + e] : 0;
    }

    const int64_t t = (int64_t)b * NT + tid;
    const bool tv = t < a.num_tokens && !a.counts_only;
    int ids[KMAX], lr[KMAX];
    load_row<KMAX>(a.topk_clone + t * K, K, a.row_vec, tv, -1, ids);
    load_row<KMAX>(a.slot_idx + t * K, K, a.row_vec, tv, 0, lr);
    // block 0's rank totals: loaded now, beside the rows and the histogram
    RankTotals rt;
    rt.early = false;
    if (b == 0 && !a.no_rank_counts) rank_totals_load<NT>(a, rt);

    for (int eb = 0; eb < E; eb += EPT) {
        const int e = eb + tid % EPT, p = tid / EPT;
        const bool act = e < E && p < P;
        const int r0 = act ? p * C / P : 0;
        const int r1 = act ? (p + 1) * C / P : 0;
        int pre = 0, all = 0;
        for (int r = r0; r < r1; r += kBatch) {
            int v[kBatch];
            if (eb == 0 && r == r0) {
#pragma unroll
                for (int j = 0; j < kBatch; ++j) v[j] = v0[j];
            } else {
#pragma unroll
                for (int j = 0; j < kBatch; ++j)
                    v[j] = r + j < r1 ? a.hist[(int64_t)(r + j) * E + e] : 0;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                all += v[j];
                pre += (r + j < cb0) ? v[j] : 0;
            }
        }
        int sp = pre, sa = all;
        if (P > 1) {   // the column's partial sums meet in LDS
            if (act) {
                part_pre[p * EPT + (e - eb)] = pre;
                part_all[p * EPT + (e - eb)] = all;
            }
            __syncthreads();
            if (act && p == 0) {
                sp = 0;
                sa = 0;
                for (int q = 0; q < P; ++q) {
                    sp += part_pre[q * EPT + (e - eb)];
                    sa += part_all[q * EPT + (e - eb)];
                }
            }
        }
        if (act && p == 0) {
            base[e] = sp;
#pragma unroll
            for (int g = 1; g < G; ++g) {
                const int r = cb0 + g - 1;
                sp += r < C ? a.hist[(int64_t)r * E + e] : 0;
                base[g * E + e] = sp;
            }
            tot[e] = sa;
        }
        if (P > 1) __syncthreads();   // the partials' LDS is reused by the next columns
    }
    if (P == 1) __syncthreads();      // tot and base complete
    aligned_prefix<NT>(a, tot, psum, scratch);

    if (!a.counts_only) {
        const int32_t* mybase = base + (tid / kLayoutBlock) * E;
        int off[KMAX];
        bool dropped = false;
        int start[KMAX], pos[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            start[k] = psum[safe_id(ids[k])];
            pos[k] = mybase[safe_id(ids[k])] + lr[k];
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            off[k] = ids[k] >= 0 ? final_slot(a, start[k], pos[k], dropped) : 0;
        flag_dropped<KMAX>(a, dropped);
        store_slots<KMAX>(a, t, ids, off);
        write_padding<NT>(a, tot, psum, b, blocks);
    }
    if (b == 0) {
        write_expert_arrays<NT>(a, tot, psum);
        if (!a.no_rank_counts) rank_totals_store<NT>(a, rt);
    }
}

}  // namespace route
}  // namespace epk
