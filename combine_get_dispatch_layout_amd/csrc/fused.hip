// Single-launch routing layout + dispatch for small batches (decode).
//
// What is computed: exactly ep_get_layout followed by ep_dispatch over the
// whole batch -- the unified dispatch call of "DeepEP V1 vs V2 深度对比分析"
// §2.2, which takes the routing and returns the received rows together with
// the handle.
//
// Design (N <= 256 tokens, K <= 8): the slot of pair (t,k) is the aligned
// prefix of its expert plus the number of earlier pairs (in (t,k) order)
// with the same expert, so a block needs only two histograms of the routing
// to place its own tokens -- all pairs, and the pairs of tokens before its
// first token -- plus the few rows between.
//   block 0:    the handle's per-expert and per-rank arrays: the histogram,
//               the aligned prefix, the distinct-token counts per rank and
//               node, the padding rows' metadata;
//   blocks 1..: one wave per (token, row chunk), as the dispatch kernel; each
//               wave first issues its chunk's loads, the block builds the two
//               histograms in LDS and the prefix, each wave computes its
//               token's K slots and scatters its chunk.  The wave holding a
//               token's first chunk also writes the token's slot_idx row,
//               source metadata, topk clone and is_token_in_rank row (and
//               raises the capacity flag; block 0 the bad-id flag).
// One launch replaces the layout kernel and the dispatch kernel, and no
// block waits for another.
#include "route.hpp"
#include "scatter.hpp"

namespace epk {

namespace {

using namespace route;
using namespace scatter;

constexpr int kBlock = 256;                      // 4 waves, one token per thread
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kKmax = 8;

// LDS: block 0 needs counts [E], prefix [E+1], scan scratch [2*256] and the
// rank / node counts; the other blocks the two histograms, the prefix, the
// scratch and the routing rows [N][K].
size_t fused_dispatch_lds(const LayoutArgs& a)
{
    const size_t rows = (size_t)kRouteDispatchMaxTokens * kKmax;
    const size_t ranks = (size_t)a.R + a.nodes;
    return ((size_t)2 * a.E + a.E + 1 + 2 * kBlock + (rows > ranks ? rows : ranks)) * 4;
}

// Block 0: every array of the handle that is not per token.
__device__ __forceinline__ void route_dispatch_arrays(const LayoutArgs& a, unsigned char* smem)
{
    const int E = a.E, tid = threadIdx.x, lane = tid & (kWave - 1);
    int32_t* cnt = reinterpret_cast<int32_t*>(smem);   // [E]
    int32_t* psum = cnt + 2 * E;                       // [E+1]
    int32_t* scratch = psum + E + 1;                   // [2*kBlock]
    int32_t* rcnt = scratch + 2 * kBlock;              // [R]
    int32_t* ncnt = rcnt + a.R;                        // [nodes]
    for (int e = tid; e < E; e += kBlock) cnt[e] = 0;
    for (int r = tid; r < a.R; r += kBlock) rcnt[r] = 0;
    for (int n = tid; n < a.nodes; n += kBlock) ncnt[n] = 0;
    int ids[kKmax];
    const bool bad = load_ids<kKmax>(a, tid, tid < a.num_tokens, ids);
    if (__ballot(bad) != 0ull && lane == 0) atomicOr(a.ctrl + kCtrlFlags, kFlagBadId);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKmax; ++k)
        if (ids[k] >= 0) atomicAdd(cnt + ids[k], 1);
    add_rank_counts<kKmax>(a, ids, rank_mask<kKmax>(a, ids), lane, rcnt, ncnt);
    __syncthreads();
    aligned_prefix<kBlock>(a, cnt, psum, scratch);
    write_expert_arrays<kBlock>(a, cnt, psum);
    write_padding<kBlock>(a, cnt, psum, 0, 1);
    for (int r = tid; r < a.R; r += kBlock)
        if (a.out_per_rank) a.out_per_rank[r] = rcnt[r];
    for (int n = tid; n < a.nodes; n += kBlock)
        if (a.out_per_node) a.out_per_node[n] = ncnt[n];
}

template <int QUANT, bool CHANNEL, int VPL, bool ROW_WAIT>
__global__ __launch_bounds__(kBlock) void k_route_dispatch(LayoutArgs la, DispatchArgs da, int NV,
                                                           int NC)
{
    extern __shared__ __align__(16) unsigned char smem[];
    if (blockIdx.x == 0) {
        route_dispatch_arrays(la, smem);
        return;
    }
    const int E = la.E, K = la.K, tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int first = (blockIdx.x - 1) * kWavesPerBlock;   // the block's first item
    const int item = first + wv;
    const int64_t T = item / NC;                           // the wave's token
    const int64_t T0 = first / NC;                         // the block's first token
    const bool has_item = T < da.t_end;
    const int vbase = (item % NC) * (kWave * VPL) + lane;

    // the wave's row chunk is in flight while the block counts
    u32x4 d[VPL];
    if (has_item) load_chunk<VPL>(da, T, vbase, NV, d);

    int32_t* hall = reinterpret_cast<int32_t*>(smem);   // [E] pairs per expert
    int32_t* hbef = hall + E;                           // [E] ... of tokens before T0
    int32_t* psum = hbef + E;                           // [E+1]
    int32_t* scratch = psum + E + 1;                    // [2*kBlock]
    int32_t* rows = scratch + 2 * kBlock;               // [N][K] sanitised routing
    for (int e = tid; e < 2 * E; e += kBlock) hall[e] = 0;
    int ids[kKmax];
    const bool tv = tid < la.num_tokens;
    load_ids<kKmax>(la, tid, tv, ids);   // bad ids are flagged by block 0
    if (tv) {
#pragma unroll
        for (int k = 0; k < kKmax; ++k)
            if (k < K) rows[tid * K + k] = ids[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKmax; ++k) {
        if (ids[k] < 0) continue;
        atomicAdd(hall + ids[k], 1);
        if (tid < T0) atomicAdd(hbef + ids[k], 1);
    }
    __syncthreads();
    aligned_prefix<kBlock>(la, hall, psum, scratch);
    if (!has_item) return;

    // the wave's token: lane k places entry k, from the pairs before T0, the
    // rows T0 .. T-1 and the earlier entries of its own row
    const int32_t* row = rows + T * K;
    int mine = -1;
    bool dropped = false;
    if (lane < K) {
        const int e = row[lane];
        if (e >= 0) {
            int pos = hbef[e];
            for (int64_t t = T0; t < T; ++t)
                for (int q = 0; q < K; ++q) pos += rows[t * K + q] == e ? 1 : 0;
            for (int q = 0; q < lane; ++q) pos += row[q] == e ? 1 : 0;
            mine = final_slot(la, psum[e], pos, dropped);
        }
    }
    int sl[kKmax];
#pragma unroll
    for (int k = 0; k < kKmax; ++k) sl[k] = k < K ? __builtin_amdgcn_readlane(mine, k) : -1;

    if (item % NC == 0) {
        // the token's handle rows, one lane per entry
        if (lane < K) {
            la.slot_idx[T * K + lane] = mine;
            la.topk_clone[T * K + lane] = row[lane];
            if (mine >= 0) {
                int2 m;
                m.x = (int)T;
                m.y = lane;
                reinterpret_cast<int2*>(la.src_meta)[mine] = m;
            }
        }
        if (la.out_in_rank != nullptr) {
            for (int r = lane; r < la.R; r += kWave) {
                uint8_t b = 0;
                for (int k = 0; k < K; ++k)
                    b |= (row[k] >= 0 && div_by(row[k], la.nle_magic) == r) ? 1 : 0;
                la.out_in_rank[T * la.R + r] = b;
            }
        }
        if (__ballot(dropped) != 0ull && lane == 0) atomicOr(la.ctrl + kCtrlFlags, kFlagCapacity);
    }
    scatter_chunk<QUANT, CHANNEL, VPL, kKmax, ROW_WAIT>(da, vbase, NV, d, sl, lane);
}

template <int QUANT, bool CHANNEL, int VPL, bool ROW_WAIT>
hipError_t launch_rd(const LayoutArgs& la, const DispatchArgs& da, int NV, hipStream_t s,
                     LaunchEvents ev)
{
    const int NC = (NV + kWave * VPL - 1) / (kWave * VPL);
    const int64_t items = la.num_tokens * NC;
    // block 0 writes the handle arrays (also for N = 0); the rest scatter
    const int blocks = 1 + (int)((items + kWavesPerBlock - 1) / kWavesPerBlock);
    launch_k(k_route_dispatch<QUANT, CHANNEL, VPL, ROW_WAIT>, dim3(blocks), dim3(kBlock),
             fused_dispatch_lds(la), s, ev.start, ev.stop, la, da, NV, NC);
    return hipGetLastError();
}

}  // namespace

bool route_dispatch_fits(const LayoutArgs& la)
{
    return la.num_tokens <= kRouteDispatchMaxTokens && la.K <= kKmax &&
           fused_dispatch_lds(la) <= kMaxLds;
}

hipError_t launch_route_dispatch(const LayoutArgs& la, const DispatchArgs& da, hipStream_t s,
                                 LaunchEvents ev)
{
    auto launch = [&](auto q, auto ch, auto vpl, auto rw, int NV) {
        return launch_rd<decltype(q)::value, decltype(ch)::value, decltype(vpl)::value,
                         decltype(rw)::value>(la, da, NV, s, ev);
    };
    return dispatch_shape(da, launch);
}

}  // namespace epk
