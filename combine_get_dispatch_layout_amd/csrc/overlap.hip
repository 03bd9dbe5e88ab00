// The next batch's routing layout, run inside the current batch's dispatch
// and combine launches (double-batch overlap on one stream).
//
// What is computed: exactly ep_get_layout for the next batch (no host sync),
// and exactly ep_dispatch / ep_combine for the current one.  "DeepEP V1 vs
// V2 深度对比分析" §5.2 overlaps one micro-batch's communication with
// another's computation; here the latency-bound layout of batch i+1 hides
// under the bandwidth-bound dispatch and combine of batch i.
//
// Design: a launch whose first blocks do layout work and whose other blocks
// are the ordinary dispatch (or combine) waves.  The layout blocks have the
// lowest block ids, so they are scheduled first; beside a prefill batch's
// streaming blocks they finish well inside the launch, while a decode
// batch's one-block layout (about 6 us) outlasts its few-microsecond launch.
// Nothing waits on another stream or an event.
//   dispatch launch: the whole layout in one block (N <= 256, when the
//                    launch moves under 4 MiB), or the count phase, one
//                    block per 256 tokens;
//   combine launch:  the second phase (finish_lean, one block per 256
//                    tokens), which reads the histogram from memory so its
//                    LDS stays small; or, for N <= 256 beside a dispatch of
//                    4 MiB or more, the whole layout in one block; the
//                    launch's LDS is set to hold the combine blocks at four
//                    per CU.
// Kernel boundaries order the phases: the count phase's histogram and ranks
// are complete before the combine launch starts, the final slots before the
// next dispatch.
#include "gather.hpp"
#include "route.hpp"
#include "scatter.hpp"
#include "sources.hpp"

namespace epk {

namespace {

constexpr int kBlock = 256;
constexpr int kWPB = kBlock / kWave;
// LDS a layout phase may add to every block of the launch.
constexpr size_t kOverlapMaxLds = 24 * 1024;
// Every block of the combine launch takes at least this much LDS, so that a
// CU holds four 256-thread blocks (16 waves) rather than five: a fifth of the
// CU's LDS (160 KiB on MI355X, read from the device once) plus 1 KiB.  The
// gather runs best at 16 waves per CU (measured on MI355X, per step:
// DeepSeek-V3 360.5 us against 363.6 at 20 waves, group-limited non-expand
// 195.2 against 196.9, Qwen3 57.6 either way and 58.3 at 12 waves).
size_t combine_occupancy_lds()
{
    static const size_t lds = [] {
        int dev = 0, per_cu = 0, per_block = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            per_cu <= 0)
            return (size_t)0;   // unknown: leave the occupancy alone
        const size_t v = (size_t)per_cu / 5 + 1024;
        return v <= (size_t)per_block ? v : (size_t)0;
    }();
    return lds;
}
// Dispatch bytes from which a small batch's layout is split over the two
// launches rather than run by one block.
constexpr int64_t kOverlapSplitMinBytes = 4 << 20;

// Occupancy asked of the dispatch launch that also lays out the next batch:
// the layout code's scalar registers would otherwise hold it at 7 waves per
// SIMD, below the plain dispatch's 8.  Shapes whose scatter already needs
// more than 64 vector registers (channel scales over 8+ vectors per lane)
// are left to the compiler.
constexpr int dl_waves(bool channel, int vpl) { return (channel && vpl >= 8) ? 1 : 8; }

// Dispatch launches of at most this many streaming blocks (decode batches)
// are resident at once whatever the occupancy, so their layout blocks need
// not fit the 64 registers above: they take the routing phase's faster form
// (batched table reads) and the launch is left to the compiler.  Measured on
// MI355X, as a graph: decode 128 x 7168 FP8 12.8 -> 12.3 us per step, tiny
// 9.2 -> 8.8 us; the Qwen3 shape (1024 blocks) is faster held to 64.
constexpr int kSmallDispatchBlocks = 512;

// Layout work of the dispatch launch's first blocks.
constexpr int kModeCount = 0, kModeFused = 1, kModeTwin = 2;

// lblocks layout blocks come first: the one-block layout (kModeFused), the
// count phase of la (kModeCount), or (kModeTwin, non-expand) the count
// phases of la in blocks [0, lblocks/2) and of lb in the rest; then, with
// stacked sources, sblocks blocks of the per-source histogram.
template <int QUANT, bool CHANNEL, int VPL, bool ROW_WAIT, int LK, bool SMALL>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(SMALL ? 1 : dl_waves(CHANNEL, VPL))))
void k_dispatch_layout(DispatchArgs da, int NV, int NC, LayoutArgs la, LayoutArgs lb,
                       SourceArgs sa, int lblocks, int mode, int sblocks)
{
    extern __shared__ __align__(16) unsigned char smem[];
    if ((int)blockIdx.x >= lblocks && (int)blockIdx.x < lblocks + sblocks) {
        const int i = blockIdx.x - lblocks, chunks = sources::hist_chunks(sa);
        sources::hist_body<LK>(sa, i % chunks, i / chunks, reinterpret_cast<int32_t*>(smem));
        return;
    }
    if ((int)blockIdx.x < lblocks) {
        if (mode == kModeFused) {
            route::fused_body<LK, kWPB, !SMALL>(la, smem);
        } else if (mode == kModeTwin) {
            const int C = lblocks / 2;
            if ((int)blockIdx.x < C) route::count_body<LK, !SMALL>(la, blockIdx.x, smem);
            else route::count_body<LK, !SMALL>(lb, blockIdx.x - C, smem);
        } else {
            route::count_body<LK, !SMALL>(la, blockIdx.x, smem);
        }
        return;
    }
    scatter::dispatch_wave<QUANT, CHANNEL, VPL, 8, ROW_WAIT, kWPB>(da, NV, NC,
                                                                 blockIdx.x - lblocks - sblocks);
}

// C: the count blocks of the layout; lblocks = ceil(C / (BLOCK/256)) finish
// blocks come first -- twice as many with twin (non-expand): those of la,
// then those of lb -- then, with stacked sources, sblocks blocks of the
// per-source scan.
// fused: the one block in front is the whole one-block layout of la
// (lblocks = 1, C unused) instead of finish blocks.
template <int KMAX, int VPL, int YQ, bool YCH, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_combine_layout(CombineArgs ca, int NV, int NC,
                                                          LayoutArgs la, LayoutArgs lb,
                                                          SourceArgs sa, int lblocks, int C,
                                                          int twin, int sblocks, int fused)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int all = twin ? 2 * lblocks : lblocks;
    if ((int)blockIdx.x < all) {
        if (fused) route::fused_body<KMAX, BLOCK / kWave>(la, smem);
        else if ((int)blockIdx.x < lblocks) route::finish_lean<KMAX, BLOCK>(la, C, blockIdx.x, smem);
        else route::finish_lean<KMAX, BLOCK>(lb, C, blockIdx.x - lblocks, smem);
        return;
    }
    if ((int)blockIdx.x < all + sblocks) {
        if (BLOCK == sources::kScanBlock) sources::scan_body(sa, blockIdx.x - all);
        return;
    }
    gather::combine_wave<KMAX, VPL, YQ, YCH, BLOCK / kWave>(ca, NV, NC,
                                                          blockIdx.x - all - sblocks);
}

template <int QUANT, bool CHANNEL, int VPL, bool ROW_WAIT, int LK>
hipError_t launch_dl(const DispatchArgs& da, int NV, const LayoutArgs& la, const LayoutArgs& lb,
                     const SourceArgs& sa, const OverlapPlan& p, hipStream_t s, LaunchEvents ev)
{
    const int NC = (NV + kWave * VPL - 1) / (kWave * VPL);
    const int64_t items = (da.t_end - da.t_begin) * NC;
    const int dblocks = items > 0 ? (int)((items + kWPB - 1) / kWPB) : 0;
    const int blocks = p.dispatch_blocks + p.src_dispatch_blocks + dblocks;
    if (blocks == 0) return hipSuccess;
    const int mode = p.fused ? kModeFused : p.twin ? kModeTwin : kModeCount;
    if (dblocks <= kSmallDispatchBlocks)
        launch_k(k_dispatch_layout<QUANT, CHANNEL, VPL, ROW_WAIT, LK, true>, dim3(blocks),
                 dim3(kBlock), p.dispatch_lds, s, ev.start, ev.stop, da, NV, NC, la, lb, sa,
                 p.dispatch_blocks, mode, p.src_dispatch_blocks);
    else
        launch_k(k_dispatch_layout<QUANT, CHANNEL, VPL, ROW_WAIT, LK, false>, dim3(blocks),
                 dim3(kBlock), p.dispatch_lds, s, ev.start, ev.stop, da, NV, NC, la, lb, sa,
                 p.dispatch_blocks, mode, p.src_dispatch_blocks);
    return hipGetLastError();
}

template <int KMAX, int VPL, int YQ, bool YCH>
hipError_t launch_cl_v(const CombineArgs& ca, const LayoutArgs& la, const LayoutArgs& lb,
                       const SourceArgs& sa, const OverlapPlan& p, hipStream_t s, LaunchEvents ev)
{
    const int NV = ca.H / 8;
    const int NC = (NV + kWave * VPL - 1) / (kWave * VPL);
    const int64_t items = (ca.t_end - ca.t_begin) * NC;
    const int C = p.combine_blocks;   // count blocks whose finish phase runs here
    auto go = [&](auto block) {
        constexpr int B = decltype(block)::value, WPB = B / kWave, G = B / kLayoutBlock;
        const int lblocks = p.fused_combine ? 1 : (C + G - 1) / G;
        const int all = p.twin ? 2 * lblocks : lblocks;
        const int sblocks = p.src_combine_blocks;
        const int cblocks = items > 0 ? (int)((items + WPB - 1) / WPB) : 0;
        if (all + sblocks + cblocks == 0) return hipSuccess;
        size_t lds = p.fused_combine ? p.combine_lds : C > 0 ? route::finish_lean_lds_bytes(la, B) : 0;
        if (p.twin && route::finish_lean_lds_bytes(lb, B) > lds)
            lds = route::finish_lean_lds_bytes(lb, B);
        if (lds < combine_occupancy_lds()) lds = combine_occupancy_lds();
        launch_k(k_combine_layout<KMAX, VPL, YQ, YCH, B>, dim3(all + sblocks + cblocks), dim3(B),
                 lds, s, ev.start, ev.stop, ca, NV, NC, la, lb, sa, lblocks, C, p.twin ? 1 : 0,
                 sblocks, p.fused_combine ? 1 : 0);
        return hipGetLastError();
    };
    // 256-thread blocks: at the combine's 5 waves per SIMD a CU holds five
    // 4-wave blocks but only two 8-wave ones (measured on MI355X, Qwen3
    // shape: 57.4 us per step with 256, 58.5 with 512-thread blocks)
    return go(std::integral_constant<int, 256>{});
}

// Two vectors per lane.  (One vector per lane for decode batches, as the
// plain combine takes, made the launch slower: measured on MI355X, decode
// 128 x 7168 as a graph, 12.8 -> 14.1 us per step; twice the waves slow the
// finish block, which is the launch's critical path.)
template <int KMAX, int YQ, bool YCH>
hipError_t launch_cl(const CombineArgs& ca, const LayoutArgs& la, const LayoutArgs& lb,
                     const SourceArgs& sa, const OverlapPlan& p, hipStream_t s, LaunchEvents ev)
{
    return launch_cl_v<KMAX, 2, YQ, YCH>(ca, la, lb, sa, p, s, ev);
}

template <int LK>
hipError_t launch_dl_k(const DispatchArgs& da, const LayoutArgs& la, const LayoutArgs& lb,
                       const SourceArgs& sa, const OverlapPlan& p, hipStream_t s, LaunchEvents ev)
{
    auto launch = [&](auto q, auto ch, auto vpl, auto rw, int NV) {
        return launch_dl<decltype(q)::value, decltype(ch)::value, decltype(vpl)::value,
                         decltype(rw)::value, LK>(da, NV, la, lb, sa, p, s, ev);
    };
    return dispatch_shape(da, launch);
}

template <int KMAX>
hipError_t launch_cl_k(const CombineArgs& ca, const LayoutArgs& la, const LayoutArgs& lb,
                       const SourceArgs& sa, const OverlapPlan& p, hipStream_t s, LaunchEvents ev)
{
    const bool ych = ca.ygroup == ca.H && ca.H != 128;
    switch (ca.yquant) {
        case 0: return launch_cl<KMAX, 0, false>(ca, la, lb, sa, p, s, ev);
        case 1: return ych ? launch_cl<KMAX, 1, true>(ca, la, lb, sa, p, s, ev)
                           : launch_cl<KMAX, 1, false>(ca, la, lb, sa, p, s, ev);
        default: return ych ? launch_cl<KMAX, 2, true>(ca, la, lb, sa, p, s, ev)
                            : launch_cl<KMAX, 2, false>(ca, la, lb, sa, p, s, ev);
    }
}

}  // namespace

OverlapPlan plan_overlap(const LayoutArgs& la, int64_t dispatch_bytes)
{
    OverlapPlan p;
    if (la.K > 8) return p;   // the layout's registers would cut the streaming blocks' occupancy
    const size_t fused = route::fused_lds_bytes(la, kWPB);
    const size_t count = route::route_lds_bytes(kWPB, la.E, la.R, la.nodes);
    const size_t finish = route::finish_lean_lds_bytes(la, kBlock);
    const int C = (int)((la.num_tokens + kLayoutBlock - 1) / kLayoutBlock);
    const bool split = C > 0 && count <= kOverlapMaxLds && finish <= kOverlapMaxLds;
    // A batch of <= 256 tokens is laid out by one block: in the dispatch
    // launch when that launch moves under 4 MiB (measured on MI355X, a
    // 128 x 256 batch: 9.0 us per step, against 10.4 split over the two
    // launches), else in the combine launch, where the CUs are not saturated
    // by stores (decode shape 128 x 7168 FP8 as a graph: 11.9 us per step,
    // the same as split into count and finish over the two launches, where
    // each phase outlasts its launch's streaming blocks by about 1 us, and
    // 12.5 with the block in the dispatch launch).
    if (la.num_tokens <= kLayoutBlock && fused <= kOverlapMaxLds) {
        p.ok = true;
        if (dispatch_bytes < kOverlapSplitMinBytes || !split) {
            p.fused = true;
            p.dispatch_blocks = 1;
            p.dispatch_lds = fused;
        } else {
            p.fused_combine = true;
            p.combine_lds = fused;
        }
        return p;
    }
    if (!split) return p;   // LDS too large, or an empty batch whose one block does not fit
    p.ok = true;
    p.dispatch_blocks = C;
    p.combine_blocks = C;
    p.dispatch_lds = count;
    p.combine_lds = finish;
    return p;
}

// Non-expand: the count and finish phases of both levels, C blocks each.
// The expert level only counts (its slots are not the receive rows); the
// rank level takes its routing straight from the expert routing and leaves
// the distinct-token totals to the expert level.
OverlapPlan plan_overlap_twin(const LayoutArgs& la, const LayoutArgs& lb)
{
    OverlapPlan p;
    if (la.K > 8) return p;
    const int C = (int)((la.num_tokens + kLayoutBlock - 1) / kLayoutBlock);
    if (C == 0) return p;
    const size_t ca = route::route_lds_bytes(kWPB, la.E, la.R, la.nodes);
    const size_t cb = route::route_lds_bytes(kWPB, lb.E, lb.R, lb.nodes);
    const size_t fa = route::finish_lean_lds_bytes(la, kBlock);
    const size_t fb = route::finish_lean_lds_bytes(lb, kBlock);
    const size_t count = ca > cb ? ca : cb, finish = fa > fb ? fa : fb;
    if (count > kOverlapMaxLds || finish > kOverlapMaxLds) return p;
    p.ok = true;
    p.twin = true;
    p.dispatch_blocks = 2 * C;
    p.combine_blocks = C;
    p.dispatch_lds = count;
    p.combine_lds = finish;
    return p;
}

// One instantiation for every K <= 8 (entries past K are masked), which
// keeps the number of merged kernels down.
// Stacked sources: the layout's own plan, plus the per-source histogram
// blocks in the dispatch launch and the per-source scan blocks in the
// combine launch (the source arrays are then complete after the combine).
OverlapPlan plan_overlap_sources(const LayoutArgs& la, const SourceArgs& sa,
                                 int64_t dispatch_bytes)
{
    OverlapPlan p = plan_overlap(la, dispatch_bytes);
    if (!p.ok) return p;
    const size_t hist = sources::hist_lds_bytes(sa);
    if (hist > kOverlapMaxLds) return OverlapPlan{};
    if (hist > p.dispatch_lds) p.dispatch_lds = hist;
    p.src_dispatch_blocks = sources::hist_chunks(sa) * sa.P;
    p.src_combine_blocks = sources::scan_blocks(sa);
    return p;
}

hipError_t launch_dispatch_layout(const DispatchArgs& da, const LayoutArgs& la,
                                  const LayoutArgs& lb, const SourceArgs& sa,
                                  const OverlapPlan& p, hipStream_t s, LaunchEvents ev)
{
    return launch_dl_k<8>(da, la, lb, sa, p, s, ev);
}

hipError_t launch_combine_layout(const CombineArgs& ca, const LayoutArgs& la, const LayoutArgs& lb,
                                 const SourceArgs& sa, const OverlapPlan& p, hipStream_t s,
                                 LaunchEvents ev)
{
    return launch_cl_k<8>(ca, la, lb, sa, p, s, ev);
}

}  // namespace epk
