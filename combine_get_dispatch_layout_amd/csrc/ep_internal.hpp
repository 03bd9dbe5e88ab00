// Internal interface between the C-ABI host runtime (api.cpp) and the HIP
// kernels (layout.hip, dispatch.hip, fused.hip, sources.hip, nonexpand.hip,
// combine.hip, overlap.hip).
// gfx950 only.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epk {

constexpr int kWave = 64;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxRanks = 1024;
constexpr int kMaxSources = 1024;
// Tokens per layout block: 4 waves, one token per lane.
constexpr int kLayoutBlock = 256;
// Largest row, in 16-byte vectors, that one wave can hold for a whole-row
// (channel) quantisation scale: 64 lanes x 16 vectors = 8192 bf16.
constexpr int kMaxVecPerLane = 16;
// Largest batch whose layout + dispatch run as one launch (every block
// counts the whole batch's routing in LDS).
constexpr int kRouteDispatchMaxTokens = 256;

// Most copies of the distinct-token accumulators: a layout of many count
// blocks spreads their atomics over several copies (LayoutArgs::acc_copies).
constexpr int kAccCopies = 8;

constexpr uint32_t kFlagBadId = 1u;
constexpr uint32_t kFlagCapacity = 2u;
constexpr uint32_t kFlagYRows = 4u;

// Control words at the start of the workspace.
enum CtrlWord { kCtrlFlags = 0, kCtrlNumSlots = 1, kCtrlWords = 64 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct LayoutArgs {
    const int32_t* topk;        // [N,K] caller's routing
    int64_t num_tokens;         // N
    int K, E, R, nle, ranks_per_node, nodes, A, counts_as_prefix;
    int cap;                    // >0: fixed-capacity layout, rows [e*cap, (e+1)*cap)
    // n / nle and n / ranks_per_node as __umulhi(n, magic) (magic 0 = divide
    // by 1); exact for n < 2^22, see div_magic()
    uint32_t nle_magic, rpn_magic;
    // handle workspace
    uint32_t* ctrl;
    int32_t* topk_clone;        // [N,K]
    int32_t* slot_idx;          // [N,K]
    int32_t* src_meta;          // [max_slots,2]
    int32_t* hist;              // [C,E]  block histograms -> exclusive bases
    int32_t* rank_acc;          // [kAccCopies][acc_stride]: distinct-token accumulators
                                // per rank (first R words of a copy), zero between calls
    int32_t* node_acc;          // rank_acc + R: the per-node ones, likewise
    int acc_stride;             // R + nodes
    int acc_copies;             // copies in use: count block b adds into b % acc_copies
    int32_t* psum_expert;       // [E+1]
    int32_t* psum_rank;         // [R+1]
    int32_t* num_unaligned;     // [E]
    int32_t* recv_list;         // [E]
    // caller outputs (nullable)
    int32_t* out_per_rank;
    int32_t* out_per_node;
    int32_t* out_per_expert;
    uint8_t* out_in_rank;
    bool in_rank_words;         // is_token_in_rank rows may be written as u32
    // [N,K] rows move as 16-byte vectors: row_vec for the workspace arrays
    // (K % 4 == 0), topk_vec for the caller's routing (also 16-byte aligned)
    bool row_vec, topk_vec;
    // Non-expand in two concurrent layouts (one per level):
    //   derive_src:     non-null: the ids are the ranks of this [N,K] expert
    //                   routing (expert / nle via derive_magic, ids outside
    //                   [0, derive_E) and repeats of a rank in a row masked)
    //   counts_only:    no in-block ranks, slots, source metadata, padding
    //                   rows, psum_rank or slot count (the other level's)
    //   no_rank_counts: no distinct-token accumulation or flush
    const int32_t* derive_src;
    uint32_t derive_magic;
    int derive_E;
    bool counts_only, no_rank_counts;
};

struct DispatchArgs {
    const void* x;              // bf16 [N,H]
    int64_t t_begin, t_end;
    int H, K;
    const int32_t* slot_idx;    // [N,K]; unused when identity
    void* recv;                 // [cap,H] bf16 / e4m3fn / int8, [cap,H/2] MXFP4 codes
    void* scales;               // [cap,G] fp32, or E8M0 bytes (scale_mode 2, MXFP4)
    int64_t capacity;
    int quant, group;
    int scale_mode;             // 0 fp32 amax/qmax, 1 power of two, 2 power of two as E8M0
    bool identity;              // row t goes to receive row t (K = 1): row quantisation
    uint32_t* flags;
};

// Non-expand per-row routing (recv_topk_idx / recv_topk_weights).
struct RecvTopkArgs {
    const int32_t* topk;        // [N,K] the handle's clone
    const int32_t* slot_idx;    // [N,K] non-expand rows (-1: none)
    const float* weights;       // [N,K] (may be NULL when recv_topk_weights is)
    int64_t t_begin, t_end;
    int K, nle;
    int64_t capacity;
    int32_t* recv_topk_idx;     // [capacity,K] (nullable)
    float* recv_topk_weights;   // [capacity,K] (nullable)
    uint32_t* flags;
};

// Per-source counts of a batch of P stacked source ranks.
struct SourceArgs {
    const int32_t* topk;        // [P*Ns, K]
    int64_t tokens_per_source;  // Ns
    int K, E, R, nle, P;
    int32_t* acc_expert;        // [P][E] accumulators, zero between calls
    int32_t* acc_rank;          // [P][R] likewise
    int32_t* expert_source_base;  // [P][E]
    int32_t* psum_source_rank;    // [R][P+1]
};

struct CombineArgs {
    const void* y;              // bf16 [y_rows,H], or E4M3FN / int8 codes (yquant)
    const float* y_scales;      // [y_rows, H/ygroup] when yquant != 0
    int yquant, ygroup;         // 0 bf16, 1 E4M3FN, 2 int8; elements per scale
    int64_t y_rows;
    const float* weights;       // [N,K]; NULL: every weight is 1
    const int32_t* slot_idx;    // [N,K]
    int64_t t_begin, t_end;
    int H, K;
    void* out;                  // bf16 [N,H]
    uint32_t* flags;
};

// ceil(2^32 / d) for 2 <= d <= 2^16, 0 for d == 1.  floor(n / d) ==
// __umulhi(n, magic) whenever n * (magic * d - 2^32) < 2^32, i.e. for all
// n < 2^32 / d >= 2^16 here (ids and ranks are below 1024).
inline uint32_t div_magic(uint32_t d)
{
    return d <= 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + d - 1) / d);
}

// Optional timestamps of a call's first kernel start and last kernel end.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Launches `kernel`; with events it goes through hipExtLaunchKernelGGL so the
// events take the kernel's own start / end timestamps.
template <typename K, typename... Args>
inline void launch_k(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t start,
                     hipEvent_t stop, Args... args)
{
    if (start != nullptr || stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, start, stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

hipError_t launch_clear(uint32_t* words, int n, hipStream_t s);
hipError_t launch_layout(const LayoutArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_combine(const CombineArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_sources(const SourceArgs& a, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_recv_topk(const RecvTopkArgs& a, hipStream_t s, LaunchEvents ev = {});
// The next batch's layout inside the current batch's dispatch and combine
// launches (overlap.hip): which phase goes where, and the LDS each launch
// needs for it.
struct OverlapPlan {
    bool ok = false;          // false: lay the next batch out on its own
    bool fused = false;       // the whole layout in one block of the dispatch launch
    bool fused_combine = false;   // the whole layout in one block of the combine launch
    bool twin = false;        // non-expand: two layouts (expert level, rank level), C blocks each
    int dispatch_blocks = 0;  // layout blocks in front of the dispatch blocks
    int combine_blocks = 0;   // count blocks whose finish phase the combine launch runs
    size_t dispatch_lds = 0;
    size_t combine_lds = 0;   // LDS of the finish phase
    int src_dispatch_blocks = 0;   // stacked sources: per-source histogram blocks
    int src_combine_blocks = 0;    // ... and per-source scan blocks
};
// dispatch_bytes: what the dispatch launch that takes the layout's first
// phase moves (decides whether a small batch is laid out in one block).
OverlapPlan plan_overlap(const LayoutArgs& la, int64_t dispatch_bytes);
// Non-expand: the expert-level layout `la` (counts only) and the rank-level
// layout `lb` (rank ids derived from la's routing) side by side.
OverlapPlan plan_overlap_twin(const LayoutArgs& la, const LayoutArgs& lb);
// Stacked sources: plan_overlap plus the per-source counts (sa).
OverlapPlan plan_overlap_sources(const LayoutArgs& la, const SourceArgs& sa,
                                 int64_t dispatch_bytes);
hipError_t launch_dispatch_layout(const DispatchArgs& da, const LayoutArgs& la,
                                  const LayoutArgs& lb, const SourceArgs& sa,
                                  const OverlapPlan& p, hipStream_t s, LaunchEvents ev = {});
hipError_t launch_combine_layout(const CombineArgs& ca, const LayoutArgs& la, const LayoutArgs& lb,
                                 const SourceArgs& sa, const OverlapPlan& p, hipStream_t s,
                                 LaunchEvents ev = {});
// Layout + dispatch of the whole batch in one launch (small batches).
bool route_dispatch_fits(const LayoutArgs& la);
hipError_t launch_route_dispatch(const LayoutArgs& la, const DispatchArgs& da, hipStream_t s,
                                 LaunchEvents ev = {});

}  // namespace epk
