// C-ABI host runtime of libep_amd.so: validation, workspace carving, handle
// state and kernel launches.  The declarations and their contracts are in
// include/ep.h.  Validation happens on the host before any HIP call; the
// library never allocates device memory (the workspace is caller-owned).
#include "ep.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "ep_internal.hpp"

// Workspace of the handles made by ep_handle_init_static, for callers that
// cannot allocate device memory.  Each GPU the library is loaded on holds
// its own copy until the process ends.  Host code never uses this name as a
// device address: the address comes from hipGetSymbolAddress, once per
// device (static_scratch_ptr below).
constexpr int64_t kStaticScratchBytes = EP_STATIC_SCRATCH_BYTES;
constexpr int kMaxHidden = EP_MAX_HIDDEN;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local char g_msg[512] = "";

ep_status fail(ep_status st, const char* file, int line, const char* fmt, ...)
{
    char body[400];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(body, sizeof(body), fmt, ap);
    va_end(ap);
    const char* base = strrchr(file, '/');
    snprintf(g_msg, sizeof(g_msg), "%s:%d %s", base ? base + 1 : file, line, body);
    return st;
}

#define EP_FAIL(st, ...) fail((st), __FILE__, __LINE__, __VA_ARGS__)
#define EP_HIP(call)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) return EP_FAIL(EP_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Carve {
    int64_t ctrl, psum_expert, psum_rank, num_unaligned, recv_list, topk, slot, meta, hist,
        acc, src_acc, src_base, src_psum, rank_ids, ne_scratch, ne_hist, total;
};

int num_sources(const ep_config& c) { return c.num_sources > 1 ? c.num_sources : 1; }

int num_nodes(const ep_config& c)
{
    return c.ranks_per_node > 0 ? (c.num_ranks + c.ranks_per_node - 1) / c.ranks_per_node : 0;
}

// Rows of the expert-level layout (the source metadata array holds them).
int64_t expert_rows_for(const ep_config& c, int64_t tokens)
{
    if (c.expert_capacity > 0) return (int64_t)c.num_experts * c.expert_capacity;
    return tokens * c.num_topk + (int64_t)c.num_experts * (c.expert_alignment - 1);
}

// Receive rows a dispatch can need: one per (token, k), plus padding, or
// with non_expand one per (token, rank).
int64_t max_slots_for(const ep_config& c, int64_t tokens)
{
    if (c.non_expand) return tokens * (c.num_topk < c.num_ranks ? c.num_topk : c.num_ranks);
    return expert_rows_for(c, tokens);
}

ep_status check_config(const ep_config* c)
{
    if (!c) return EP_FAIL(EP_ERR_INVALID_ARG, "config is NULL");
    if (c->hidden <= 0 || c->hidden % 8 != 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "hidden=%d must be a positive multiple of 8", c->hidden);
    // row bytes (2 * hidden) and per-row byte offsets stay far inside 32 bits
    if (c->hidden > kMaxHidden)
        return EP_FAIL(EP_ERR_INVALID_ARG, "hidden=%d above %d", c->hidden, kMaxHidden);
    if (c->num_topk < 1 || c->num_topk > epk::kMaxTopk)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_topk=%d outside [1,%d]", c->num_topk, epk::kMaxTopk);
    if (c->num_experts < 1 || c->num_experts > epk::kMaxExperts)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_experts=%d outside [1,%d]", c->num_experts,
                       epk::kMaxExperts);
    if (c->num_ranks < 1 || c->num_ranks > epk::kMaxRanks || c->num_experts % c->num_ranks != 0)
        return EP_FAIL(EP_ERR_INVALID_ARG,
                       "num_ranks=%d must be in [1,%d] and divide num_experts=%d", c->num_ranks,
                       epk::kMaxRanks, c->num_experts);
    if (c->ranks_per_node < 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "ranks_per_node=%d is negative", c->ranks_per_node);
    if (c->expert_alignment < 1)
        return EP_FAIL(EP_ERR_INVALID_ARG, "expert_alignment=%d < 1", c->expert_alignment);
    if (c->expert_capacity < 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "expert_capacity=%d < 0", c->expert_capacity);
    if (c->expert_capacity > 0 && c->expert_alignment != 1)
        return EP_FAIL(EP_ERR_INVALID_ARG, "expert_capacity needs expert_alignment == 1 (got %d)",
                       c->expert_alignment);
    if ((int64_t)c->num_experts * c->expert_capacity >= (int64_t)1 << 31)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_experts * expert_capacity exceeds 2^31 - 1");
    if (c->num_sources < 0 || c->num_sources > epk::kMaxSources)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_sources=%d outside [0,%d]", c->num_sources,
                       epk::kMaxSources);
    if (c->quant < EP_QUANT_NONE || c->quant > EP_QUANT_MXFP4)
        return EP_FAIL(EP_ERR_INVALID_ARG, "quant=%d unknown", c->quant);
    if (c->scale_mode < EP_SCALE_FP32 || c->scale_mode > EP_SCALE_UE8M0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "scale_mode=%d unknown", c->scale_mode);
    if (c->quant == EP_QUANT_MXFP4) {
        if (c->quant_group != 32 || c->hidden % 32 != 0)
            return EP_FAIL(EP_ERR_INVALID_ARG,
                           "MXFP4 needs quant_group 32 and hidden %% 32 == 0 (got %d, %d)",
                           c->quant_group, c->hidden);
    } else if (c->quant != EP_QUANT_NONE) {
        if (c->quant_group == 128) {
            if (c->hidden % 128 != 0)
                return EP_FAIL(EP_ERR_INVALID_ARG, "quant_group 128 needs hidden %% 128 == 0 (hidden=%d)",
                               c->hidden);
        } else if (c->quant_group == c->hidden) {
            if (c->hidden > epk::kWave * epk::kMaxVecPerLane * 8)
                return EP_FAIL(EP_ERR_INVALID_ARG, "channel quantisation supports hidden <= %d (hidden=%d)",
                               epk::kWave * epk::kMaxVecPerLane * 8, c->hidden);
        } else {
            return EP_FAIL(EP_ERR_INVALID_ARG, "quant_group=%d must be 128 or hidden=%d",
                           c->quant_group, c->hidden);
        }
    }
    if (c->non_expand != 0 && c->non_expand != 1)
        return EP_FAIL(EP_ERR_INVALID_ARG, "non_expand=%d must be 0 or 1", c->non_expand);
    if (c->non_expand && c->expert_capacity > 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "non_expand needs expert_capacity == 0");
    if (c->combine_quant != EP_QUANT_NONE && c->combine_quant != EP_QUANT_FP8_E4M3 &&
        c->combine_quant != EP_QUANT_INT8)
        return EP_FAIL(EP_ERR_INVALID_ARG, "combine_quant=%d must be none, FP8 or int8",
                       c->combine_quant);
    if (c->combine_quant != EP_QUANT_NONE &&
        !(c->combine_group == c->hidden || (c->combine_group == 128 && c->hidden % 128 == 0)))
        return EP_FAIL(EP_ERR_INVALID_ARG, "combine_group=%d must be hidden=%d, or 128 dividing it",
                       c->combine_group, c->hidden);
    return EP_OK;
}

ep_status carve(const ep_config& c, int64_t max_tokens, Carve* o)
{
    if (max_tokens < 0) return EP_FAIL(EP_ERR_INVALID_ARG, "max_tokens=%lld < 0", (long long)max_tokens);
    const int64_t slots = expert_rows_for(c, max_tokens);
    if (slots >= (int64_t)1 << 31 || max_tokens * c.num_topk >= (int64_t)1 << 31)
        return EP_FAIL(EP_ERR_INVALID_ARG, "max_tokens=%lld needs %lld receive rows (limit 2^31-1)",
                       (long long)max_tokens, (long long)slots);
    const int64_t C = (max_tokens + epk::kLayoutBlock - 1) / epk::kLayoutBlock;
    const int64_t Cc = C > 0 ? C : 1;
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = align_up(off + (bytes > 0 ? bytes : 4), kAlign);
        return at;
    };
    o->ctrl = take(4 * epk::kCtrlWords);
    o->psum_expert = take(4 * (int64_t)(c.num_experts + 1));
    o->psum_rank = take(4 * (int64_t)(c.num_ranks + 1));
    o->num_unaligned = take(4 * (int64_t)c.num_experts);
    o->recv_list = take(4 * (int64_t)c.num_experts);
    o->topk = take(4 * max_tokens * c.num_topk);
    // slack of kMaxTopk entries: kernels read a token's slots as one batch of
    // kMaxTopk words and ignore those past K
    o->slot = take(4 * (max_tokens * c.num_topk + epk::kMaxTopk));
    o->meta = take(8 * slots);
    o->hist = take(4 * Cc * c.num_experts);
    o->acc = take(4 * (int64_t)epk::kAccCopies * (c.num_ranks + num_nodes(c)));
    const int64_t P = num_sources(c);
    if (P > 1) {
        o->src_acc = take(4 * P * (c.num_experts + c.num_ranks));
        o->src_base = take(4 * P * c.num_experts);
        o->src_psum = take(4 * (int64_t)c.num_ranks * (P + 1));
    } else {
        o->src_acc = o->src_base = o->src_psum = -1;
    }
    if (c.non_expand) {
        o->rank_ids = take(4 * max_tokens * c.num_topk);
        o->ne_scratch = take(4 * (3 * (int64_t)c.num_ranks + 1));   // psum', counts', list'
        o->ne_hist = take(4 * Cc * c.num_ranks);   // the rank level's block histograms
    } else {
        o->rank_ids = o->ne_scratch = o->ne_hist = -1;
    }
    o->total = off;
    return EP_OK;
}

}  // namespace

struct ep_handle {
    ep_config cfg;
    int64_t max_tokens;
    int64_t max_slots;
    int nodes;
    unsigned char* ws;
    Carve cv;
    int64_t num_tokens;   // -1 before the first ep_get_layout
    int64_t host_slots;   // S known on the host, else -1
    // layout counted inside a dispatch launch, to be finished inside the
    // next ep_combine_overlap launch (see ep_dispatch_overlap)
    bool pending = false;
    bool is_static = false;   // ep_handle_init_static's per-device handle: never deleted
    epk::LayoutArgs pending_args, pending_args2;   // second: the rank level (non-expand)
    epk::SourceArgs pending_src;                   // stacked sources
    epk::OverlapPlan pending_plan;
    // events armed by ep_set_kernel_events for the next call
    mutable epk::LaunchEvents armed;

    epk::LaunchEvents take_events() const
    {
        epk::LaunchEvents e = armed;
        armed = epk::LaunchEvents{};
        return e;
    }

    template <typename T>
    T* at(int64_t off) const { return reinterpret_cast<T*>(ws + off); }
};

namespace {

// A layout counted inside a dispatch launch and not finished (the caller lays
// the handle out again instead of calling ep_combine_overlap) has added its
// distinct-token counts, and with stacked sources its per-source counts, to
// accumulators that only the finish phase reads and re-zeroes: clear them
// before the handle is laid out again.
hipError_t drop_pending(ep_handle* h, hipStream_t s)
{
    if (!h->pending) return hipSuccess;
    hipError_t e = epk::launch_clear(h->at<uint32_t>(h->cv.acc),
                                     epk::kAccCopies * (h->cfg.num_ranks + h->nodes), s);
    if (e == hipSuccess && h->cv.src_acc >= 0)
        e = epk::launch_clear(h->at<uint32_t>(h->cv.src_acc),
                              num_sources(h->cfg) * (h->cfg.num_experts + h->cfg.num_ranks), s);
    if (e == hipSuccess) h->pending = false;
    return e;
}

// Validates the layout arguments and fills the kernel arguments.
ep_status layout_args(ep_handle* h, const int32_t* d_topk_idx, int64_t num_tokens,
                      int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                      int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                      epk::LayoutArgs* out)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    if (num_tokens < 0 || num_tokens > h->max_tokens)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_tokens=%lld outside [0, max_tokens=%lld]",
                       (long long)num_tokens, (long long)h->max_tokens);
    if (num_tokens > 0 && !d_topk_idx) return EP_FAIL(EP_ERR_INVALID_ARG, "topk_idx is NULL");
    if (d_topk_idx && !aligned(d_topk_idx, 4))
        return EP_FAIL(EP_ERR_INVALID_ARG, "topk_idx is not 4-byte aligned");
    if (d_num_tokens_per_rdma_rank && h->nodes == 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_tokens_per_rdma_rank needs ranks_per_node > 0");
    const ep_config& c = h->cfg;
    if (num_tokens % num_sources(c) != 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "num_tokens=%lld is not a multiple of num_sources=%d",
                       (long long)num_tokens, num_sources(c));
    epk::LayoutArgs& a = *out;
    a.topk = d_topk_idx;
    a.num_tokens = num_tokens;
    a.K = c.num_topk;
    a.E = c.num_experts;
    a.R = c.num_ranks;
    a.nle = c.num_experts / c.num_ranks;
    a.ranks_per_node = c.ranks_per_node;
    a.nle_magic = epk::div_magic((uint32_t)a.nle);
    a.rpn_magic = epk::div_magic((uint32_t)(c.ranks_per_node > 0 ? c.ranks_per_node : 1));
    a.nodes = h->nodes;
    a.A = c.expert_alignment;
    a.counts_as_prefix = c.counts_as_prefix ? 1 : 0;
    a.cap = c.expert_capacity;
    a.ctrl = h->at<uint32_t>(h->cv.ctrl);
    a.topk_clone = h->at<int32_t>(h->cv.topk);
    a.slot_idx = h->at<int32_t>(h->cv.slot);
    a.src_meta = h->at<int32_t>(h->cv.meta);
    a.hist = h->at<int32_t>(h->cv.hist);
    a.rank_acc = h->at<int32_t>(h->cv.acc);
    a.node_acc = a.rank_acc + c.num_ranks;
    a.acc_stride = c.num_ranks + h->nodes;
    // one copy per 16 count blocks once there are 64 or more (below that the
    // atomics per address cost less than the spreading; measured on MI355X:
    // 128 blocks, 8 copies: the count kernel 8.1 -> 6.9 us)
    const int64_t C = (num_tokens + epk::kLayoutBlock - 1) / epk::kLayoutBlock;
    a.acc_copies = C >= 64 ? (int)(C / 16 < epk::kAccCopies ? C / 16 : epk::kAccCopies) : 1;
    a.psum_expert = h->at<int32_t>(h->cv.psum_expert);
    a.psum_rank = h->at<int32_t>(h->cv.psum_rank);
    a.num_unaligned = h->at<int32_t>(h->cv.num_unaligned);
    a.recv_list = h->at<int32_t>(h->cv.recv_list);
    a.out_per_rank = d_num_tokens_per_rank;
    a.out_per_node = d_num_tokens_per_rdma_rank;
    a.out_per_expert = d_num_tokens_per_expert;
    a.out_in_rank = d_is_token_in_rank;
    a.in_rank_words = (c.num_ranks % 4 == 0) && aligned(d_is_token_in_rank, 4);
    a.row_vec = c.num_topk % 4 == 0;
    a.topk_vec = a.row_vec && aligned(d_topk_idx, 16);
    a.derive_src = nullptr;
    a.derive_magic = 0u;
    a.derive_E = 0;
    a.counts_only = false;
    a.no_rank_counts = false;
    return EP_OK;
}

// Validates the dispatch arguments for tokens [token_begin, token_end) of a
// layout over num_tokens tokens and fills the kernel arguments.
ep_status dispatch_args(const ep_handle* h, int64_t num_tokens, const void* d_x,
                        int64_t token_begin, int64_t token_end, void* d_recv_x,
                        void* d_recv_scales, int64_t recv_capacity_rows, epk::DispatchArgs* out)
{
    if (token_begin < 0 || token_begin > token_end || token_end > num_tokens)
        return EP_FAIL(EP_ERR_INVALID_ARG, "token range [%lld,%lld) outside [0,%lld]",
                       (long long)token_begin, (long long)token_end, (long long)num_tokens);
    if (recv_capacity_rows < 0) return EP_FAIL(EP_ERR_INVALID_ARG, "recv_capacity_rows < 0");
    const ep_config& c = h->cfg;
    if (token_end > token_begin) {
        if (!d_x || !d_recv_x) return EP_FAIL(EP_ERR_INVALID_ARG, "x or recv_x is NULL");
        if (!aligned(d_x, 16) || !aligned(d_recv_x, 16))
            return EP_FAIL(EP_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
        const bool byte_scales = c.quant == EP_QUANT_MXFP4 || c.scale_mode == EP_SCALE_UE8M0;
        if (c.quant != EP_QUANT_NONE &&
            (!d_recv_scales || (!byte_scales && !aligned(d_recv_scales, 4))))
            return EP_FAIL(EP_ERR_INVALID_ARG, "quantised dispatch needs recv_scales%s",
                           byte_scales ? "" : " (4-byte aligned)");
    }
    if (c.quant == EP_QUANT_NONE && d_recv_scales)
        return EP_FAIL(EP_ERR_INVALID_ARG, "recv_scales must be NULL without quantisation");
    if (recv_capacity_rows >= (int64_t)1 << 31) recv_capacity_rows = ((int64_t)1 << 31) - 1;
    epk::DispatchArgs& a = *out;
    a.x = d_x;
    a.t_begin = token_begin;
    a.t_end = token_end;
    a.H = c.hidden;
    a.K = c.num_topk;
    a.slot_idx = h->at<int32_t>(h->cv.slot);
    a.recv = d_recv_x;
    a.scales = d_recv_scales;
    a.capacity = recv_capacity_rows;
    a.quant = c.quant;
    a.group = c.quant_group;
    a.scale_mode = c.scale_mode;
    a.identity = false;
    a.flags = h->at<uint32_t>(h->cv.ctrl) + epk::kCtrlFlags;
    return EP_OK;
}

// Layout kernels, preceded with several sources by the per-source counts;
// `ev` spans all of them.
// The per-source counts of a stacked-sources layout `a` (P > 1).
epk::SourceArgs source_args(const ep_handle* h, const epk::LayoutArgs& a)
{
    const int P = num_sources(h->cfg);
    epk::SourceArgs sa;
    sa.topk = a.topk;
    sa.tokens_per_source = a.num_tokens / P;
    sa.K = a.K;
    sa.E = a.E;
    sa.R = a.R;
    sa.nle = a.nle;
    sa.P = P;
    sa.acc_expert = h->at<int32_t>(h->cv.src_acc);
    sa.acc_rank = sa.acc_expert + (int64_t)P * a.E;
    sa.expert_source_base = h->at<int32_t>(h->cv.src_base);
    sa.psum_source_rank = h->at<int32_t>(h->cv.src_psum);
    return sa;
}

hipError_t launch_layout_all(const ep_handle* h, const epk::LayoutArgs& a, hipStream_t s,
                             epk::LaunchEvents ev)
{
    if (num_sources(h->cfg) == 1) return epk::launch_layout(a, s, ev);
    const epk::SourceArgs sa = source_args(h, a);
    hipError_t e = epk::launch_sources(sa, s, epk::LaunchEvents{ev.start, nullptr});
    if (e != hipSuccess) return e;
    return epk::launch_layout(a, s, epk::LaunchEvents{nullptr, ev.stop});
}

// Non-expand: the expert-level layout (counts, per-expert arrays, host list)
// followed by the layout of the derived rank-id routing, whose rows are the
// receive rows (one per token and rank); it writes slot_idx, src_meta, the
// row count and, through its per-"expert" prefix, psum_rank.
// The rank-level layout of a non-expand handle: the expand layout
// (alignment 1) of the derived routing whose entries are the ranks of the
// expert routing's entries, each rank once per row, over R one-expert ranks.
// Its slots are the receive rows; its per-"expert" prefix is psum_rank.  The
// routing is derived inline from the expert routing (the derived rows are
// kept in rank_ids, the level's clone).
epk::LayoutArgs rank_level_args(const ep_handle* h, const epk::LayoutArgs& a)
{
    epk::LayoutArgs b = a;
    int32_t* scratch = h->at<int32_t>(h->cv.ne_scratch);
    b.derive_src = a.topk;
    b.derive_magic = a.nle_magic;
    b.derive_E = a.E;
    b.topk_clone = h->at<int32_t>(h->cv.rank_ids);
    b.hist = h->at<int32_t>(h->cv.ne_hist);
    b.no_rank_counts = true;               // the expert level counts tokens per rank
    b.counts_only = false;
    b.E = a.R;
    b.nle = 1;
    b.nle_magic = 0;
    b.ranks_per_node = 0;
    b.rpn_magic = 0;
    b.nodes = 0;
    b.A = 1;
    b.counts_as_prefix = 0;
    b.cap = 0;
    b.psum_expert = a.psum_rank;           // the rank partitions of the receive rows
    b.psum_rank = scratch;                 // [R+1] (same values)
    b.num_unaligned = scratch + a.R + 1;   // [R]
    b.recv_list = scratch + 2 * a.R + 1;   // [R]
    b.out_per_rank = nullptr;
    b.out_per_node = nullptr;
    b.out_per_expert = nullptr;
    b.out_in_rank = nullptr;
    b.in_rank_words = false;
    return b;
}

hipError_t launch_layout_nonexpand(const ep_handle* h, const epk::LayoutArgs& a, hipStream_t s,
                                   epk::LaunchEvents ev)
{
    hipError_t e = launch_layout_all(h, a, s, epk::LaunchEvents{ev.start, nullptr});
    if (e != hipSuccess) return e;
    return epk::launch_layout(rank_level_args(h, a), s, epk::LaunchEvents{nullptr, ev.stop});
}

hipError_t launch_layout_any(const ep_handle* h, const epk::LayoutArgs& a, hipStream_t s,
                             epk::LaunchEvents ev)
{
    return h->cfg.non_expand ? launch_layout_nonexpand(h, a, s, ev)
                             : launch_layout_all(h, a, s, ev);
}

// Validates the combine arguments and fills the kernel arguments.
ep_status combine_args(const ep_handle* h, const void* d_y, const float* d_y_scales,
                       int64_t y_rows, const float* d_topk_weights, int64_t token_begin,
                       int64_t token_end, void* d_out, epk::CombineArgs* out)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    if (h->num_tokens < 0) return EP_FAIL(EP_ERR_STATE, "ep_get_layout has not run on this handle");
    if (h->pending) return EP_FAIL(EP_ERR_STATE, "the handle's layout is waiting for ep_combine_overlap");
    if (token_begin < 0 || token_begin > token_end || token_end > h->num_tokens)
        return EP_FAIL(EP_ERR_INVALID_ARG, "token range [%lld,%lld) outside [0,%lld]",
                       (long long)token_begin, (long long)token_end, (long long)h->num_tokens);
    if (y_rows < 0) return EP_FAIL(EP_ERR_INVALID_ARG, "y_rows < 0");
    if (token_end > token_begin) {
        if (!d_out || (y_rows > 0 && !d_y))
            return EP_FAIL(EP_ERR_INVALID_ARG, "y or out is NULL");
        if ((d_y && !aligned(d_y, 16)) || !aligned(d_out, 16) || !aligned(d_topk_weights, 4))
            return EP_FAIL(EP_ERR_INVALID_ARG,
                           "y and out must be 16-byte aligned, topk_weights 4-byte aligned");
    }
    const ep_config& c = h->cfg;
    if (c.combine_quant == EP_QUANT_NONE && d_y_scales)
        return EP_FAIL(EP_ERR_INVALID_ARG, "y_scales must be NULL without combine_quant");
    if (c.combine_quant != EP_QUANT_NONE && token_end > token_begin && y_rows > 0 &&
        (!d_y_scales || !aligned(d_y_scales, 4)))
        return EP_FAIL(EP_ERR_INVALID_ARG, "combine_quant needs 4-byte aligned y_scales");
    epk::CombineArgs& a = *out;
    a.y = d_y;
    a.y_scales = d_y_scales;
    a.yquant = c.combine_quant;
    a.ygroup = c.combine_group;
    a.y_rows = y_rows;
    a.weights = d_topk_weights;
    a.slot_idx = h->at<int32_t>(h->cv.slot);
    a.t_begin = token_begin;
    a.t_end = token_end;
    a.H = c.hidden;
    a.K = c.num_topk;
    a.out = d_out;
    a.flags = h->at<uint32_t>(h->cv.ctrl) + epk::kCtrlFlags;
    return EP_OK;
}

// The next batch's layout for the overlapped calls: the checks of
// ep_get_layout, and which phases can run inside the launches.
ep_status next_layout(const ep_handle* h, ep_handle* h_next, const int32_t* d_topk_next,
                      int64_t num_tokens_next, int32_t* d_per_rank, int32_t* d_per_rdma,
                      int32_t* d_per_expert, uint8_t* d_in_rank, int64_t dispatch_bytes,
                      epk::LayoutArgs* la, epk::LayoutArgs* lb, epk::SourceArgs* sa,
                      epk::OverlapPlan* plan)
{
    if (h_next == h) return EP_FAIL(EP_ERR_INVALID_ARG, "h_next must differ from h");
    if (memcmp(&h->cfg, &h_next->cfg, sizeof(ep_config)) != 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "h and h_next must have the same configuration");
    ep_status st = layout_args(h_next, d_topk_next, num_tokens_next, d_per_rank, d_per_rdma,
                               d_per_expert, d_in_rank, la);
    if (st != EP_OK) return st;
    const ep_config& c = h_next->cfg;
    *lb = *la;
    *sa = epk::SourceArgs{};
    if (num_sources(c) > 1) {
        // stacked sources: the per-source counts ride in the same launches
        if (c.non_expand) {
            *plan = epk::OverlapPlan{};
        } else {
            *sa = source_args(h_next, *la);
            *plan = epk::plan_overlap_sources(*la, *sa, dispatch_bytes);
        }
    } else if (c.non_expand) {
        // both levels side by side; the expert level only counts
        *lb = rank_level_args(h_next, *la);
        *plan = epk::plan_overlap_twin(*la, *lb);
        if (plan->ok) la->counts_only = true;
    } else {
        *plan = epk::plan_overlap(*la, dispatch_bytes);
    }
    return EP_OK;
}

// Per-device state of ep_handle_init_static: the device address of
// `scratch` (looked up once per device, with that device current) and the
// one handle whose workspace it is.
constexpr int kMaxStaticDevices = 64;
std::mutex g_static_mu;
unsigned char* g_static_ws[kMaxStaticDevices] = {};
ep_handle g_static_handles[kMaxStaticDevices];

ep_status static_scratch_ptr(int dev, unsigned char** ws)
{
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ws[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return EP_FAIL(EP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                           hipGetErrorString(e));
        g_static_ws[dev] = static_cast<unsigned char*>(p);
    }
    *ws = g_static_ws[dev];
    return EP_OK;
}

}  // namespace

extern "C" {

ep_status ep_workspace_size(const ep_config* cfg, int64_t max_tokens, int64_t* bytes)
{
    ep_status st = check_config(cfg);
    if (st != EP_OK) return st;
    if (!bytes) return EP_FAIL(EP_ERR_INVALID_ARG, "bytes is NULL");
    Carve cv;
    st = carve(*cfg, max_tokens, &cv);
    if (st != EP_OK) return st;
    *bytes = cv.total;
    return EP_OK;
}

ep_status ep_recv_capacity(const ep_config* cfg, int64_t num_tokens, int64_t* rows)
{
    ep_status st = check_config(cfg);
    if (st != EP_OK) return st;
    if (!rows) return EP_FAIL(EP_ERR_INVALID_ARG, "rows is NULL");
    if (num_tokens < 0) return EP_FAIL(EP_ERR_INVALID_ARG, "num_tokens < 0");
    *rows = max_slots_for(*cfg, num_tokens);
    return EP_OK;
}

ep_status ep_handle_init(const ep_config* cfg, int64_t max_tokens, void* d_workspace,
                         int64_t workspace_bytes, void* stream, ep_handle** out)
{
    ep_status st = check_config(cfg);
    if (st != EP_OK) return st;
    if (!out) return EP_FAIL(EP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    Carve cv;
    st = carve(*cfg, max_tokens, &cv);
    if (st != EP_OK) return st;
    if (!d_workspace) return EP_FAIL(EP_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(d_workspace, kAlign))
        return EP_FAIL(EP_ERR_WORKSPACE, "workspace is not %lld-byte aligned", (long long)kAlign);
    if (workspace_bytes < cv.total)
        return EP_FAIL(EP_ERR_WORKSPACE, "workspace has %lld bytes, needs %lld",
                       (long long)workspace_bytes, (long long)cv.total);
    ep_handle* h = new (std::nothrow) ep_handle();
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "out of host memory");
    h->cfg = *cfg;
    h->max_tokens = max_tokens;
    h->max_slots = max_slots_for(*cfg, max_tokens);
    h->nodes = num_nodes(*cfg);
    h->ws = static_cast<unsigned char*>(d_workspace);
    h->cv = cv;
    h->num_tokens = -1;
    h->host_slots = -1;
    hipError_t e = epk::launch_clear(h->at<uint32_t>(cv.ctrl), epk::kCtrlWords,
                                     static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = epk::launch_clear(h->at<uint32_t>(cv.acc), epk::kAccCopies * (cfg->num_ranks + h->nodes),
                              static_cast<hipStream_t>(stream));
    if (e == hipSuccess && cv.src_acc >= 0)
        e = epk::launch_clear(h->at<uint32_t>(cv.src_acc),
                              num_sources(*cfg) * (cfg->num_experts + cfg->num_ranks),
                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        delete h;
        return EP_FAIL(EP_ERR_HIP, "clearing the control words: %s", hipGetErrorString(e));
    }
    *out = h;
    return EP_OK;
}

void ep_handle_free(ep_handle* h)
{
    if (h && !h->is_static) delete h;
}

ep_status ep_handle_init_static(const ep_config* cfg, int64_t max_tokens, void* stream,
                                ep_handle** out)
{
    ep_status st = check_config(cfg);
    if (st != EP_OK) return st;
    if (!out) return EP_FAIL(EP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    Carve cv;
    st = carve(*cfg, max_tokens, &cv);
    if (st != EP_OK) return st;
    if (cv.total > kStaticScratchBytes)
        return EP_FAIL(EP_ERR_WORKSPACE,
                       "the handle needs %lld bytes of workspace; the static scratch holds %lld "
                       "(use ep_handle_init with a workspace)",
                       (long long)cv.total, (long long)kStaticScratchBytes);
    int dev = 0;
    EP_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxStaticDevices)
        return EP_FAIL(EP_ERR_INVALID_ARG, "device %d beyond the %d static handles", dev,
                       kMaxStaticDevices);
    unsigned char* ws = nullptr;
    st = static_scratch_ptr(dev, &ws);
    if (st != EP_OK) return st;
    ep_handle* h = &g_static_handles[dev];
    *h = ep_handle{};
    h->is_static = true;
    h->cfg = *cfg;
    h->max_tokens = max_tokens;
    h->max_slots = max_slots_for(*cfg, max_tokens);
    h->nodes = num_nodes(*cfg);
    h->ws = ws;
    h->cv = cv;
    h->num_tokens = -1;
    h->host_slots = -1;
    // the array keeps the last call's contents: clear what starts at zero
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = epk::launch_clear(h->at<uint32_t>(cv.ctrl), epk::kCtrlWords, s);
    if (e == hipSuccess)
        e = epk::launch_clear(h->at<uint32_t>(cv.acc), epk::kAccCopies * (cfg->num_ranks + h->nodes),
                              s);
    if (e == hipSuccess && cv.src_acc >= 0)
        e = epk::launch_clear(h->at<uint32_t>(cv.src_acc),
                              num_sources(*cfg) * (cfg->num_experts + cfg->num_ranks), s);
    if (e != hipSuccess) return EP_FAIL(EP_ERR_HIP, "clearing the control words: %s", hipGetErrorString(e));
    *out = h;
    return EP_OK;
}

ep_status ep_get_layout(ep_handle* h, const int32_t* d_topk_idx, int64_t num_tokens,
                        int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                        int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                        int do_cpu_sync, int32_t* h_num_recv_tokens_per_expert,
                        int64_t* h_num_recv_slots, void* stream)
{
    epk::LayoutArgs a;
    ep_status st = layout_args(h, d_topk_idx, num_tokens, d_num_tokens_per_rank,
                               d_num_tokens_per_rdma_rank, d_num_tokens_per_expert,
                               d_is_token_in_rank, &a);
    if (st != EP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    EP_HIP(drop_pending(h, s));
    EP_HIP(launch_layout_any(h, a, s, h->take_events()));
    h->num_tokens = num_tokens;
    h->host_slots = -1;
    h->pending = false;
    if (do_cpu_sync) {
        uint32_t S = 0;
        if (h_num_recv_tokens_per_expert)
            EP_HIP(hipMemcpyAsync(h_num_recv_tokens_per_expert, a.recv_list,
                                  sizeof(int32_t) * h->cfg.num_experts, hipMemcpyDeviceToHost, s));
        EP_HIP(hipMemcpyAsync(&S, a.ctrl + epk::kCtrlNumSlots, sizeof(uint32_t),
                              hipMemcpyDeviceToHost, s));
        EP_HIP(hipStreamSynchronize(s));
        h->host_slots = S;
        if (h_num_recv_slots) *h_num_recv_slots = S;
    }
    return EP_OK;
}

ep_status ep_dispatch(const ep_handle* h, const void* d_x, int64_t token_begin, int64_t token_end,
                      void* d_recv_x, void* d_recv_scales, int64_t recv_capacity_rows, void* stream)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    if (h->num_tokens < 0) return EP_FAIL(EP_ERR_STATE, "ep_get_layout has not run on this handle");
    if (h->pending) return EP_FAIL(EP_ERR_STATE, "the handle's layout is waiting for ep_combine_overlap");
    epk::DispatchArgs a;
    ep_status st = dispatch_args(h, h->num_tokens, d_x, token_begin, token_end, d_recv_x,
                                 d_recv_scales, recv_capacity_rows, &a);
    if (st != EP_OK) return st;
    if (h->host_slots >= 0 && h->host_slots > recv_capacity_rows)
        return EP_FAIL(EP_ERR_CAPACITY, "layout needs %lld receive rows, capacity is %lld",
                       (long long)h->host_slots, (long long)recv_capacity_rows);
    EP_HIP(epk::launch_dispatch(a, static_cast<hipStream_t>(stream), h->take_events()));
    return EP_OK;
}

ep_status ep_layout_dispatch(ep_handle* h, const int32_t* d_topk_idx, int64_t num_tokens,
                             int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                             int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                             const void* d_x, void* d_recv_x, void* d_recv_scales,
                             int64_t recv_capacity_rows, void* stream)
{
    epk::LayoutArgs la;
    ep_status st = layout_args(h, d_topk_idx, num_tokens, d_num_tokens_per_rank,
                               d_num_tokens_per_rdma_rank, d_num_tokens_per_expert,
                               d_is_token_in_rank, &la);
    if (st != EP_OK) return st;
    epk::DispatchArgs da;
    st = dispatch_args(h, num_tokens, d_x, 0, num_tokens, d_recv_x, d_recv_scales,
                       recv_capacity_rows, &da);
    if (st != EP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    EP_HIP(drop_pending(h, s));
    const epk::LaunchEvents ev = h->take_events();
    if (num_sources(h->cfg) == 1 && !h->cfg.non_expand && epk::route_dispatch_fits(la)) {
        EP_HIP(epk::launch_route_dispatch(la, da, s, ev));
    } else {
        EP_HIP(launch_layout_any(h, la, s, epk::LaunchEvents{ev.start, nullptr}));
        EP_HIP(epk::launch_dispatch(da, s, epk::LaunchEvents{nullptr, ev.stop}));
    }
    h->num_tokens = num_tokens;
    h->host_slots = -1;
    h->pending = false;
    return EP_OK;
}

ep_status ep_dispatch_topk(const ep_handle* h, const float* d_topk_weights, int64_t token_begin,
                           int64_t token_end, int32_t* d_recv_topk_idx, float* d_recv_topk_weights,
                           int64_t recv_capacity_rows, void* stream)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    if (!h->cfg.non_expand) return EP_FAIL(EP_ERR_INVALID_ARG, "ep_dispatch_topk needs non_expand");
    if (h->num_tokens < 0) return EP_FAIL(EP_ERR_STATE, "ep_get_layout has not run on this handle");
    if (h->pending) return EP_FAIL(EP_ERR_STATE, "the handle's layout is waiting for ep_combine_overlap");
    if (token_begin < 0 || token_begin > token_end || token_end > h->num_tokens)
        return EP_FAIL(EP_ERR_INVALID_ARG, "token range [%lld,%lld) outside [0,%lld]",
                       (long long)token_begin, (long long)token_end, (long long)h->num_tokens);
    if (recv_capacity_rows < 0) return EP_FAIL(EP_ERR_INVALID_ARG, "recv_capacity_rows < 0");
    if (d_recv_topk_weights && !d_topk_weights)
        return EP_FAIL(EP_ERR_INVALID_ARG, "recv_topk_weights needs topk_weights");
    if (!aligned(d_topk_weights, 4) || !aligned(d_recv_topk_idx, 4) ||
        !aligned(d_recv_topk_weights, 4))
        return EP_FAIL(EP_ERR_INVALID_ARG, "arrays must be 4-byte aligned");
    if (h->host_slots >= 0 && h->host_slots > recv_capacity_rows)
        return EP_FAIL(EP_ERR_CAPACITY, "layout needs %lld receive rows, capacity is %lld",
                       (long long)h->host_slots, (long long)recv_capacity_rows);
    epk::RecvTopkArgs a;
    a.topk = h->at<int32_t>(h->cv.topk);
    a.slot_idx = h->at<int32_t>(h->cv.slot);
    a.weights = d_topk_weights;
    a.t_begin = token_begin;
    a.t_end = token_end;
    a.K = h->cfg.num_topk;
    a.nle = h->cfg.num_experts / h->cfg.num_ranks;
    a.capacity = recv_capacity_rows;
    a.recv_topk_idx = d_recv_topk_idx;
    a.recv_topk_weights = d_recv_topk_weights;
    a.flags = h->at<uint32_t>(h->cv.ctrl) + epk::kCtrlFlags;
    EP_HIP(epk::launch_recv_topk(a, static_cast<hipStream_t>(stream), h->take_events()));
    return EP_OK;
}

ep_status ep_combine(const ep_handle* h, const void* d_y, const float* d_y_scales, int64_t y_rows,
                     const float* d_topk_weights, int64_t token_begin, int64_t token_end,
                     void* d_out, void* stream)
{
    epk::CombineArgs a;
    ep_status st = combine_args(h, d_y, d_y_scales, y_rows, d_topk_weights, token_begin, token_end,
                                d_out, &a);
    if (st != EP_OK) return st;
    EP_HIP(epk::launch_combine(a, static_cast<hipStream_t>(stream), h->take_events()));
    return EP_OK;
}

ep_status ep_dispatch_overlap(const ep_handle* h, const void* d_x, int64_t token_begin,
                              int64_t token_end, void* d_recv_x, void* d_recv_scales,
                              int64_t recv_capacity_rows, ep_handle* h_next,
                              const int32_t* d_topk_next, int64_t num_tokens_next,
                              int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                              int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                              void* stream)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    if (h->num_tokens < 0) return EP_FAIL(EP_ERR_STATE, "ep_get_layout has not run on this handle");
    if (h->pending) return EP_FAIL(EP_ERR_STATE, "the handle's layout is waiting for ep_combine_overlap");
    epk::DispatchArgs da;
    ep_status st = dispatch_args(h, h->num_tokens, d_x, token_begin, token_end, d_recv_x,
                                 d_recv_scales, recv_capacity_rows, &da);
    if (st != EP_OK) return st;
    if (h->host_slots >= 0 && h->host_slots > recv_capacity_rows)
        return EP_FAIL(EP_ERR_CAPACITY, "layout needs %lld receive rows, capacity is %lld",
                       (long long)h->host_slots, (long long)recv_capacity_rows);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!h_next) {
        EP_HIP(epk::launch_dispatch(da, s, h->take_events()));
        return EP_OK;
    }
    epk::LayoutArgs la, lb;
    epk::SourceArgs sa;
    epk::OverlapPlan plan;
    // bytes this dispatch writes: one row per pair (codes: one byte per element)
    const int64_t dispatch_bytes = (token_end - token_begin) * h->cfg.num_topk *
                                   h->cfg.hidden * (h->cfg.quant == EP_QUANT_NONE ? 2 : 1);
    st = next_layout(h, h_next, d_topk_next, num_tokens_next, d_num_tokens_per_rank,
                     d_num_tokens_per_rdma_rank, d_num_tokens_per_expert, d_is_token_in_rank,
                     dispatch_bytes, &la, &lb, &sa, &plan);
    if (st != EP_OK) return st;
    EP_HIP(drop_pending(h_next, s));
    const epk::LaunchEvents ev = h->take_events();
    if (plan.ok) {
        EP_HIP(epk::launch_dispatch_layout(da, la, lb, sa, plan, s, ev));
    } else {
        EP_HIP(epk::launch_dispatch(da, s, epk::LaunchEvents{ev.start, nullptr}));
        EP_HIP(launch_layout_any(h_next, la, s, epk::LaunchEvents{nullptr, ev.stop}));
    }
    h_next->num_tokens = num_tokens_next;
    h_next->host_slots = -1;
    // pending until the combine launch finishes the layout or the source counts
    h_next->pending = plan.ok && (!plan.fused || plan.src_combine_blocks > 0);
    h_next->pending_args = la;
    h_next->pending_args2 = lb;
    h_next->pending_src = sa;
    h_next->pending_plan = plan;
    return EP_OK;
}

ep_status ep_combine_overlap(const ep_handle* h, const void* d_y, const float* d_y_scales,
                             int64_t y_rows, const float* d_topk_weights, int64_t token_begin,
                             int64_t token_end, void* d_out, ep_handle* h_next, void* stream)
{
    epk::CombineArgs ca;
    ep_status st = combine_args(h, d_y, d_y_scales, y_rows, d_topk_weights, token_begin, token_end,
                                d_out, &ca);
    if (st != EP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!h_next || !h_next->pending) {
        EP_HIP(epk::launch_combine(ca, s, h->take_events()));
        return EP_OK;
    }
    if (h_next == h) return EP_FAIL(EP_ERR_INVALID_ARG, "h_next must differ from h");
    if (memcmp(&h->cfg, &h_next->cfg, sizeof(ep_config)) != 0)
        return EP_FAIL(EP_ERR_INVALID_ARG, "h and h_next must have the same configuration");
    EP_HIP(epk::launch_combine_layout(ca, h_next->pending_args, h_next->pending_args2,
                                      h_next->pending_src, h_next->pending_plan, s,
                                      h->take_events()));
    h_next->pending = false;
    return EP_OK;
}

ep_status ep_quantize_rows(const ep_config* cfg, const void* d_x, int64_t rows, void* d_codes,
                           float* d_scales, void* stream)
{
    ep_status st = check_config(cfg);
    if (st != EP_OK) return st;
    if (cfg->combine_quant == EP_QUANT_NONE)
        return EP_FAIL(EP_ERR_INVALID_ARG, "ep_quantize_rows needs combine_quant FP8 or int8");
    if (rows < 0 || rows >= (int64_t)1 << 31)
        return EP_FAIL(EP_ERR_INVALID_ARG, "rows=%lld outside [0, 2^31)", (long long)rows);
    if (cfg->combine_group == cfg->hidden && cfg->hidden != 128 &&
        cfg->hidden > epk::kWave * epk::kMaxVecPerLane * 8)
        return EP_FAIL(EP_ERR_INVALID_ARG, "row quantisation supports hidden <= %d (hidden=%d)",
                       epk::kWave * epk::kMaxVecPerLane * 8, cfg->hidden);
    if (rows == 0) return EP_OK;
    if (!d_x || !d_codes || !d_scales) return EP_FAIL(EP_ERR_INVALID_ARG, "x, codes or scales is NULL");
    if (!aligned(d_x, 16) || !aligned(d_codes, 16) || !aligned(d_scales, 4))
        return EP_FAIL(EP_ERR_INVALID_ARG,
                       "x and codes must be 16-byte aligned, scales 4-byte aligned");
    epk::DispatchArgs a;
    a.x = d_x;
    a.t_begin = 0;
    a.t_end = rows;
    a.H = cfg->hidden;
    a.K = 1;
    a.slot_idx = nullptr;
    a.recv = d_codes;
    a.scales = d_scales;
    a.capacity = rows;
    a.quant = cfg->combine_quant;
    a.group = cfg->combine_group;
    a.scale_mode = cfg->scale_mode == EP_SCALE_FP32 ? 0 : 1;   // fp32 storage
    a.identity = true;
    a.flags = nullptr;   // row t goes to row t < capacity: never flagged
    EP_HIP(epk::launch_dispatch(a, static_cast<hipStream_t>(stream)));
    return EP_OK;
}

ep_status ep_set_kernel_events(ep_handle* h, void* start_event, void* stop_event)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    h->armed.start = static_cast<hipEvent_t>(start_event);
    h->armed.stop = static_cast<hipEvent_t>(stop_event);
    return EP_OK;
}

ep_status ep_handle_view(const ep_handle* h, ep_handle_view_t* v)
{
    if (!h || !v) return EP_FAIL(EP_ERR_INVALID_ARG, "handle or view is NULL");
    v->psum_expert = h->at<int32_t>(h->cv.psum_expert);
    v->psum_rank = h->at<int32_t>(h->cv.psum_rank);
    v->num_unaligned = h->at<int32_t>(h->cv.num_unaligned);
    v->slot_idx = h->at<int32_t>(h->cv.slot);
    v->src_meta = h->at<int32_t>(h->cv.meta);
    v->topk_idx = h->at<int32_t>(h->cv.topk);
    v->num_tokens = h->num_tokens;
    v->max_tokens = h->max_tokens;
    v->max_slots = h->max_slots;
    v->num_recv_slots = h->host_slots;
    v->num_sources = num_sources(h->cfg);
    v->psum_source_rank = h->cv.src_psum >= 0 ? h->at<int32_t>(h->cv.src_psum) : nullptr;
    v->expert_source_base = h->cv.src_base >= 0 ? h->at<int32_t>(h->cv.src_base) : nullptr;
    return EP_OK;
}

ep_status ep_handle_get_view(const ep_handle* h, ep_handle_view_t* v) { return ep_handle_view(h, v); }

ep_status ep_check_error(ep_handle* h, void* stream, uint32_t* flags)
{
    if (!h) return EP_FAIL(EP_ERR_INVALID_ARG, "handle is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t f = 0;
    uint32_t* dflags = h->at<uint32_t>(h->cv.ctrl) + epk::kCtrlFlags;
    EP_HIP(hipMemcpyAsync(&f, dflags, sizeof(f), hipMemcpyDeviceToHost, s));
    EP_HIP(hipStreamSynchronize(s));
    if (f != 0) EP_HIP(epk::launch_clear(dflags, 1, s));
    if (flags) *flags = f;
    if (f & (epk::kFlagBadId | epk::kFlagYRows))
        return EP_FAIL(EP_ERR_DEVICE_INDEX, "device flags 0x%x: expert id or combine slot out of range",
                       f);
    if (f & epk::kFlagCapacity)
        return EP_FAIL(EP_ERR_CAPACITY, "device flags 0x%x: dispatch slot beyond capacity", f);
    return EP_OK;
}

const char* ep_status_str(ep_status s)
{
    // A C caller may pass any int; reading it as the enum would be undefined
    // for a value outside the enumerators, so its bits are read as an int.
    int v = 0;
    memcpy(&v, &s, sizeof(v) < sizeof(s) ? sizeof(v) : sizeof(s));
    switch (v) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
        case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE";
        case EP_ERR_CAPACITY: return "EP_ERR_CAPACITY";
        case EP_ERR_DEVICE_INDEX: return "EP_ERR_DEVICE_INDEX";
        case EP_ERR_HIP: return "EP_ERR_HIP";
        case EP_ERR_STATE: return "EP_ERR_STATE";
    }
    return "EP_ERR_UNKNOWN";
}

const char* ep_last_error_message(void) { return g_msg; }

}  // extern "C"
