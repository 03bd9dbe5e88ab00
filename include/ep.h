/*
 * ep.h -- C ABI of libep_amd.so: the MoE expert-parallel token shuffle on one
 * MI355X (gfx950).  Four stages, each a HIP kernel path:
 *   routing layout  -> slot assignment  -> dispatch (+quant) -> combine.
 * Destination EP ranks are partitions of one receive buffer in HBM.
 *
 * Sources (web pages), cited by title and section:
 *   [P3] "DeepEP V1 vs V2 深度对比分析" (backyes.github.io): §2.1 the
 *        get_dispatch_layout -> dispatch -> combine call sequence and the
 *        layout outputs; §2.2 one dispatch call with a reusable handle;
 *        §3.1 the EPHandle fields; §3.2 cached dispatch (handle reuse, no CPU
 *        sync); §8.4 deterministic receive order.
 *   [P2] sgl-kernel-npu "A2_DEEPEP.md": the dispatch/combine API table; the
 *        HCCL_BUFFSIZE note (receive bound; num_local_experts =
 *        num_experts / ep_world_size); "Ant moving home" long-sequence
 *        rounds; int8 prefill quantisation; MOE_EXPERT_TOKEN_NUMS_TYPE
 *        (per-expert counts or prefix sums).
 *   [P5] Aliyun "DeepEP 通信库使用指南（v2.1）" §1.3.1: int8 quant_size,
 *        group mode (128) or channel mode (= hidden).
 *   [P4] lmdeploy PR #4783 "Integrate DeepEPv2": its status-check macro turns
 *        a failed call into an error text carrying the source file and line.
 *
 * Conventions for every call:
 *   - Pointers named d_* are device pointers (HBM of the current HIP device),
 *     h_* are host pointers.  The caller owns all memory; the library never
 *     allocates device memory.  Device buffers are contiguous row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous unless stated otherwise.
 *   - A handle is used by one stream at a time.
 *   - EP_ERR_STATE: the handle has no layout yet, or its layout is half done
 *     (ep_dispatch_overlap) and waits for ep_combine_overlap.
 *   - Errors are returned as ep_status; ep_last_error_message() gives a
 *     "file:line reason" text for the calling thread.  Invalid arguments are
 *     rejected on the host before any HIP call.  Conditions only the device
 *     can see (an expert id outside [-1, num_experts), a receive row beyond
 *     the capacity passed to dispatch, a slot beyond the rows passed to
 *     combine) set a sticky flag word in the handle's workspace -- the
 *     offending entry is skipped, never written out of bounds -- and are
 *     reported by ep_check_error().
 */
#ifndef EP_AMD_EP_H
#define EP_AMD_EP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,   /* bad configuration, pointer, size or range      */
    EP_ERR_WORKSPACE = 2,     /* workspace missing, misaligned or too small     */
    EP_ERR_CAPACITY = 3,      /* receive rows exceed the capacity passed in     */
    EP_ERR_DEVICE_INDEX = 4,  /* device saw an expert id or slot out of range   */
    EP_ERR_HIP = 5,           /* a HIP runtime call failed                      */
    EP_ERR_STATE = 6          /* handle has no layout yet, or it is half done   */
} ep_status;

/* Dispatch-side quantisation ([P5] §1.3.1; [P2] int8 prefill option; FP8
 * storage type float8_e4m3fn per [P3] §7.4). */
enum {
    EP_QUANT_NONE = 0,      /* recv_x is bf16, a bit copy of x                  */
    EP_QUANT_FP8_E4M3 = 1,  /* recv_x is OCP E4M3FN bytes, one scale per group  */
    EP_QUANT_INT8 = 2,      /* recv_x is int8, one scale per group              */
    EP_QUANT_MXFP4 = 3      /* [P5] §1.3.3 / OCP MX v1.0: recv_x holds two E2M1
                               codes per byte (element 2i in the low nibble),
                               one E8M0 scale byte per 32 elements              */
};

/* Scale format of EP_QUANT_FP8_E4M3 / EP_QUANT_INT8 ([P5] §1.3.1 API flags
 * round_scale and use_ue8m0; the pages name them, the readings are ours). */
enum {
    EP_SCALE_FP32 = 0,      /* fp32 amax / qmax                                */
    EP_SCALE_POW2 = 1,      /* round_scale: the smallest power of two >= that  */
    EP_SCALE_UE8M0 = 2      /* use_ue8m0: that power of two as one E8M0 byte
                               (2^(b-127)); recv_scales is then uint8          */
};

/* Flag bits reported by ep_check_error(). */
enum {
    EP_FLAG_BAD_EXPERT_ID = 1u,  /* topk_idx entry outside [-1, num_experts)   */
    EP_FLAG_RECV_CAPACITY = 2u,  /* dispatch: slot >= recv_capacity_rows       */
    EP_FLAG_Y_ROWS = 4u          /* combine: slot >= y_rows                    */
};

/* Largest hidden size: rows of up to 32 MiB of bf16 keep every byte offset
 * inside a row well within 32 bits. */
#define EP_MAX_HIDDEN (1 << 24)

typedef struct ep_config {
    int32_t hidden;            /* H: elements per token row, multiple of 8, at
                                  most EP_MAX_HIDDEN                              */
    int32_t num_topk;          /* K: experts per token, 1..16                    */
    int32_t num_experts;       /* E: 1..1024, multiple of num_ranks              */
    int32_t num_ranks;         /* R: simulated EP ranks, 1..1024; rank r owns
                                  experts [r*E/R, (r+1)*E/R)                     */
    int32_t ranks_per_node;    /* >0: also count distinct tokens per node of
                                  this many ranks (num_tokens_per_rdma_rank)     */
    int32_t expert_alignment;  /* A >= 1: each expert segment is padded to a
                                  multiple of A rows ([P3] §3.1)                 */
    int32_t quant;             /* EP_QUANT_*                                     */
    int32_t quant_group;       /* elements per scale: 128 or hidden (FP8, int8),
                                  32 (MXFP4)                                     */
    int32_t counts_as_prefix;  /* host list: 0 = per-expert aligned counts,
                                  1 = inclusive prefix restarting per rank
                                  ([P2] MOE_EXPERT_TOKEN_NUMS_TYPE)              */
    int32_t expert_capacity;   /* 0: packed layout (aligned segments placed by
                                  prefix sums).  >0: fixed-capacity layout, the
                                  low-latency buffer shape of [P3] §6.3: expert
                                  e owns rows [e*cap, (e+1)*cap) whatever its
                                  count; pairs past cap are dropped (slot -1)
                                  and flagged EP_FLAG_RECV_CAPACITY.  Needs
                                  expert_alignment == 1.  The host list then
                                  holds the filled rows min(count, cap).       */
    int32_t num_sources;       /* P: 0 or 1 = one source rank.  P > 1: the batch
                                  stacks P simulated source ranks, source p
                                  owning tokens [p*N/P, (p+1)*N/P) (N must be a
                                  multiple of P; P <= 1024).  Receive rows then
                                  follow (source, token, k) order, and the
                                  handle also holds the per-source arrays of
                                  ep_handle_view ([P3] §3.1
                                  psum_num_recv_tokens_per_scaleup_rank).      */
    int32_t scale_mode;        /* EP_SCALE_* for FP8 / int8 dispatch scales and
                                  ep_quantize_rows (there UE8M0 = POW2, stored
                                  fp32)                                          */
    int32_t combine_quant;     /* EP_QUANT_NONE: ep_combine reads bf16 y.
                                  EP_QUANT_FP8_E4M3 / EP_QUANT_INT8: y holds
                                  codes with fp32 scales ([P5] combine int8/fp8
                                  from v2.1)                                     */
    int32_t combine_group;     /* elements per y scale: 128 or hidden           */
    int32_t non_expand;        /* 0: one receive row per (token, k) ([P3] §3.1
                                  do_expand).  1: one row per (token, rank
                                  holding one of its experts), the V1 normal
                                  dispatch of [P3] §2.1: rank r's rows are
                                  [psum_rank[r], psum_rank[r+1]) in token
                                  order; slot_idx[t,k] is the row of the
                                  token's first entry on that rank, -1 for
                                  later entries on the same rank; src_meta =
                                  (t, that k).  psum_expert, num_unaligned and
                                  the host list stay per expert (aligned by
                                  expert_alignment); S is the row count.  Needs
                                  expert_capacity == 0.                          */
} ep_config;

typedef struct ep_handle ep_handle;

/* Device arrays of a handle ([P3] §3.1 EPHandle), as ep_handle_view fills
 * them. */
typedef struct ep_handle_view_s {
    const int32_t* psum_expert;    /* [E+1] exclusive prefix of aligned counts   */
    const int32_t* psum_rank;      /* [R+1] psum_expert at each rank's first
                                      expert: rank r's partition of the receive
                                      buffer is rows [psum_rank[r], psum_rank[r+1]) */
    const int32_t* num_unaligned;  /* [E] raw per-expert pair counts             */
    const int32_t* slot_idx;       /* [num_tokens, K] receive row of (t,k); -1 masked */
    const int32_t* src_meta;       /* [max_slots, 2] (t,k) of each receive row;
                                      (-1,-1) on padding rows; rows >= S stale   */
    const int32_t* topk_idx;       /* [num_tokens, K] clone of the routing (ids
                                      outside [-1,E) stored as -1)               */
    int64_t num_tokens;            /* N of the last ep_get_layout                */
    int64_t max_tokens;            /* capacity the handle was created with       */
    int64_t max_slots;             /* receive rows that can ever be needed:
                                      max_tokens*K + E*(A-1), or E*capacity      */
    int64_t num_recv_slots;        /* S if known on the host (do_cpu_sync), else -1 */
    int64_t num_sources;           /* P (1 for a single source)                  */
    const int32_t* psum_source_rank;   /* [R, P+1] (P > 1, else NULL): for
                                      receiving rank r, tokens received from the
                                      sources before p, a token counted once per
                                      rank it has an expert on; [r][P] equals
                                      num_tokens_per_rank[r]                      */
    const int32_t* expert_source_base; /* [P, E] (P > 1, else NULL): pairs of
                                      expert e from the sources before p; source
                                      p's rows of e start at psum_expert[e] + this */
} ep_handle_view_t;

/* Bytes of device workspace a handle needs for up to max_tokens tokens: the
 * EPHandle arrays of [P3] §3.1 (prefix sums, the topk clone, slot indices,
 * source metadata for ep_recv_capacity rows) plus the layout's block
 * histograms, accumulators and flag word.  Sizing memory up front from the
 * shape is the buffer rule of [P2]'s HCCL_BUFFSIZE note.
 * Returns EP_ERR_INVALID_ARG for an invalid configuration. */
ep_status ep_workspace_size(const ep_config* cfg, int64_t max_tokens, int64_t* bytes);

/* Receive rows a dispatch of num_tokens tokens can need in the worst case
 * ([P2] HCCL_BUFFSIZE note: the receive buffer is sized from the token
 * count, ranks, local experts and top-k; here every pair valid and every
 * expert fully padded): num_tokens*K + E*(A-1), or
 * E*expert_capacity in the fixed-capacity layout, or num_tokens*min(K, R)
 * with non_expand.
 * Sizing recv_x / y with this many rows never triggers EP_ERR_CAPACITY. */
ep_status ep_recv_capacity(const ep_config* cfg, int64_t num_tokens, int64_t* rows);

/* Creates a handle, the routing state of [P3] §3.1 EPHandle that dispatch
 * returns and combine reuses, over a caller-owned workspace (d_workspace, 256-byte
 * aligned, at least ep_workspace_size bytes; it must stay alive and unused by
 * anything else while the handle lives).  Clears the handle's flag word with
 * a kernel on `stream`.  The handle (host memory) is freed by ep_handle_free. */
ep_status ep_handle_init(const ep_config* cfg, int64_t max_tokens, void* d_workspace,
                         int64_t workspace_bytes, void* stream, ep_handle** out);

/* Workspace limit of ep_handle_init_static (4 MiB: the largest workload
 * here, 32768 tokens with top-6 over 64 experts, needs about 3.1 MiB). */
#define EP_STATIC_SCRATCH_BYTES (4ll << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): a
 * handle without a workspace argument.  Its workspace is a static device
 * array of EP_STATIC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; the call allocates nothing, on the device or the
 * host, and launches on `stream` the same clearing kernels as
 * ep_handle_init (so it may be captured).
 *   - There is one such handle per device: every call on a device returns
 *     the same handle, set up again for cfg and max_tokens (the layout it
 *     held is discarded, and views taken from it then show the new one).
 *     Calls that use it from several streams or threads at once on one GPU
 *     race; so do two overlapped batches, which need two handles.
 *   - EP_ERR_WORKSPACE, with the sizes in the message, if
 *     ep_workspace_size(cfg, max_tokens) exceeds EP_STATIC_SCRATCH_BYTES.
 *   - ep_handle_free on it does nothing.
 * Every other call takes it like a handle from ep_handle_init, with the
 * same results. */
ep_status ep_handle_init_static(const ep_config* cfg, int64_t max_tokens, void* stream,
                                ep_handle** out);

/* Frees the host-side handle ([P3] §3.1 EPHandle); never touches the
 * workspace.  NULL is a no-op. */
void ep_handle_free(ep_handle* h);

/* a1 + a2: routing layout and slot assignment ([P3] §2.1, §3.1, §8.4).
 *   d_topk_idx: int32 [num_tokens, K]; -1 = masked entry; 0 <= num_tokens <=
 *   max_tokens, a multiple of num_sources when that is above 1.  Outputs
 *   (each may be NULL to skip it):
 *     d_num_tokens_per_rank     int32 [R]  distinct tokens with an expert on r
 *     d_num_tokens_per_rdma_rank int32 [ceil(R/ranks_per_node)] distinct tokens
 *                                per node (needs ranks_per_node > 0)
 *     d_num_tokens_per_expert   int32 [E]  (t,k) pairs routed to e
 *     d_is_token_in_rank        uint8 [num_tokens, R] 0/1
 *   The handle receives psum_expert, psum_rank, num_unaligned, slot_idx,
 *   src_meta and the topk clone (and, with several sources, the per-source
 *   arrays).  Slot order inside an expert segment is (token, k) ascending,
 *   padding rows last: one deterministic result.
 *   do_cpu_sync != 0: waits for the stream and writes, when non-NULL,
 *     h_num_recv_tokens_per_expert [E] (aligned counts, or per-rank inclusive
 *     prefix if counts_as_prefix) and *h_num_recv_slots = S. */
ep_status ep_get_layout(ep_handle* h, const int32_t* d_topk_idx, int64_t num_tokens,
                        int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                        int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                        int do_cpu_sync, int32_t* h_num_recv_tokens_per_expert,
                        int64_t* h_num_recv_slots, void* stream);

/* a3: dispatch ([P3] §2.1/§2.2 expand form: one receive row per (t,k);
 * [P2] "Ant moving home" rounds = token ranges over one handle).
 *   d_x: bf16 [num_tokens, H] (the full batch; row t at d_x + t*H).
 *   Tokens [token_begin, token_end) are sent: for each (t,k) with a slot,
 *   row slot of d_recv_x receives token t.  Padding rows are not written.
 *   d_recv_x: [recv_capacity_rows, H] of bf16 (EP_QUANT_NONE), E4M3FN bytes
 *     or int8, or [recv_capacity_rows, H/2] bytes of E2M1 pairs (MXFP4);
 *     d_recv_scales: [recv_capacity_rows, H/quant_group] of fp32, or of E8M0
 *     bytes (EP_SCALE_UE8M0, MXFP4); NULL iff quant == EP_QUANT_NONE.
 *     FP8 / int8: scale = max(amax, 1e-4) / (448 or 127) (rounded up to a
 *     power of two unless EP_SCALE_FP32), code = x / scale rounded to
 *     nearest-even (E4M3FN saturating, int8 clamped to +-127).  MXFP4: per 32
 *     elements e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 when
 *     amax is 0), scale byte e + 127, codes E2M1(x * 2^-e) nearest-even,
 *     saturating at 6.  The quantised formats expect finite x: a row or
 *     group holding an infinity or NaN gets unspecified codes and scale.
 *   Reusing a handle across calls is cached dispatch ([P3] §3.2).
 *   EP_ERR_CAPACITY if S is known on the host and exceeds the capacity;
 *   otherwise rows beyond it are skipped and flagged on the device. */
ep_status ep_dispatch(const ep_handle* h, const void* d_x, int64_t token_begin, int64_t token_end,
                      void* d_recv_x, void* d_recv_scales, int64_t recv_capacity_rows,
                      void* stream);

/* a1 + a2 + a3 in one call: the unified dispatch of [P3] §2.2, which takes
 * the routing and returns the received rows together with the handle, with
 * no host synchronisation (the decode-step form; [P3] §6 low-latency mode).
 *   Same result as ep_get_layout(h, d_topk_idx, num_tokens, <the four
 *   outputs>, do_cpu_sync = 0, ...) followed by ep_dispatch(h, d_x, 0,
 *   num_tokens, d_recv_x, d_recv_scales, recv_capacity_rows): every argument
 *   has the meaning, layout and checks given there, and the handle is left
 *   in the same state (num_recv_slots unknown on the host).
 *   For num_tokens <= 256, num_topk <= 8 and one source (when the routing of
 *   the whole batch fits one workgroup's LDS) this is a single kernel launch;
 *   otherwise it launches the layout kernels and then the dispatch kernel.
 *   Receive rows beyond recv_capacity_rows are skipped and flagged on the
 *   device (ep_check_error); size recv_x with ep_recv_capacity to avoid it. */
ep_status ep_layout_dispatch(ep_handle* h, const int32_t* d_topk_idx, int64_t num_tokens,
                             int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                             int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                             const void* d_x, void* d_recv_x, void* d_recv_scales,
                             int64_t recv_capacity_rows, void* stream);

/* Non-expand only: the routing of each received row ([P3] §2.1
 * recv_topk_idx / recv_topk_weights), for tokens [token_begin, token_end):
 * row s of (t, rank r) gets, for every k, the local expert id idx[t,k] -
 * r*nle and the weight d_topk_weights[t,k] where expert idx[t,k] is on r,
 * else -1 and 0.  d_recv_topk_idx int32 [recv_capacity_rows, K] and
 * d_recv_topk_weights fp32 [recv_capacity_rows, K] may each be NULL (the
 * weights output needs d_topk_weights fp32 [num_tokens, K]).  Rows beyond
 * the capacity are skipped and flagged. */
ep_status ep_dispatch_topk(const ep_handle* h, const float* d_topk_weights, int64_t token_begin,
                           int64_t token_end, int32_t* d_recv_topk_idx, float* d_recv_topk_weights,
                           int64_t recv_capacity_rows, void* stream);

/* a4: combine ([P2] API table: the paired inverse of dispatch).
 *   d_y: bf16 [y_rows, H] expert outputs in receive-row order, or with
 *   combine_quant set their E4M3FN / int8 codes [y_rows, H] and d_y_scales
 *   fp32 [y_rows, H/combine_group] (element = code * scale; NULL iff
 *   combine_quant == EP_QUANT_NONE);
 *   d_topk_weights: fp32 [num_tokens, K], or NULL for weights of 1 (the
 *   non-expand combine, whose rank rows already carry the weights);
 *   d_out: bf16 [num_tokens, H].
 *   For t in [token_begin, token_end): out[t] = bf16_rne( sum over k with a
 *   slot, k ascending, of w[t,k] * y[slot] ), accumulated in fp32 with fused
 *   multiply-add.  Masked entries contribute nothing; an all-masked row is
 *   +0.  Slots >= y_rows are skipped and flagged. */
ep_status ep_combine(const ep_handle* h, const void* d_y, const float* d_y_scales, int64_t y_rows,
                     const float* d_topk_weights, int64_t token_begin, int64_t token_end,
                     void* d_out, void* stream);

/* Double-batch overlap on one stream ([P3] §5.2 overlaps one micro-batch's
 * communication with another's computation): the next batch's layout runs
 * inside the current batch's dispatch and combine launches, so its latency
 * hides under their HBM-bound work and nothing waits on another stream.
 *
 * ep_dispatch_overlap: ep_dispatch(h, d_x, token_begin, token_end, d_recv_x,
 *   d_recv_scales, recv_capacity_rows) and, when h_next is non-NULL, the
 *   start of ep_get_layout(h_next, d_topk_next, num_tokens_next, <the four
 *   outputs>, do_cpu_sync = 0): every argument has the meaning, layout and
 *   checks given there.  h_next must differ from h and have the same
 *   configuration.  For num_tokens_next <= 256 with a dispatch that moves
 *   under 4 MiB (one source, expand form) the layout completes in this
 *   launch; otherwise it completes in the next ep_combine_overlap(...,
 *   h_next) call,
 *   and until then h_next may be used only there (other calls return
 *   EP_ERR_STATE; ep_get_layout, ep_layout_dispatch or another
 *   ep_dispatch_overlap naming it as h_next start over, discarding the
 *   counted part).
 *   Configurations whose layout cannot share the launches (num_topk > 8,
 *   non_expand with stacked sources, a routing LDS above 24 KiB) lay h_next
 *   out with the ordinary kernels after the dispatch.
 * ep_combine_overlap: ep_combine(h, ...) and, when h_next is waiting, the
 *   rest of its layout.  With h_next NULL or not waiting it is ep_combine.
 * Kernel events armed on h (ep_set_kernel_events) span the call's launches. */
ep_status ep_dispatch_overlap(const ep_handle* h, const void* d_x, int64_t token_begin,
                              int64_t token_end, void* d_recv_x, void* d_recv_scales,
                              int64_t recv_capacity_rows, ep_handle* h_next,
                              const int32_t* d_topk_next, int64_t num_tokens_next,
                              int32_t* d_num_tokens_per_rank, int32_t* d_num_tokens_per_rdma_rank,
                              int32_t* d_num_tokens_per_expert, uint8_t* d_is_token_in_rank,
                              void* stream);
/* The combine half of the double-batch overlap ([P3] §5.2): ep_combine of h
 * and the finish of h_next's layout, as described above. */
ep_status ep_combine_overlap(const ep_handle* h, const void* d_y, const float* d_y_scales,
                             int64_t y_rows, const float* d_topk_weights, int64_t token_begin,
                             int64_t token_end, void* d_out, ep_handle* h_next, void* stream);

/* Quantises bf16 rows d_x [rows, H] one row at a time into the form
 * ep_combine reads with combine_quant (the sending side of a quantised
 * combine, [P5] v2.1): d_codes [rows, H] E4M3FN / int8 codes, d_scales fp32
 * [rows, H/combine_group], the arithmetic of ep_dispatch's FP8 / int8 mode
 * (scale_mode POW2 or UE8M0: power-of-two scales, stored fp32).
 * EP_ERR_INVALID_ARG if combine_quant is EP_QUANT_NONE. */
ep_status ep_quantize_rows(const ep_config* cfg, const void* d_x, int64_t rows, void* d_codes,
                           float* d_scales, void* stream);

/* Profiling (the per-stage timing behind the bandwidth figures of [P3] §4.3,
 * measured on one GPU): the next ep_get_layout, ep_dispatch or ep_combine call on h
 * records start_event when its first kernel starts and stop_event when its
 * last kernel ends (timestamps of the kernel launches themselves, taken with
 * hipExtLaunchKernelGGL, so no marker is queued between kernels); the events
 * are then released from the handle.  Both are caller-created hipEvent_t
 * (either may be NULL).  Not thread-safe with calls on the same handle. */
ep_status ep_set_kernel_events(ep_handle* h, void* start_event, void* stop_event);

/* Device pointers and sizes held by a handle: the EPHandle fields of [P3]
 * §3.1 (psum_num_recv_tokens_per_expert = psum_expert,
 * num_unaligned_recv_tokens_per_expert = num_unaligned, dst_buffer_slot_idx =
 * slot_idx, recv_src_metadata = src_meta, the topk_idx clone,
 * psum_num_recv_tokens_per_scaleup_rank = psum_source_rank).  The pointers
 * stay valid while the handle lives; their contents change with the next
 * layout on the handle. */
ep_status ep_handle_view(const ep_handle* h, ep_handle_view_t* view);

/* Another name for ep_handle_view (same arguments and result). */
ep_status ep_handle_get_view(const ep_handle* h, ep_handle_view_t* view);

/* Reports what only the device could see ([P4]'s convention: a failure is
 * returned with a "file:line reason" text rather than lost).
 * Waits for `stream`, reads and clears the handle's flag word.  *flags (if
 * non-NULL) receives the EP_FLAG_* bits.  Returns EP_ERR_DEVICE_INDEX for a
 * bad expert id or combine slot, EP_ERR_CAPACITY for a dispatch capacity
 * overflow, EP_OK if no flag was set. */
ep_status ep_check_error(ep_handle* h, void* stream, uint32_t* flags);

/* Name of a status code ("EP_OK", "EP_ERR_CAPACITY", ...; "EP_ERR_UNKNOWN"
 * for a value outside ep_status): the status half of [P4]'s error text. */
const char* ep_status_str(ep_status s);

/* Text of the last error raised on the calling thread ("" if none), in the
 * "file:line reason" form of [P4]'s status checks, e.g.
 * "api.cpp:123 num_topk=17 outside [1,16]".  Owned by the library; valid
 * until the thread's next failing call. */
const char* ep_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif
