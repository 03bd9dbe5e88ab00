/*
 * Plain CPU oracle for the MoE expert-parallel token shuffle (routing layout,
 * slot assignment, dispatch with optional quantisation, weighted combine).
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that tests, the smoke
 * check and the CPU-baseline leg of the benchmark can check the HIP library
 * against an independent, obviously-correct definition.  Nothing in the
 * product path links, loads or calls it, and it shares no code, header or
 * constant with the HIP library.
 *
 * Sources (web pages), cited by title and section:
 *   [P3] "DeepEP V1 vs V2 深度对比分析" (backyes.github.io):
 *        §2.1 (get_dispatch_layout outputs), §2.2 (unified dispatch),
 *        §3.1 (EPHandle fields), §3.2 (cached dispatch), §7.4 (FP8 storage
 *        type float8_e4m3fn), §8.4 (deterministic sort).
 *   [P2] sgl-kernel-npu "A2_DEEPEP.md": API table (dispatch/combine pair),
 *        the HCCL_BUFFSIZE note (non-layered receive bound,
 *        num_local_experts = num_experts / ep_world_size), the "Ant moving
 *        home" long-sequence rounds, the int8 prefill quantisation option and
 *        the MOE_EXPERT_TOKEN_NUMS_TYPE count/prefix option.
 *   [P5] Aliyun "DeepEP 通信库使用指南（v2.1）" §1.3.1 (int8 quant_size:
 *        group mode 128, channel mode = hidden; the round_scale, use_ue8m0
 *        flags; combine int8 / fp8), §1.3.3 (MXFP4, quant_size 32).
 *   OCP Microscaling Formats (MX) v1.0: the E2M1 element and E8M0 scale
 *        types and the block conversion MXFP4 uses.
 *
 * Where the pages are silent the oracle takes one stated reading; every
 * reading is listed with the function that takes it.
 *
 * Floating point: quantisation codes are decided in fp32 (the precision the
 * kernels decide them in); scales are fp32.  The combine is given twice: as
 * its plain definition (the weighted sum formed in fp64, rounded once to
 * bf16) and as the fp32 reduction the path states (k ascending, one fused
 * multiply-add per term, then bf16); the tests pin the second against
 * exact arithmetic and the first.
 *
 * Threads: the plain build (libep_oracle.so) is serial and is the parity
 * reference.  The same source built with OpenMP (libep_oracle_omp.so) runs
 * the per-token loops of dispatch and combine in parallel, with the same
 * results; it exists to time the oracle on a host's cores.
 *
 * Parity status: every function here is pinned by the CPU test suite
 * (closed forms, exhaustive format checks against torch's converters,
 * numpy library routines, brute force, exact rational sums, invariants).
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads the library runs its per-token loops on (1 in the plain build). */
int orc_num_threads(void);

/* ---- number formats (written from the format definitions) ---- */

/* fp32 -> bf16 bits, round to nearest, ties to even (finite inputs). */
uint16_t orc_bf16_from_f32(float v);
/* fp64 -> bf16 bits with a single rounding (nearest, ties to even). */
uint16_t orc_bf16_from_f64(double v);
/* bf16 bits -> fp32 (exact). */
float orc_f32_from_bf16(uint16_t b);
/* fp32 -> OCP FP8 E4M3FN byte: nearest, ties to even, |v| beyond the
 * largest finite value (448) saturates to +-448; NaN is never produced. */
uint8_t orc_e4m3fn_from_f32(float v);
/* OCP FP8 E4M3FN byte -> fp32 (0x7F/0xFF decode to NaN). */
float orc_f32_from_e4m3fn(uint8_t b);
/* fp32 -> OCP FP4 E2M1 code (low 4 bits; sign in bit 3): nearest, ties to
 * even, |v| beyond 6 saturates to +-6. */
uint8_t orc_e2m1_from_f32(float v);
/* E2M1 code -> fp32 (exact). */
float orc_f32_from_e2m1(uint8_t code);
/* E8M0 byte -> 2^(b-127) (0xFF -> NaN). */
float orc_f32_from_e8m0(uint8_t b);

/* ---- a1: routing layout ([P3] §2.1) ----
 * topk_idx: int32 [N,K], entries in [-1, E); -1 = masked.
 * Outputs: num_tokens_per_expert [E] (pairs), num_tokens_per_rank [R]
 * (distinct tokens), is_token_in_rank u8 [N,R], and, when ranks_per_node > 0
 * and num_tokens_per_rdma_rank != NULL, num_tokens_per_rdma_rank
 * [ceil(R/ranks_per_node)] (distinct tokens per node).
 * Returns 0, or -1 if an id lies outside [-1, E) (outputs then undefined). */
int orc_layout(const int32_t* topk_idx, int64_t N, int K, int E, int R, int ranks_per_node,
               int32_t* num_tokens_per_rank, int32_t* num_tokens_per_rdma_rank,
               int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank);

/* ---- a2: slot assignment ([P3] §3.1, §8.4) ----
 * psum_expert [E+1]: exclusive prefix of the A-aligned per-expert counts.
 * psum_rank [R+1]:   psum_expert at each rank's first expert.
 * num_unaligned [E]: raw per-expert counts.
 * slot_idx [N,K]:    receive row of each (t,k), -1 where masked.
 * src_meta [meta_cap,2]: (t,k) of each receive row, (-1,-1) on padding rows.
 * Returns S (total receive rows incl. padding), -1 on a bad id, -2 if
 * S > meta_cap. */
int64_t orc_slots(const int32_t* topk_idx, int64_t N, int K, int E, int R, int A,
                  int32_t* psum_expert, int32_t* psum_rank, int32_t* num_unaligned,
                  int32_t* slot_idx, int32_t* src_meta, int64_t meta_cap);

/* Fixed-capacity receive layout (the low-latency buffer shape
 * [num_local_experts, ranks x max_tokens, hidden] of [P3] §6.3, with one
 * source rank): expert e owns rows [e*cap, (e+1)*cap) whatever its count;
 * slot = e*cap + position of (t,k) among the pairs of e in (t,k) order.
 * A pair whose position reaches cap gets slot -1 (dropped).  psum_expert[e]
 * = e*cap, psum_rank[r] = r*nle*cap, num_unaligned = raw counts, src_meta
 * [E*cap, 2] with (-1,-1) on unused rows.  Returns the number of dropped
 * pairs, or -1 on a bad id. */
int64_t orc_slots_fixed(const int32_t* topk_idx, int64_t N, int K, int E, int R, int cap,
                        int32_t* psum_expert, int32_t* psum_rank, int32_t* num_unaligned,
                        int32_t* slot_idx, int32_t* src_meta);

/* Several source ranks stacked in one batch ([P3] §3.1
 * psum_num_recv_tokens_per_scaleup_rank): source p owns tokens
 * [p*N/P, (p+1)*N/P), so the (source, token, k) receive order is the (t,k)
 * order of orc_slots.  psum_source_rank [R][P+1]: per receiving rank, the
 * exclusive prefix over sources of the tokens received from each source
 * (a token counted once per rank).  expert_source_base [P][E]: pairs of
 * expert e from the sources before p.  Returns 0, -1 on a bad id, -2 if
 * P < 1 or N % P != 0. */
int orc_source_counts(const int32_t* topk_idx, int64_t N, int K, int E, int R, int P,
                      int32_t* psum_source_rank, int32_t* expert_source_base);

/* Non-expand receive layout ([P3] §2.1 V1 normal dispatch, §3.1 do_expand):
 * one row per (token, rank holding one of its experts); rank r's rows are
 * [psum_rank[r], psum_rank[r+1]) in token order; slot_idx[t,k] is the row of
 * (t, rank of idx[t,k]) for the row's first k on that rank, else -1;
 * src_meta [rows,2] = (t, first k).  psum_rank [R+1].  Returns the number of
 * rows, -1 on a bad id. */
int64_t orc_slots_nonexpand(const int32_t* topk_idx, int64_t N, int K, int E, int R,
                            int32_t* psum_rank, int32_t* slot_idx, int32_t* src_meta);

/* recv_topk_idx / recv_topk_weights [rows,K] of the non-expand layout: local
 * expert id and weight where expert idx[t,k] is on the row's rank, else -1
 * and 0. */
void orc_recv_topk(const int32_t* topk_idx, const float* topk_weights, const int32_t* src_meta,
                   int64_t rows, int K, int E, int R, int32_t* recv_topk_idx,
                   float* recv_topk_weights);

/* Host list of received tokens per expert ([P2] MOE_EXPERT_TOKEN_NUMS_TYPE):
 * counts_as_prefix == 0: aligned count of each expert;
 * counts_as_prefix != 0: inclusive prefix of those counts restarting at each
 * rank's first local expert. list [E]. */
void orc_recv_list(const int32_t* psum_expert, int E, int R, int counts_as_prefix, int32_t* list);

/* Host list of the fixed-capacity layout (orc_slots_fixed): the rows each
 * expert's segment actually holds, min(num_unaligned[e], cap), or with
 * counts_as_prefix their inclusive prefix restarting at each rank's first
 * local expert.  list [E]. */
void orc_recv_list_fixed(const int32_t* num_unaligned, int E, int R, int cap,
                         int counts_as_prefix, int32_t* list);

/* ---- a3: dispatch ([P3] §2.1/§2.2; quantisation [P5] §1.3.1, §1.3.3,
 *      [P3] §7.4) ----
 * x: bf16 bits [N,H]. For every t in [t_begin, t_end) and every k with
 * slot_idx[t,k] >= 0, receive row slot_idx[t,k] receives token t.
 * quant 0: recv_x is bf16 [*,H] (bit copy), recv_scales unused.
 * quant 1: recv_x is E4M3FN bytes [*,H]; quant 2: int8 [*,H].
 *   group = elements per scale (128 or H), G = H/group.  scale_mode 0:
 *   recv_scales fp32 [*,G] = amax/qmax; 1: fp32, rounded up to a power of
 *   two; 2: that power of two as an E8M0 byte, recv_scales uint8 [*,G].
 * quant 3 (MXFP4): group 32; recv_x holds two E2M1 codes per byte [*,H/2]
 *   (element 2i in the low nibble), recv_scales one E8M0 byte per group
 *   [*,H/32]; scale_mode unused. */
void orc_dispatch(const uint16_t* x, int64_t N, int H, const int32_t* slot_idx, int K,
                  int quant, int group, int scale_mode, int64_t t_begin, int64_t t_end,
                  void* recv_x, void* recv_scales);

/* ---- a4: combine ([P2] API table; weighted reduce) ----
 * out[t,:] = bf16( sum over k with slot_idx[t,k] >= 0 of w[t,k] * y[slot,:] ),
 * the exact sum rounded once (nearest, ties to even).  Rows with every k
 * masked, and exact zero sums, are +0. */
void orc_combine(const uint16_t* y, const float* topk_weights, const int32_t* slot_idx,
                 int64_t N, int K, int H, int64_t t_begin, int64_t t_end, uint16_t* out);

/* The combine in fp32: acc = +0; for k ascending with slot_idx[t,k] >= 0,
 * acc = fmaf(w[t,k], y[slot,h], acc); out[t,h] = bf16(acc), nearest-even. */
void orc_combine_fma(const uint16_t* y, const float* topk_weights, const int32_t* slot_idx,
                     int64_t N, int K, int H, int64_t t_begin, int64_t t_end, uint16_t* out);

/* Combine of quantised expert outputs ([P5]: combine int8 / fp8 from v2.1):
 * y_codes [*,H] E4M3FN (quant 1) or int8 (quant 2) with fp32 y_scales
 * [*,H/group]; element value code * scale; otherwise as orc_combine. */
void orc_combine_q(const void* y_codes, const float* y_scales, int quant, int group,
                   const float* topk_weights, const int32_t* slot_idx, int64_t N, int K, int H,
                   int64_t t_begin, int64_t t_end, uint16_t* out);

/* The same in fp32: value = code * scale rounded to fp32, then the fmaf
 * chain of orc_combine_fma. */
void orc_combine_q_fma(const void* y_codes, const float* y_scales, int quant, int group,
                       const float* topk_weights, const int32_t* slot_idx, int64_t N, int K,
                       int H, int64_t t_begin, int64_t t_end, uint16_t* out);

#ifdef __cplusplus
}
#endif

#endif
