/*
 * Plain CPU oracle for the MoE token shuffle.  TEST INFRASTRUCTURE ONLY:
 * used by the tests, the smoke check and the benchmark's CPU-baseline leg,
 * never by the product path.  Shares nothing with the HIP library.
 *
 * Every function is the plain definition, in the order the pages state the
 * method; no blocking, fusion or reordering.  Sources are cited by page
 * title and section (see ep_oracle.h for the key [P2], [P3], [P5]).
 */
#include "ep_oracle.h"

#include <fenv.h>
#include <math.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The plain build is serial.  The same source built with OpenMP runs the
 * per-token loops of dispatch and combine on several threads (each token's
 * results depend on that token alone, so both builds give the same bits);
 * that build only serves to time the oracle on a host's cores. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* Round v to the nearest number that has p significant bits and an exponent
 * of at least emin (numbers below 2^emin share the fixed step
 * 2^(emin - p + 1), i.e. the subnormal range), ties to even.  Dividing by a
 * power of two is exact in fp64, so the only rounding is nearbyint() in the
 * default round-to-nearest-even mode. */
static double round_to_format(double v, int p, int emin)
{
    if (v == 0.0 || !isfinite(v)) return v;
    int e2;
    frexp(fabs(v), &e2);          /* |v| = m * 2^e2, m in [0.5, 1) */
    int ex = e2 - 1;              /* 2^ex <= |v| < 2^(ex+1) */
    if (ex < emin) ex = emin;
    double step = ldexp(1.0, ex - (p - 1));
    return nearbyint(v / step) * step;
}

/* bf16: 8 significant bits, fp32's exponent range (min normal 2^-126). */
uint16_t orc_bf16_from_f64(double v)
{
    double r = round_to_format(v, 8, -126);
    uint32_t sign = signbit(r) ? 0x8000u : 0u;
    if (fabs(r) > 3.3895313892515355e38) /* largest finite bf16 */
        return (uint16_t)(sign | 0x7F80u);      /* rounds to infinity */
    float f = (float)r;                         /* exact: r has 8 bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(bits >> 16);
}

uint16_t orc_bf16_from_f32(float v) { return orc_bf16_from_f64((double)v); }

float orc_f32_from_bf16(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* OCP 8-bit floating point, E4M3FN variant ([P3] §7.4 names
 * torch.float8_e4m3fn as the FP8 storage type): 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormal step 2^-9, largest finite 448, no
 * infinities, S.1111.111 is NaN. */
uint8_t orc_e4m3fn_from_f32(float v)
{
    double r = round_to_format((double)v, 4, -6);
    uint8_t sign = signbit(r) ? 0x80 : 0x00;
    double a = fabs(r);
    if (a > 448.0) a = 448.0;                   /* saturate (reading) */
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -6)) {                   /* subnormal: a = m * 2^-9 */
        int m = (int)(a / ldexp(1.0, -9));
        return (uint8_t)(sign | m);
    }
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;                            /* -6 .. 8 */
    int m = (int)((a / ldexp(1.0, ex) - 1.0) * 8.0);
    return (uint8_t)(sign | ((ex + 7) << 3) | m);
}

float orc_f32_from_e4m3fn(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
    double a;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) a = ldexp((double)m, -9);
    else a = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -a : a);
}

/* OCP FP4 E2M1 (OCP Microscaling Formats v1.0; the element type of MXFP4,
 * which "DeepEP 通信库使用指南（v2.1）" §1.3.3 names with its group of 32):
 * 1 sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6.  Nearest, ties to even; |v| beyond 6 saturates to 6.
 * Returns the 4-bit code (sign in bit 3). */
uint8_t orc_e2m1_from_f32(float v)
{
    double r = round_to_format((double)v, 2, 0);
    uint8_t sign = signbit(r) ? 0x8 : 0x0;
    double a = fabs(r);
    if (a > 6.0) a = 6.0;
    if (a == 0.0) return sign;
    if (a < 1.0) return (uint8_t)(sign | 1);    /* subnormal 0.5 */
    int e2;
    frexp(a, &e2);
    int ex = e2 - 1;                            /* 0 .. 2 */
    int m = (int)((a / ldexp(1.0, ex) - 1.0) * 2.0);
    return (uint8_t)(sign | ((ex + 1) << 1) | m);
}

float orc_f32_from_e2m1(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double a = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (float)(s ? -a : a);
}

/* E8M0 (OCP MX scale type): the byte b stands for 2^(b - 127); 0xFF is NaN. */
float orc_f32_from_e8m0(uint8_t b)
{
    if (b == 0xFF) return NAN;
    return (float)ldexp(1.0, (int)b - 127);
}

/* Array forms for tests. */
void orc_bf16_from_f32_n(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(in[i]);
}
void orc_bf16_from_f64_n(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f64(in[i]);
}
void orc_e4m3fn_from_f32_n(const float* in, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3fn_from_f32(in[i]);
}
void orc_f32_from_e4m3fn_n(const uint8_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_from_e4m3fn(in[i]);
}

/* ------------------------------------------------------------------------ */
/* a1: routing layout                                                        */
/* ------------------------------------------------------------------------ */

/* Expert e belongs to rank e / num_local_experts, num_local_experts =
 * num_experts / ep_world_size ([P2] HCCL_BUFFSIZE note).  Reading: each rank
 * owns a contiguous block of experts. */
static int rank_of_expert(int e, int num_local_experts) { return e / num_local_experts; }

static int ids_valid(const int32_t* topk_idx, int64_t n, int E)
{
    for (int64_t i = 0; i < n; ++i)
        if (topk_idx[i] < -1 || topk_idx[i] >= E) return 0;
    return 1;
}

int orc_layout(const int32_t* topk_idx, int64_t N, int K, int E, int R, int ranks_per_node,
               int32_t* num_tokens_per_rank, int32_t* num_tokens_per_rdma_rank,
               int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank)
{
    if (!ids_valid(topk_idx, N * K, E)) return -1;
    int nle = E / R;

    /* num_tokens_per_expert: every (token, k) routed to the expert counts. */
    for (int e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int e = topk_idx[t * K + k];
            if (e >= 0) num_tokens_per_expert[e] += 1;
        }

    /* is_token_in_rank: the token has at least one expert on the rank. */
    for (int64_t t = 0; t < N; ++t) {
        for (int r = 0; r < R; ++r) is_token_in_rank[t * R + r] = 0;
        for (int k = 0; k < K; ++k) {
            int e = topk_idx[t * K + k];
            if (e >= 0) is_token_in_rank[t * R + rank_of_expert(e, nle)] = 1;
        }
    }

    /* num_tokens_per_rank: tokens the rank receives (each token once). */
    for (int r = 0; r < R; ++r) {
        int32_t c = 0;
        for (int64_t t = 0; t < N; ++t) c += is_token_in_rank[t * R + r];
        num_tokens_per_rank[r] = c;
    }

    /* num_tokens_per_rdma_rank: tokens a node (ranks_per_node consecutive
     * ranks) receives, each token once. */
    if (ranks_per_node > 0 && num_tokens_per_rdma_rank) {
        int nodes = (R + ranks_per_node - 1) / ranks_per_node;
        for (int n = 0; n < nodes; ++n) {
            int32_t c = 0;
            for (int64_t t = 0; t < N; ++t) {
                int hit = 0;
                for (int r = n * ranks_per_node; r < (n + 1) * ranks_per_node && r < R; ++r)
                    if (is_token_in_rank[t * R + r]) hit = 1;
                c += hit;
            }
            num_tokens_per_rdma_rank[n] = c;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a2: slot assignment                                                       */
/* ------------------------------------------------------------------------ */

int64_t orc_slots(const int32_t* topk_idx, int64_t N, int K, int E, int R, int A,
                  int32_t* psum_expert, int32_t* psum_rank, int32_t* num_unaligned,
                  int32_t* slot_idx, int32_t* src_meta, int64_t meta_cap)
{
    if (!ids_valid(topk_idx, N * K, E)) return -1;
    int nle = E / R;

    for (int e = 0; e < E; ++e) num_unaligned[e] = 0;
    for (int64_t i = 0; i < N * K; ++i)
        if (topk_idx[i] >= 0) num_unaligned[topk_idx[i]] += 1;

    /* Each expert's receive segment is its count rounded up to a multiple of
     * expert_alignment; psum_num_recv_tokens_per_expert is the prefix of the
     * aligned sizes ([P3] §3.1: psum vs num_unaligned field pair). */
    psum_expert[0] = 0;
    for (int e = 0; e < E; ++e) {
        int32_t aligned = ((num_unaligned[e] + A - 1) / A) * A;
        psum_expert[e + 1] = psum_expert[e] + aligned;
    }
    for (int r = 0; r <= R; ++r) psum_rank[r] = psum_expert[r * nle];

    int64_t S = psum_expert[E];
    if (S > meta_cap) return -2;
    for (int64_t s = 0; s < S; ++s) {
        src_meta[2 * s] = -1;
        src_meta[2 * s + 1] = -1;
    }
    for (int64_t i = 0; i < N * K; ++i) slot_idx[i] = -1;

    /* Inside an expert's segment the rows follow source token order, then k
     * (reading of the deterministic order of [P3] §8.4; with a single source
     * rank this is the stable order).  Padding rows sit at the segment end. */
    for (int e = 0; e < E; ++e) {
        int32_t next = psum_expert[e];
        for (int64_t t = 0; t < N; ++t)
            for (int k = 0; k < K; ++k)
                if (topk_idx[t * K + k] == e) {
                    slot_idx[t * K + k] = next;
                    src_meta[2 * (int64_t)next] = (int32_t)t;
                    src_meta[2 * (int64_t)next + 1] = k;
                    next += 1;
                }
    }
    return S;
}

int64_t orc_slots_fixed(const int32_t* topk_idx, int64_t N, int K, int E, int R, int cap,
                        int32_t* psum_expert, int32_t* psum_rank, int32_t* num_unaligned,
                        int32_t* slot_idx, int32_t* src_meta)
{
    if (!ids_valid(topk_idx, N * K, E)) return -1;
    int nle = E / R;
    for (int e = 0; e <= E; ++e) psum_expert[e] = e * cap;
    for (int r = 0; r <= R; ++r) psum_rank[r] = r * nle * cap;
    for (int64_t s = 0; s < (int64_t)E * cap; ++s) {
        src_meta[2 * s] = -1;
        src_meta[2 * s + 1] = -1;
    }
    int64_t dropped = 0;
    for (int e = 0; e < E; ++e) {
        int32_t pos = 0;
        for (int64_t t = 0; t < N; ++t)
            for (int k = 0; k < K; ++k) {
                if (topk_idx[t * K + k] != e) continue;
                if (pos < cap) {
                    int64_t s = (int64_t)e * cap + pos;
                    slot_idx[t * K + k] = (int32_t)s;
                    src_meta[2 * s] = (int32_t)t;
                    src_meta[2 * s + 1] = k;
                } else {
                    slot_idx[t * K + k] = -1;
                    dropped += 1;
                }
                pos += 1;
            }
        num_unaligned[e] = pos;
    }
    for (int64_t i = 0; i < N * K; ++i)
        if (topk_idx[i] < 0) slot_idx[i] = -1;
    return dropped;
}

/* Several source ranks in one batch: source p owns tokens [p*Ns, (p+1)*Ns),
 * Ns = N / P.  Ordering receive rows by (source, token, k) is then the
 * (t, k) order of the stacked batch, so orc_slots already places them; this
 * adds the per-source quantities of the EPHandle ([P3] §3.1
 * psum_num_recv_tokens_per_scaleup_rank, §3.2 its caching):
 *   psum_source_rank [R][P+1]: for receiving rank r, the exclusive prefix
 *     over sources of the tokens r receives from each source, a token
 *     counted once per rank it has an expert on (reading: as for
 *     num_tokens_per_rank, one copy of a token travels to each rank);
 *   expert_source_base [P][E]: pairs of expert e from sources before p --
 *     source p's rows of expert e start at psum_expert[e] + this.
 * Returns 0, -1 on a bad id, -2 if P < 1 or N is not a multiple of P. */
int orc_source_counts(const int32_t* topk_idx, int64_t N, int K, int E, int R, int P,
                      int32_t* psum_source_rank, int32_t* expert_source_base)
{
    if (P < 1 || N % P != 0) return -2;
    if (!ids_valid(topk_idx, N * K, E)) return -1;
    int nle = E / R;
    int64_t Ns = N / P;
    for (int r = 0; r < R; ++r) psum_source_rank[r * (P + 1)] = 0;
    for (int e = 0; e < E; ++e) expert_source_base[e] = 0;   /* source 0 */
    for (int p = 0; p < P; ++p) {
        /* this source's tokens per rank and pairs per expert */
        for (int r = 0; r < R; ++r) {
            int32_t c = 0;
            for (int64_t t = p * Ns; t < (p + 1) * Ns; ++t) {
                int hit = 0;
                for (int k = 0; k < K; ++k) {
                    int e = topk_idx[t * K + k];
                    if (e >= 0 && rank_of_expert(e, nle) == r) hit = 1;
                }
                c += hit;
            }
            psum_source_rank[r * (P + 1) + p + 1] = psum_source_rank[r * (P + 1) + p] + c;
        }
        if (p + 1 < P)
            for (int e = 0; e < E; ++e) {
                int32_t c = 0;
                for (int64_t t = p * Ns; t < (p + 1) * Ns; ++t)
                    for (int k = 0; k < K; ++k) c += topk_idx[t * K + k] == e;
                expert_source_base[(int64_t)(p + 1) * E + e] = expert_source_base[(int64_t)p * E + e] + c;
            }
    }
    return 0;
}

/* Non-expand receive layout (the V1 normal dispatch of "DeepEP V1 vs V2
 * 深度对比分析" §2.1, which returns recv_x with recv_topk_idx /
 * recv_topk_weights; EPHandle.do_expand of §3.1 chooses between the two
 * forms): a token travels once to each rank that holds one of its experts.
 * Rank r's rows are [psum_rank[r], psum_rank[r+1]), psum_rank the exclusive
 * prefix of num_tokens_per_rank, in source-token order.  slot_idx[t,k] is the
 * row of (t, rank of expert idx[t,k]) for the first k of the row on that
 * rank, -1 for later k on the same rank and for masked entries (reading: the
 * row belongs to the token's first entry on the rank).  src_meta[row] =
 * (t, that first k).  Returns the number of rows, or -1 on a bad id. */
int64_t orc_slots_nonexpand(const int32_t* topk_idx, int64_t N, int K, int E, int R,
                            int32_t* psum_rank, int32_t* slot_idx, int32_t* src_meta)
{
    if (!ids_valid(topk_idx, N * K, E)) return -1;
    int nle = E / R;
    /* rows per rank: distinct tokens */
    for (int r = 0; r <= R; ++r) psum_rank[r] = 0;
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) {
            int e = topk_idx[t * K + k];
            if (e < 0) continue;
            int r = rank_of_expert(e, nle), first = 1;
            for (int q = 0; q < k; ++q) {
                int eq = topk_idx[t * K + q];
                if (eq >= 0 && rank_of_expert(eq, nle) == r) first = 0;
            }
            if (first) psum_rank[r + 1] += 1;
        }
    for (int r = 0; r < R; ++r) psum_rank[r + 1] += psum_rank[r];
    /* rows in token order within each rank */
    for (int r = 0; r < R; ++r) {
        int32_t next = psum_rank[r];
        for (int64_t t = 0; t < N; ++t)
            for (int k = 0; k < K; ++k) {
                int e = topk_idx[t * K + k];
                if (e < 0 || rank_of_expert(e, nle) != r) continue;
                int first = 1;
                for (int q = 0; q < k; ++q) {
                    int eq = topk_idx[t * K + q];
                    if (eq >= 0 && rank_of_expert(eq, nle) == r) first = 0;
                }
                if (!first) continue;
                src_meta[2 * (int64_t)next] = (int32_t)t;
                src_meta[2 * (int64_t)next + 1] = k;
                next += 1;
            }
    }
    for (int64_t t = 0; t < N; ++t)
        for (int k = 0; k < K; ++k) slot_idx[t * K + k] = -1;
    for (int64_t s = 0; s < psum_rank[R]; ++s)
        slot_idx[(int64_t)src_meta[2 * s] * K + src_meta[2 * s + 1]] = (int32_t)s;
    return psum_rank[R];
}

/* Per received row of the non-expand layout, the token's routing as seen by
 * the receiving rank ([P3] §2.1 recv_topk_idx / recv_topk_weights): entry k
 * is the local expert id idx[t,k] - r*nle and the weight w[t,k] when expert
 * idx[t,k] is on the row's rank r, else -1 and 0.  rows = psum_rank[R]. */
void orc_recv_topk(const int32_t* topk_idx, const float* topk_weights, const int32_t* src_meta,
                   int64_t rows, int K, int E, int R, int32_t* recv_topk_idx,
                   float* recv_topk_weights)
{
    int nle = E / R;
    for (int64_t s = 0; s < rows; ++s) {
        int64_t t = src_meta[2 * s];
        int r = rank_of_expert(topk_idx[t * K + src_meta[2 * s + 1]], nle);
        for (int k = 0; k < K; ++k) {
            int e = topk_idx[t * K + k];
            int on = e >= 0 && rank_of_expert(e, nle) == r;
            recv_topk_idx[s * K + k] = on ? e - r * nle : -1;
            recv_topk_weights[s * K + k] = on ? topk_weights[t * K + k] : 0.0f;
        }
    }
}

void orc_recv_list(const int32_t* psum_expert, int E, int R, int counts_as_prefix, int32_t* list)
{
    int nle = E / R;
    for (int e = 0; e < E; ++e) {
        int32_t c = psum_expert[e + 1] - psum_expert[e];
        if (counts_as_prefix && e % nle != 0) c += list[e - 1];
        list[e] = c;
    }
}

/* Host list of the fixed-capacity layout: expert e's segment holds the
 * rows actually filled, min(count, cap) (pairs past cap are dropped), so
 * the list counts those, and with counts_as_prefix their inclusive prefix
 * restarting at each rank's first local expert ("A2_DEEPEP.md"
 * MOE_EXPERT_TOKEN_NUMS_TYPE, over the low-latency receive buffer of
 * "DeepEP V1 vs V2 深度对比分析" §6.3). */
void orc_recv_list_fixed(const int32_t* num_unaligned, int E, int R, int cap,
                         int counts_as_prefix, int32_t* list)
{
    int nle = E / R;
    for (int e = 0; e < E; ++e) {
        int32_t c = num_unaligned[e] < cap ? num_unaligned[e] : cap;
        if (counts_as_prefix && e % nle != 0) c += list[e - 1];
        list[e] = c;
    }
}

/* ------------------------------------------------------------------------ */
/* a3: dispatch                                                              */
/* ------------------------------------------------------------------------ */

/* Per-group symmetric quantisation.  Readings (the pages name the modes
 * -- FP8 with 128-element groups, int8 group 128 or channel = hidden -- but
 * not the arithmetic): amax = max |x| over the group, floored at 1e-4;
 * scale = amax / qmax in fp32 with qmax = 448 (E4M3FN) or 127 (int8);
 * code = x / scale in fp32, rounded to nearest-even into the format
 * (E4M3FN saturating; int8 clamped to [-127, 127]).
 *
 * Scale modes ("DeepEP 通信库使用指南（v2.1）" §1.3.1 API: round_scale,
 * use_ue8m0 -- named, not defined).  Readings: round_scale replaces the fp32
 * quotient amax / qmax by the smallest power of two not below it (so no
 * code saturates), and use_ue8m0 stores that power of two as one E8M0 byte
 * (its biased exponent) instead of an fp32 word. */
static float group_amax(const uint16_t* xg, int len)
{
    float amax = 0.0f;
    for (int i = 0; i < len; ++i) {
        float a = fabsf(orc_f32_from_bf16(xg[i]));
        if (a > amax) amax = a;
    }
    return amax;
}

/* Smallest power of two >= s (s > 0, normal). */
static float pow2_ceil(float s)
{
    int e;
    double m = frexp((double)s, &e);        /* s = m * 2^e, m in [0.5, 1) */
    return (float)ldexp(1.0, m == 0.5 ? e - 1 : e);
}

/* Biased exponent of a power of two: 2^k -> k + 127. */
static uint8_t e8m0_of_pow2(float s)
{
    int e;
    frexp((double)s, &e);
    return (uint8_t)(e - 1 + 127);
}

static float group_scale(const uint16_t* xg, int len, float qmax, int scale_mode)
{
    float amax = group_amax(xg, len);
    if (amax < 1e-4f) amax = 1e-4f;
    float s = amax / qmax;
    return scale_mode != 0 ? pow2_ceil(s) : s;
}

static int8_t int8_code(float q)
{
    double r = nearbyint((double)q);
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (int8_t)r;
}

/* MXFP4 shared exponent (OCP Microscaling Formats v1.0, conversion of a
 * block to MX): floor(log2(amax)) minus the exponent of E2M1's largest
 * value 6 = 1.5 * 2^2, i.e. minus 2, clamped to E8M0's range [-127, 127];
 * an all-zero group takes -127 (reading: the spec leaves it open). */
static int mx_shared_exp(float amax)
{
    if (amax == 0.0f) return -127;
    int e;
    frexp((double)amax, &e);                /* floor(log2 amax) = e - 1 */
    int x = e - 1 - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return x;
}

void orc_dispatch(const uint16_t* x, int64_t N, int H, const int32_t* slot_idx, int K,
                  int quant, int group, int scale_mode, int64_t t_begin, int64_t t_end,
                  void* recv_x, void* recv_scales)
{
    (void)N;
    if (quant == 0) {
        uint16_t* rx = (uint16_t*)recv_x;
#pragma omp parallel for schedule(static)
        for (int64_t t = t_begin; t < t_end; ++t)
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                for (int h = 0; h < H; ++h) rx[s * H + h] = x[t * H + h];
            }
        return;
    }

    int G = H / group;
    /* bytes per received row: one per element, or two E2M1 codes per byte */
    int row_bytes = quant == 3 ? H / 2 : H;
    int byte_scales = quant == 3 || scale_mode == 2;
    uint8_t* rx = (uint8_t*)recv_x;
#pragma omp parallel
    {
    /* one token's codes and scales (per thread in the OpenMP build) */
    uint8_t* codes = (uint8_t*)calloc((size_t)row_bytes, 1);
    float* scales = (float*)malloc(sizeof(float) * (size_t)G);
    uint8_t* scale_bytes = (uint8_t*)malloc((size_t)G);
#pragma omp for schedule(static)
    for (int64_t t = t_begin; t < t_end; ++t) {
        const uint16_t* xt = x + t * H;
        for (int g = 0; g < G; ++g) {
            const uint16_t* xg = xt + (int64_t)g * group;
            if (quant == 3) {
                /* MXFP4: element i of the row in nibble i % 2 of byte i / 2
                 * (low nibble first; reading) */
                int sx = mx_shared_exp(group_amax(xg, group));
                scale_bytes[g] = (uint8_t)(sx + 127);
                for (int i = g * group; i < (g + 1) * group; ++i) {
                    float q = (float)ldexp((double)orc_f32_from_bf16(xt[i]), -sx);
                    uint8_t c = orc_e2m1_from_f32(q);
                    if (i % 2 == 0) codes[i / 2] = c;
                    else codes[i / 2] |= (uint8_t)(c << 4);
                }
                continue;
            }
            float scale = group_scale(xg, group, quant == 1 ? 448.0f : 127.0f, scale_mode);
            scales[g] = scale;
            scale_bytes[g] = scale_mode == 2 ? e8m0_of_pow2(scale) : 0;
            for (int i = g * group; i < (g + 1) * group; ++i) {
                float q = orc_f32_from_bf16(xt[i]) / scale;
                codes[i] = (quant == 1) ? orc_e4m3fn_from_f32(q) : (uint8_t)int8_code(q);
            }
        }
        for (int k = 0; k < K; ++k) {
            int64_t s = slot_idx[t * K + k];
            if (s < 0) continue;
            for (int h = 0; h < row_bytes; ++h) rx[s * row_bytes + h] = codes[h];
            for (int g = 0; g < G; ++g) {
                if (byte_scales) ((uint8_t*)recv_scales)[s * G + g] = scale_bytes[g];
                else ((float*)recv_scales)[s * G + g] = scales[g];
            }
        }
    }
    free(codes);
    free(scales);
    free(scale_bytes);
    }
}

/* ------------------------------------------------------------------------ */
/* a4: combine                                                               */
/* ------------------------------------------------------------------------ */

/* Exact sums of products, rounded once to bf16.
 *
 * A term is the product of two or three finite factors (an fp32 weight, a
 * bf16 value, or a weight, a code and an fp32 scale).  Each factor is an odd
 * integer significand times a power of two; the term's significand is the
 * product of those (at most 24 + 24 + 9 bits) and its exponent the sum, never
 * below -EXACT_LOW.  The terms are added into a two's-complement integer of
 * EXACT_LIMBS 64-bit limbs in units of 2^-EXACT_LOW, which holds the exact sum
 * of up to 2^30 terms below 2^270 in magnitude.  The sum is then rounded to
 * the nearest bf16, ties to the even significand, from its bits.
 *
 * The fp64 sum is used instead whenever it is exact: every product is exact
 * in fp64 (checked with a fused multiply-add) and every addition is exact
 * (checked with Knuth's two-sum, whose error term is then zero). */
#define EXACT_LIMBS 10
#define EXACT_LOW 320

typedef struct {
    uint64_t l[EXACT_LIMBS];
} exact_acc;

/* |v| = sig * 2^exp with sig odd (sig = 0 for a zero); v finite, at most 53
 * significant bits. */
static void split_finite(double v, uint64_t* sig, int* exp, int* neg)
{
    *neg = signbit(v) != 0;
    v = fabs(v);
    *sig = 0;
    *exp = 0;
    if (v == 0.0) return;
    int e;
    double m = frexp(v, &e);                 /* v = m * 2^e, 0.5 <= m < 1 */
    uint64_t s = (uint64_t)ldexp(m, 53);
    e -= 53;
    while ((s & 1u) == 0) {
        s >>= 1;
        ++e;
    }
    *sig = s;
    *exp = e;
}

static void exact_add_product(exact_acc* a, const double* f, int nf)
{
    uint64_t sig = 1;
    int exp = 0, neg = 0;
    for (int i = 0; i < nf; ++i) {
        uint64_t s;
        int e, n;
        split_finite(f[i], &s, &e, &n);
        if (s == 0) return;                  /* the product is zero */
        sig *= s;
        exp += e;
        neg ^= n;
    }
    const int sh = exp + EXACT_LOW;          /* >= 0: see EXACT_LOW */
    const int li = sh / 64, bo = sh % 64;
    uint64_t part[EXACT_LIMBS] = {0};
    part[li] = sig << bo;
    if (bo != 0 && li + 1 < EXACT_LIMBS) part[li + 1] = sig >> (64 - bo);
    if (!neg) {
        uint64_t carry = 0;
        for (int i = 0; i < EXACT_LIMBS; ++i) {
            uint64_t x = a->l[i] + part[i];
            uint64_t c1 = x < part[i];
            uint64_t y = x + carry;
            uint64_t c2 = y < carry;
            a->l[i] = y;
            carry = c1 | c2;
        }
    } else {
        uint64_t borrow = 0;
        for (int i = 0; i < EXACT_LIMBS; ++i) {
            uint64_t x = a->l[i] - part[i];
            uint64_t b1 = a->l[i] < part[i];
            uint64_t y = x - borrow;
            uint64_t b2 = x < borrow;
            a->l[i] = y;
            borrow = b1 | b2;
        }
    }
}

static int exact_bit(const exact_acc* a, int i) { return (int)((a->l[i / 64] >> (i % 64)) & 1u); }

static int exact_any_below(const exact_acc* a, int i)
{
    for (int j = 0; j < i; ++j)
        if (exact_bit(a, j)) return 1;
    return 0;
}

static uint16_t exact_to_bf16(const exact_acc* acc)
{
    exact_acc m = *acc;
    const int neg = (int)(m.l[EXACT_LIMBS - 1] >> 63);
    if (neg) {                               /* magnitude: two's-complement negation */
        uint64_t carry = 1;
        for (int i = 0; i < EXACT_LIMBS; ++i) {
            uint64_t x = ~m.l[i] + carry;
            carry = (carry && x == 0) ? 1 : 0;
            m.l[i] = x;
        }
    }
    int p = -1;                              /* highest set bit */
    for (int i = EXACT_LIMBS - 1; i >= 0 && p < 0; --i)
        for (int j = 63; j >= 0; --j)
            if ((m.l[i] >> j) & 1u) {
                p = 64 * i + j;
                break;
            }
    if (p < 0) return 0;                     /* an exact zero sum is +0 */
    const int E = p - EXACT_LOW;             /* the sum lies in [2^E, 2^(E+1)) */
    const int q = E >= -126 ? E - 7 : -133;  /* bf16 spacing there (normal / subnormal) */
    const int b = q + EXACT_LOW;             /* bit of the spacing unit (>= 187) */
    uint64_t kept = 0;
    for (int i = p; i >= b; --i) kept = (kept << 1) | (uint64_t)exact_bit(&m, i);
    const int half = exact_bit(&m, b - 1), below = exact_any_below(&m, b - 1);
    if (half && (below || (kept & 1u))) ++kept;   /* nearest, ties to even */
    const double v = ldexp((double)kept, q);      /* a bf16 value, or 2^128 */
    return orc_bf16_from_f64(neg ? -v : v);
}

/* Knuth's two-sum: s = fl(a + b) and whether a + b == s exactly. */
static double two_sum(double a, double b, int* exact)
{
    const double s = a + b;
    const double bb = s - a;
    const double err = (a - (s - bb)) + (b - bb);
    if (err != 0.0) *exact = 0;
    return s;
}

/* Combine, the plain definition: the weighted sum of the token's expert
 * outputs, exact, rounded once to bf16 (see exact_to_bf16 above). */
void orc_combine(const uint16_t* y, const float* topk_weights, const int32_t* slot_idx,
                 int64_t N, int K, int H, int64_t t_begin, int64_t t_end, uint16_t* out)
{
    (void)N;
#pragma omp parallel for schedule(static)
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            int exact = 1;
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                /* exact: 24 x 8 significant bits */
                const double p = (double)topk_weights[t * K + k] * (double)orc_f32_from_bf16(y[s * H + h]);
                acc = two_sum(acc, p, &exact);
            }
            if (exact && isfinite(acc)) {
                out[t * H + h] = orc_bf16_from_f64(acc);
                continue;
            }
            exact_acc e = {{0}};
            int finite = 1;
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                const double f[2] = {(double)topk_weights[t * K + k],
                                     (double)orc_f32_from_bf16(y[s * H + h])};
                if (!isfinite(f[0]) || !isfinite(f[1])) finite = 0;
                else exact_add_product(&e, f, 2);
            }
            out[t * H + h] = finite ? exact_to_bf16(&e) : orc_bf16_from_f64(acc);
        }
}

/* Combine accumulated in fp32 (the stated precision of the reduction; the
 * order and the fused multiply-add are the reading): acc starts at +0 and,
 * for k = 0, 1, ..., K-1 with a slot, acc = fmaf(w[t,k], y[slot, h], acc),
 * one rounding per step; out = bf16(acc), nearest-even.  fmaf is the C
 * library's correctly rounded fused multiply-add. */
void orc_combine_fma(const uint16_t* y, const float* topk_weights, const int32_t* slot_idx,
                     int64_t N, int K, int H, int64_t t_begin, int64_t t_end, uint16_t* out)
{
    (void)N;
#pragma omp parallel for schedule(static)
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                acc = fmaf(topk_weights[t * K + k], orc_f32_from_bf16(y[s * H + h]), acc);
            }
            out[t * H + h] = orc_bf16_from_f32(acc);
        }
}

/* Value of element h of a quantised expert-output row: code * scale. */
static double code_of(const uint8_t* yc, int quant, int H, int64_t s, int h)
{
    uint8_t c = yc[s * H + h];
    return quant == 1 ? (double)orc_f32_from_e4m3fn(c) : (double)(int8_t)c;
}

/* Combine of quantised expert outputs ("DeepEP 通信库使用指南（v2.1）":
 * from v2.1 combine accepts int8 / fp8 quantisation, with the same
 * quant_size choice as dispatch): y row s holds codes (E4M3FN bytes when
 * quant == 1, int8 when quant == 2) and fp32 scales [*, H/group]; the value
 * of element h is code * scale.  The sum is exact and rounded once to bf16,
 * as in orc_combine. */
void orc_combine_q(const void* y_codes, const float* y_scales, int quant, int group,
                   const float* topk_weights, const int32_t* slot_idx, int64_t N, int K, int H,
                   int64_t t_begin, int64_t t_end, uint16_t* out)
{
    (void)N;
    const uint8_t* yc = (const uint8_t*)y_codes;
    const int G = H / group;
#pragma omp parallel for schedule(static)
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            int exact = 1;
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                /* code * scale is exact (at most 9 x 24 bits); the weight's
                 * product with it may not be: fma recovers its error */
                const double w = (double)topk_weights[t * K + k];
                const double v = code_of(yc, quant, H, s, h) * (double)y_scales[s * G + h / group];
                const double p = w * v;
                if (fma(w, v, -p) != 0.0) exact = 0;
                acc = two_sum(acc, p, &exact);
            }
            if (exact && isfinite(acc)) {
                out[t * H + h] = orc_bf16_from_f64(acc);
                continue;
            }
            exact_acc e = {{0}};
            int finite = 1;
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                const double f[3] = {(double)topk_weights[t * K + k], code_of(yc, quant, H, s, h),
                                     (double)y_scales[s * G + h / group]};
                if (!isfinite(f[0]) || !isfinite(f[1]) || !isfinite(f[2])) finite = 0;
                else exact_add_product(&e, f, 3);
            }
            out[t * H + h] = finite ? exact_to_bf16(&e) : orc_bf16_from_f64(acc);
        }
}

/* The same in fp32, as orc_combine_fma: the element value is the fp32
 * product code * scale (one rounding), then acc = fmaf(w, value, acc) for k
 * ascending, out = bf16(acc). */
void orc_combine_q_fma(const void* y_codes, const float* y_scales, int quant, int group,
                       const float* topk_weights, const int32_t* slot_idx, int64_t N, int K,
                       int H, int64_t t_begin, int64_t t_end, uint16_t* out)
{
    (void)N;
    const uint8_t* yc = (const uint8_t*)y_codes;
#pragma omp parallel for schedule(static)
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int64_t s = slot_idx[t * K + k];
                if (s < 0) continue;
                uint8_t c = yc[s * H + h];
                float code = quant == 1 ? orc_f32_from_e4m3fn(c) : (float)(int8_t)c;
                float v = code * y_scales[s * (H / group) + h / group];
                acc = fmaf(topk_weights[t * K + k], v, acc);
            }
            out[t * H + h] = orc_bf16_from_f32(acc);
        }
}
