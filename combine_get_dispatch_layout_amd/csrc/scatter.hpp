// Device building blocks of the dispatch scatter (load a row chunk, quantise,
// write it to the token's receive rows), shared by the dispatch kernel
// (dispatch.hip), the single-launch layout + dispatch (fused.hip) and the
// dispatch launch that also runs the next batch's layout (overlap.hip).  See
// dispatch.hip for what is computed and its sources.
#pragma once

#include <type_traits>

#include "ep_internal.hpp"

// Whether x loads and receive-row stores carry the non-temporal hint.
#ifndef EP_DISPATCH_NT
#define EP_DISPATCH_NT 1
#endif

// >= 0: force the per-shape choices below (for measurements).
#ifndef EP_DISPATCH_VPL
#define EP_DISPATCH_VPL -1
#endif
#ifndef EP_DISPATCH_ROW_WAIT
#define EP_DISPATCH_ROW_WAIT -1
#endif

namespace epk {

// Row-wait choice: rows of 8 KiB or more are written one row at a time per
// wave; shorter rows keep all K rows' stores in flight (measured on MI355X:
// 14 KiB rows 187 us vs 205 us, 4 KiB rows 27.3 us vs 29.2 us).
inline bool dispatch_row_wait(int row_bytes)
{
    return EP_DISPATCH_ROW_WAIT >= 0 ? EP_DISPATCH_ROW_WAIT != 0 : row_bytes >= 8192;
}

// Vectors per lane of the plain scatter: long rows (>= 8 KiB) one 1 KiB piece
// per wave; shorter rows as few waves per row as possible, up to 4 KiB each.
inline int dispatch_plain_vpl(int NV, int row_bytes)
{
    if (EP_DISPATCH_VPL >= 0) return EP_DISPATCH_VPL;
    return row_bytes >= 8192 ? 1 : (NV <= 64 ? 1 : NV <= 128 ? 2 : 4);
}

#ifndef EP_DISPATCH_QVPL
#define EP_DISPATCH_QVPL -1
#endif

// Vectors per lane of the quantised scatter with per-group scales (each
// vector of a lane is its own group slice): the plain scatter's rule on the
// input row (2H bytes).  Measured on MI355X, Qwen3 shape (H 2048): FP8 17.8
// us with 4 vectors per lane vs 19.8 us with 1, MXFP4 11.0 vs 14.3 us; rows
// of 7168 and decode batches are fastest with 1.
inline int dispatch_quant_vpl(int NV)
{
    if (EP_DISPATCH_QVPL >= 0) return EP_DISPATCH_QVPL;
    return dispatch_plain_vpl(NV, NV * 16);
}

// The dispatch launch shape for a's format and row size: calls
// launch(quant, channel, vpl, row_wait, NV) with the first four as
// std::integral_constant / std::bool_constant values, NV = H/8 vectors.
//   bf16: dispatch_plain_vpl vectors per lane;
//   FP8 / int8 per 128 elements, MXFP4: dispatch_quant_vpl;
//   FP8 / int8 per row: the whole row in one wave (VPL = 64*VPL >= NV).
// Row waits follow dispatch_row_wait on the receive row's bytes.
template <int Q, bool CH, int VPL, class L>
inline hipError_t shape_rw(int NV, int row_bytes, L& launch)
{
    using RW1 = std::bool_constant<true>;
    using RW0 = std::bool_constant<false>;
    using QC = std::integral_constant<int, Q>;
    using CC = std::bool_constant<CH>;
    using VC = std::integral_constant<int, VPL>;
    // Receive rows of 8 KiB or more come with one vector per lane, or with a
    // whole row per wave (channel scales, 16 vectors per lane); the other
    // shapes are not instantiated with row waits (the wait is a performance
    // choice only: the rows written are the same).
    constexpr bool may_wait = VPL == 1 || (CH && VPL == 16) || EP_DISPATCH_VPL >= 0;
    if constexpr (may_wait)
        return dispatch_row_wait(row_bytes) ? launch(QC{}, CC{}, VC{}, RW1{}, NV)
                                            : launch(QC{}, CC{}, VC{}, RW0{}, NV);
    else
        return launch(QC{}, CC{}, VC{}, RW0{}, NV);
}

template <int Q, class L>
inline hipError_t shape_group(int NV, int row_bytes, L& launch)
{
    switch (dispatch_quant_vpl(NV)) {
        case 2: return shape_rw<Q, false, 2>(NV, row_bytes, launch);
        case 4: return shape_rw<Q, false, 4>(NV, row_bytes, launch);
        default: return shape_rw<Q, false, 1>(NV, row_bytes, launch);
    }
}

template <int Q, class L>
inline hipError_t shape_channel(int NV, L& launch)
{
    const int rb = NV * 8;   // one byte per element
    if (NV <= 64) return shape_rw<Q, true, 1>(NV, rb, launch);
    if (NV <= 128) return shape_rw<Q, true, 2>(NV, rb, launch);
    if (NV <= 256) return shape_rw<Q, true, 4>(NV, rb, launch);
    if (NV <= 512) return shape_rw<Q, true, 8>(NV, rb, launch);
    return shape_rw<Q, true, 16>(NV, rb, launch);
}

template <class L>
inline hipError_t dispatch_shape(const DispatchArgs& a, L& launch)
{
    const int NV = a.H / 8;
    const bool channel = a.quant != 0 && a.group == a.H && a.H != 128;
    switch (a.quant) {
        case 0: {
            const int rb = a.H * 2;
            switch (dispatch_plain_vpl(NV, rb)) {
                case 1: return shape_rw<0, false, 1>(NV, rb, launch);
                case 2: return shape_rw<0, false, 2>(NV, rb, launch);
                case 8: return shape_rw<0, false, 8>(NV, rb, launch);
                default: return shape_rw<0, false, 4>(NV, rb, launch);
            }
        }
        case 1: return channel ? shape_channel<1>(NV, launch) : shape_group<1>(NV, a.H, launch);
        case 2: return channel ? shape_channel<2>(NV, launch) : shape_group<2>(NV, a.H, launch);
        default: return shape_group<3>(NV, a.H / 2, launch);
    }
}

namespace scatter {

template <typename T>
__device__ __forceinline__ T load_stream(const T* p)
{
    if constexpr (EP_DISPATCH_NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Receive-row stores go through a buffer resource per row (base = the row,
// bound = the row's bytes; the third word is the gfx9 raw-buffer format):
// the row address lives in scalar registers and the lane offset in one
// vector register that never changes, so consecutive stores of a wave need
// no wait between them, and the hardware drops anything outside the row.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStoreAux = EP_DISPATCH_NT ? 2 : 0;   // nt cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(char* row, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(row, 0, bytes, kBufferWord3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// x from another lane of the same row of 16 (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Maximum over aligned groups of WIDTH lanes (4, 16 or the wave), in every
// lane of the group, by DPP exchanges: lane ^ 1 and lane ^ 2 inside a quad,
// then the mirrored lane of the half-row (the other quad) and of the row
// (the other half-row); across rows by reading the four row maxima.  The
// whole wave must be active.
template <int WIDTH>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(WIDTH == 4 || WIDTH == 16 || WIDTH == kWave, "groups of 4, 16 or 64 lanes");
    v = fmaxf(v, dpp_f<0xB1>(v));       // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4E>(v));       // quad_perm [2,3,0,1]
    if constexpr (WIDTH >= 16) {
        v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
        v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
    }
    if constexpr (WIDTH == kWave) {
        const int b = __float_as_int(v);
        v = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                        __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                  fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                        __int_as_float(__builtin_amdgcn_readlane(b, 48))));
    }
    return v;
}

// Four int8 codes: clamp(round_nearest_even(q), -127, 127).  Adding 1.5 * 2^23
// to the clamped value rounds it to an integer (ties to even) that then sits
// in the low mantissa bits, its low byte being the two's complement code; a
// byte permute gathers the four low bytes.
__device__ __forceinline__ uint32_t pack_int8x4(float a, float b, float c, float d)
{
    constexpr float kRound = 12582912.0f;
    const uint32_t ia = __float_as_uint(fminf(fmaxf(a, -127.0f), 127.0f) + kRound);
    const uint32_t ib = __float_as_uint(fminf(fmaxf(b, -127.0f), 127.0f) + kRound);
    const uint32_t ic = __float_as_uint(fminf(fmaxf(c, -127.0f), 127.0f) + kRound);
    const uint32_t id = __float_as_uint(fminf(fmaxf(d, -127.0f), 127.0f) + kRound);
    // v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7
    // of the first, 0x0c gives zero
    const uint32_t lo = __builtin_amdgcn_perm(ib, ia, 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(id, ic, 0x04000C0Cu);
    return lo | hi;
}

// Largest magnitude of a vector's eight bf16 values.  Finite bf16 magnitudes
// order like their 15-bit patterns, so the maximum is an integer maximum
// over the 16-bit halves (sign bits cleared), widened back to fp32.
__device__ __forceinline__ float absmax8(const u32x4& w)
{
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int j = 1; j < 4; ++j)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    const uint32_t top = m[0] > m[1] ? m[0] : m[1];
    return __uint_as_float(top << 16);
}

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// x / s rounded to nearest even, for a divisor shared by a whole group:
// r = 1/s is one IEEE division per group, then each element takes a product
// and one remainder correction in fused multiply-adds (Markstein's
// correction step: with r the correctly rounded reciprocal and q0 = x*r
// within an ulp, q0 + (x - q0*s)*r rounds to the quotient).  Checked on the
// CPU against the division for every bf16 x and every bf16 amax of the FP8
// and int8 scales: equal except below 1e-20 in magnitude, where both round
// to a zero code.  The copysign keeps -0 for x = -0.
__device__ __forceinline__ float div_shared(float x, float s, float r)
{
    const float q0 = x * r;
    const float rem = __builtin_fmaf(-q0, s, x);
    return __builtin_copysignf(__builtin_fmaf(rem, r, q0), x);
}

// Smallest power of two >= s, for a positive normal s (round_scale).
__device__ __forceinline__ float pow2_ceil(float s)
{
    uint32_t u = __float_as_uint(s);
    if (u & 0x007FFFFFu) u = (u & 0xFF800000u) + 0x00800000u;
    return __uint_as_float(u);
}

// E8M0 byte of a power of two: its biased exponent.
__device__ __forceinline__ uint8_t e8m0_of_pow2(float s)
{
    return (uint8_t)((__float_as_uint(s) >> 23) & 0xFFu);
}

// MXFP4 shared exponent of a 32-element block with largest magnitude m:
// floor(log2 m) - 2 (E2M1's largest value is 1.5 * 2^2), clamped to E8M0's
// [-127, 127]; zero and subnormal m give -127.
__device__ __forceinline__ int mx_shared_exp(float m)
{
    const int e = (int)((__float_as_uint(m) >> 23) & 0xFFu);   // biased; m is finite
    return e == 0 ? -127 : max(e - 129, -127);
}

// OCP FP4 E2M1 code of q (sign in bit 3): nearest of 0, 0.5, 1, 1.5, 2, 3,
// 4, 6 with ties to the even code, saturating at 6.  Each comparison is one
// boundary between neighbouring codes; a tie stays on the even side.
__device__ __forceinline__ uint32_t e2m1_code(float q)
{
    const float m = fabsf(q);
    const uint32_t c = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                       (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) +
                       (uint32_t)(m > 5.0f);
    return c | ((__float_as_uint(q) >> 28) & 8u);
}

// Lane exchanges inside a quad of lanes (DPP quad_perm): the value of lane
// (lane ^ 1), and the value of quad lane j.
__device__ __forceinline__ uint32_t swap_pair(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
}

template <int J>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, J * 0x55, 0xF, 0xF, false);   // [J,J,J,J]
}

// Loads the wave's chunk of row t: VPL 16-byte vectors per lane starting at
// vector vbase (lane-contiguous), zero past the row end.
template <int VPL>
__device__ __forceinline__ void load_chunk(const DispatchArgs& a, int64_t t, int vbase, int NV,
                                           u32x4 (&d)[VPL])
{
    const u32x4* xrow = reinterpret_cast<const u32x4*>(a.x) + t * NV;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = vbase + kWave * i;
        d[i] = (v < NV) ? load_stream(xrow + v) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Writes the chunk (loaded by load_chunk) to the token's receive rows
// sl[0..K), quantising it first when QUANT != 0.
// QUANT: 0 none, 1 E4M3FN, 2 int8, 3 MXFP4.  CHANNEL: one scale per row (the
// chunk covers the row), else one per 128 elements (32 for MXFP4).
// ROW_WAIT: wait for each receive row's stores before writing the next row,
// which bounds the writes a wave keeps in flight (faster for long rows).
template <int QUANT, bool CHANNEL, int VPL, int KMAX, bool ROW_WAIT>
__device__ __forceinline__ void scatter_chunk(const DispatchArgs& a, int vbase, int NV,
                                              u32x4 (&d)[VPL], const int (&sl)[KMAX], int lane)
{
    const int K = a.K;
    if constexpr (QUANT == 0) {
        // Wait for the row once (s_waitcnt vmcnt(0), other counters left
        // alone): the stores below sit in separate branches, and without it
        // each would wait for every earlier store as well.
        __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            const int s = sl[k];
            if (s < 0) continue;
            if (s >= a.capacity) {
                if (lane == 0) atomicOr(a.flags, kFlagCapacity);
                continue;
            }
            const __amdgpu_buffer_rsrc_t r =
                row_rsrc(reinterpret_cast<char*>(a.recv) + (int64_t)s * NV * 16, NV * 16);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = vbase + kWave * i;
                if (v < NV) __builtin_amdgcn_raw_buffer_store_b128(d[i], r, v * 16, 0, kStoreAux);
            }
            if constexpr (ROW_WAIT) __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    } else if constexpr (QUANT == 3) {
        // MXFP4: 32 elements = 4 lanes x one vector share an E8M0 scale
        uint32_t code[VPL];
        uint32_t sbyte[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const float m = group_max<4>(absmax8(d[i]));
            const int sx = mx_shared_exp(m);
            const float mul = __uint_as_float((uint32_t)(127 - sx) << 23);   // 2^-sx, exact
            uint32_t w = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w |= e2m1_code(bf16_lo(d[i][j]) * mul) << (8 * j);
                w |= e2m1_code(bf16_hi(d[i][j]) * mul) << (8 * j + 4);
            }
            code[i] = w;
            sbyte[i] = (uint32_t)(sx + 127);
        }
        // 16-byte code stores: the quad of lanes holding a group's 4 vectors
        // holds its 16 code bytes; quad lane q gathers the quad's codes of
        // slot q (four DPP broadcasts per slot) and stores them at once
        const int q = lane & 3;
        u32x4 pk = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const u32x4 g = {quad_bcast<0>(code[i]), quad_bcast<1>(code[i]), quad_bcast<2>(code[i]),
                             quad_bcast<3>(code[i])};
            if (q == i) pk = g;
        }
        const int vq = vbase - q + kWave * q;      // first vector of the group lane q stores
        const bool quad_store = q < VPL && vq < NV;
        const int G = NV / 4;
        // Scale bytes: slot i's 16 groups (one per quad) are 16 consecutive
        // bytes; lane i gathers them (16 shuffles from the quads' lane i) and
        // stores them at once, when the rows' scale bytes sit on 16-byte
        // boundaries (H a multiple of 512, an aligned scales array) and the
        // wave's groups fill the 16; otherwise each quad stores its byte.
        const int g0 = (vbase - lane) / 4;          // the wave's first group
        const bool wide_scales = G % 16 == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15) == 0;
        u32x4 sb = {0u, 0u, 0u, 0u};
        if (wide_scales) {
            const uint32_t mine = sbyte[q < VPL ? q : VPL - 1];
#pragma unroll
            for (int Q = 0; Q < 16; ++Q) {
                const uint32_t b = (uint32_t)__shfl((int)mine, 4 * Q + q);
                sb[Q / 4] |= b << (8 * (Q % 4));
            }
        }
        const int gs = g0 + 16 * q;                 // first group of lane q's slot
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            const int s = sl[k];
            if (s < 0) continue;
            if (s >= a.capacity) {
                if (lane == 0) atomicOr(a.flags, kFlagCapacity);
                continue;
            }
            const __amdgpu_buffer_rsrc_t r =
                row_rsrc(reinterpret_cast<char*>(a.recv) + (int64_t)s * NV * 4, NV * 4);
            uint8_t* srow = reinterpret_cast<uint8_t*>(a.scales) + (int64_t)s * G;
            if (quad_store) __builtin_amdgcn_raw_buffer_store_b128(pk, r, vq * 4, 0, kStoreAux);
            if (wide_scales) {
                if (lane < VPL && gs + 16 <= G) *reinterpret_cast<u32x4*>(srow + gs) = sb;
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int v = vbase + kWave * i;
                    if (v < NV && q == 0) srow[v / 4] = (uint8_t)sbyte[i];
                }
            }
            if constexpr (ROW_WAIT) __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    } else {
        constexpr float kQ = (QUANT == 1) ? 448.0f : 127.0f;
        float amax[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) amax[i] = absmax8(d[i]);
        const bool pow2 = a.scale_mode != 0;
        float scale[VPL];
        if constexpr (CHANNEL) {
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) m = fmaxf(m, amax[i]);
            m = group_max<kWave>(m);
            float sc = fmaxf(m, 1e-4f) / kQ;
            if (pow2) sc = pow2_ceil(sc);
#pragma unroll
            for (int i = 0; i < VPL; ++i) scale[i] = sc;
        } else {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                scale[i] = fmaxf(group_max<16>(amax[i]), 1e-4f) / kQ;
                if (pow2) scale[i] = pow2_ceil(scale[i]);
            }
        }
        u32x2 code[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const float rs = 1.0f / scale[i];
            float q[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                q[2 * j] = div_shared(bf16_lo(d[i][j]), scale[i], rs);
                q[2 * j + 1] = div_shared(bf16_hi(d[i][j]), scale[i], rs);
            }
            if constexpr (QUANT == 1) {
                code[i] = u32x2{pack_fp8x4(q[0], q[1], q[2], q[3]), pack_fp8x4(q[4], q[5], q[6], q[7])};
            } else {
                code[i] = u32x2{pack_int8x4(q[0], q[1], q[2], q[3]), pack_int8x4(q[4], q[5], q[6], q[7])};
            }
        }
        // 16-byte code stores: adjacent lanes hold adjacent vectors, whose 16
        // codes are contiguous.  For each pair of slots (i, i+1) the even lane
        // stores the pair's codes of slot i and the odd lane those of slot
        // i+1, after one DPP swap of the halves each needs; a lone last slot
        // (VPL odd) is stored by the even lanes.
        constexpr int NP = (VPL + 1) / 2;
        const bool odd = lane & 1;
        u32x4 pk[NP];
        int pv[NP];   // first vector of the pair the lane stores (-1: none)
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int i0 = 2 * p, i1 = 2 * p + 1;
            if (i1 < VPL) {
                const u32x2 send = odd ? code[i0] : code[i1];
                const u32x2 recv = {swap_pair(send[0]), swap_pair(send[1])};
                pk[p] = odd ? u32x4{recv[0], recv[1], code[i1][0], code[i1][1]}
                            : u32x4{code[i0][0], code[i0][1], recv[0], recv[1]};
                pv[p] = vbase - (lane & 1) + kWave * (odd ? i1 : i0);
            } else {
                const u32x2 recv = {swap_pair(code[i0][0]), swap_pair(code[i0][1])};
                pk[p] = u32x4{code[i0][0], code[i0][1], recv[0], recv[1]};
                pv[p] = odd ? -1 : vbase + kWave * i0;
            }
        }
        const int G = CHANNEL ? 1 : NV / 16;
        const bool byte_scales = a.scale_mode == 2;
        // Group scales: slot i's 4 groups (16 lanes each) hold consecutive
        // scales; lane i gathers them (4 shuffles) and stores 16 bytes (fp32)
        // or 4 (E8M0) at once when the rows' scales sit on those boundaries
        // (H a multiple of 512, an aligned scales array).
        const int g0 = (vbase - lane) / 16;         // the wave's first group
        const bool wide_scales =
            !CHANNEL && G % 4 == 0 &&
            (reinterpret_cast<uintptr_t>(a.scales) & (byte_scales ? 3 : 15)) == 0;
        u32x4 sw = {0u, 0u, 0u, 0u};
        if (wide_scales) {
            const int li = lane & 15;
            const float mine = scale[li < VPL ? li : VPL - 1];
            const uint32_t bits = byte_scales ? (uint32_t)e8m0_of_pow2(mine) : __float_as_uint(mine);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t b = (uint32_t)__shfl((int)bits, 16 * j + li);
                if (byte_scales) sw[0] |= b << (8 * j);
                else sw[j] = b;
            }
        }
        const int gs = g0 + 4 * (lane & 15);        // first group of lane i's slot
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            const int s = sl[k];
            if (s < 0) continue;
            if (s >= a.capacity) {
                if (lane == 0) atomicOr(a.flags, kFlagCapacity);
                continue;
            }
            const __amdgpu_buffer_rsrc_t r =
                row_rsrc(reinterpret_cast<char*>(a.recv) + (int64_t)s * NV * 8, NV * 8);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int v = pv[p];
                // a row of odd length (per-row scales) ends in half a pair
                if (v >= 0 && v + 1 < NV)
                    __builtin_amdgcn_raw_buffer_store_b128(pk[p], r, v * 8, 0, kStoreAux);
                else if (v >= 0 && v < NV)
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pk[p][0], pk[p][1]}, r, v * 8, 0,
                                                         kStoreAux);
            }
            if (wide_scales) {
                if (lane < VPL && gs < G) {
                    const int64_t at = (int64_t)s * G + gs;
                    if (byte_scales) reinterpret_cast<uint32_t*>(a.scales)[at / 4] = sw[0];
                    else *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(a.scales) + at) = sw;
                }
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int v = vbase + kWave * i;
                    const bool writer = CHANNEL ? v == 0 : (lane & 15) == 0;
                    if (v < NV && writer) {
                        const int64_t at = (int64_t)s * G + (CHANNEL ? 0 : v / 16);
                        if (byte_scales)
                            reinterpret_cast<uint8_t*>(a.scales)[at] = e8m0_of_pow2(scale[i]);
                        else
                            reinterpret_cast<float*>(a.scales)[at] = scale[i];
                    }
                }
            }
            if constexpr (ROW_WAIT) __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    }
}

// One wave's share of the dispatch: block `block` of a launch with WPB waves
// per block; wave item -> (token, column chunk of VPL vectors per lane).
template <int QUANT, bool CHANNEL, int VPL, int KMAX, bool ROW_WAIT, int WPB>
__device__ __forceinline__ void dispatch_wave(const DispatchArgs& a, int NV, int NC, int block)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int item = block * WPB + wv;
    const int64_t t = a.t_begin + item / NC;
    const int c = item % NC;
    if (t >= a.t_end) return;
    const int vbase = c * (kWave * VPL) + lane;
    u32x4 d[VPL];
    load_chunk<VPL>(a, t, vbase, NV, d);
    // the token's slots as one batch of scalar loads (the slot array carries
    // kMaxTopk words of slack, so reading KMAX words is in bounds; words past
    // K are ignored)
    int sl[KMAX];
    if (a.identity) {   // row quantisation: row t to receive row t
#pragma unroll
        for (int k = 0; k < KMAX; ++k) sl[k] = k == 0 ? (int)t : -1;
    } else {
        const int32_t* srow = a.slot_idx + t * a.K;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) sl[k] = srow[k];
    }
    scatter_chunk<QUANT, CHANNEL, VPL, KMAX, ROW_WAIT>(a, vbase, NV, d, sl, lane);
}

}  // namespace scatter
}  // namespace epk
