// Combine on gfx950 (a4): gather each token's top-k expert outputs back to
// source order and reduce them with the routing weights.
//
// What is computed ("A2_DEEPEP.md" API table: combine is the paired inverse
// of dispatch; the reduction is weighted by topk_weights):
//   out[t] = bf16_rne( sum over k, ascending, with slot(t,k) >= 0 of
//                      w[t,k] * y[slot(t,k)] )
// accumulated in fp32 with fused multiply-add, one rounding to bf16 at the
// end (v_cvt_pk_bf16_f32).  y may also arrive quantised (Aliyun "DeepEP
// 通信库使用指南（v2.1）": combine int8 / fp8 from v2.1, quant_size 128 or
// hidden): element = code * scale in fp32, then the same reduction.
//
// Design: one wavefront per (token, column chunk) of VPL 16-byte vectors per
// lane.  All K gathers of the chunk are issued before the arithmetic so each
// wave keeps K*VPL 16-byte loads in flight; the output is one 16-byte store
// per vector.  No atomics: each output element is owned by one lane.
// HBM-bound (K rows read per row written).
#include "gather.hpp"

// Launch shape: 16-byte vectors per lane per wave; threads per block for
// large launches (at least EP_COMBINE_BIG_ITEMS waves) and for small ones;
// whether y loads / out stores carry the non-temporal hint.  Measured on
// MI355X: 512-thread blocks take the Qwen3-shape combine from 26.7 to 25.8
// us, but a 128-token decode batch (896 waves) runs faster on more, smaller
// blocks.
#ifndef EP_COMBINE_VPL
#define EP_COMBINE_VPL 2
#endif
#ifndef EP_COMBINE_BLOCK
#define EP_COMBINE_BLOCK 512
#endif
#ifndef EP_COMBINE_SMALL_BLOCK
#define EP_COMBINE_SMALL_BLOCK 128
#endif
#ifndef EP_COMBINE_BIG_ITEMS
#define EP_COMBINE_BIG_ITEMS 8192
#endif

namespace epk {

namespace {

using namespace gather;

template <int KMAX, int VPL, int YQ, bool YCH, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_combine(CombineArgs a, int NV, int NC)
{
    combine_wave<KMAX, VPL, YQ, YCH, BLOCK / kWave>(a, NV, NC, blockIdx.x);
}

// Small launches (decode batches) take one vector per lane: twice the waves,
// each with half the loads in flight (measured on MI355X, decode 128 x 7168:
// 4.88 -> 4.60 us); large ones EP_COMBINE_VPL.
template <int KMAX, int VPL, int YQ, bool YCH, int B>
hipError_t launch_b(const CombineArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    const int NC = (NV + kWave * VPL - 1) / (kWave * VPL);
    const int64_t items = (a.t_end - a.t_begin) * NC;
    const int blocks = (int)((items + B / kWave - 1) / (B / kWave));
    launch_k(k_combine<KMAX, VPL, YQ, YCH, B>, dim3(blocks), dim3(B), 0, s, ev.start, ev.stop, a, NV,
             NC);
    return hipGetLastError();
}

template <int KMAX, int VPL, int YQ, bool YCH>
hipError_t launch_kv(const CombineArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    const int NC = (NV + kWave * VPL - 1) / (kWave * VPL);
    const int64_t items = (a.t_end - a.t_begin) * NC;
    if (items <= 0) return hipSuccess;
    if (items >= EP_COMBINE_BIG_ITEMS) return launch_b<KMAX, VPL, YQ, YCH, EP_COMBINE_BLOCK>(a, NV, s, ev);
    return launch_b<KMAX, 1, YQ, YCH, EP_COMBINE_SMALL_BLOCK>(a, NV, s, ev);
}

template <int YQ, bool YCH>
hipError_t launch_q(const CombineArgs& a, int NV, hipStream_t s, LaunchEvents ev)
{
    if (a.K <= 2) return launch_kv<2, EP_COMBINE_VPL, YQ, YCH>(a, NV, s, ev);
    if (a.K <= 4) return launch_kv<4, EP_COMBINE_VPL, YQ, YCH>(a, NV, s, ev);
    if (a.K <= 8) return launch_kv<8, EP_COMBINE_VPL, YQ, YCH>(a, NV, s, ev);
    return launch_kv<16, (EP_COMBINE_VPL > 1 ? EP_COMBINE_VPL / 2 : 1), YQ, YCH>(a, NV, s, ev);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s, LaunchEvents ev)
{
    const int NV = a.H / 8;
    const bool ych = a.ygroup == a.H && a.H != 128;
    switch (a.yquant) {
        case 0: return launch_q<0, false>(a, NV, s, ev);
        case 1: return ych ? launch_q<1, true>(a, NV, s, ev) : launch_q<1, false>(a, NV, s, ev);
        default: return ych ? launch_q<2, true>(a, NV, s, ev) : launch_q<2, false>(a, NV, s, ev);
    }
}

}  // namespace epk
