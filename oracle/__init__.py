"""numpy front end of the plain CPU oracle (``ep_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the product path never imports it.
It shares no code with the HIP library.

Parity status: every function is pinned by the CPU tests (see the
``test_oracle_*`` files): number formats against torch's own converters and
exhaustive format properties, layout and slots against numpy routines,
brute force and invariants, combine against exact rational sums (the fp32
chain of ``combine_fma`` step by step against exactly rounded fused
multiply-adds).

``dispatch``, ``combine*`` take ``parallel=True`` to run on the OpenMP build
(same results; for timing the oracle on a host's cores only).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_libs = {}


def lib(parallel=False):
    """The serial oracle library, or with parallel the OpenMP build."""
    L = _libs.get(parallel)
    if L is None:
        path = _build.build(force=False, openmp=parallel)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.orc_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P]
        L.orc_layout.restype = i32
        L.orc_slots.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, i64]
        L.orc_slots.restype = i64
        L.orc_slots_fixed.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P]
        L.orc_slots_fixed.restype = i64
        L.orc_slots_nonexpand.argtypes = [P, i64, i32, i32, i32, P, P, P]
        L.orc_slots_nonexpand.restype = i64
        L.orc_recv_topk.argtypes = [P, P, P, i64, i32, i32, i32, P, P]
        L.orc_recv_topk.restype = None
        L.orc_source_counts.argtypes = [P, i64, i32, i32, i32, i32, P, P]
        L.orc_source_counts.restype = i32
        L.orc_recv_list.argtypes = [P, i32, i32, i32, P]
        L.orc_recv_list.restype = None
        L.orc_dispatch.argtypes = [P, i64, i32, P, i32, i32, i32, i32, i64, i64, P, P]
        L.orc_dispatch.restype = None
        L.orc_combine_q.argtypes = [P, P, i32, i32, P, P, i64, i32, i32, i64, i64, P]
        L.orc_combine_q.restype = None
        L.orc_e2m1_from_f32.argtypes = [ctypes.c_float]
        L.orc_e2m1_from_f32.restype = ctypes.c_uint8
        L.orc_f32_from_e2m1.argtypes = [ctypes.c_uint8]
        L.orc_f32_from_e2m1.restype = ctypes.c_float
        L.orc_f32_from_e8m0.argtypes = [ctypes.c_uint8]
        L.orc_f32_from_e8m0.restype = ctypes.c_float
        L.orc_combine.argtypes = [P, P, P, i64, i32, i32, i64, i64, P]
        L.orc_combine.restype = None
        L.orc_combine_fma.argtypes = [P, P, P, i64, i32, i32, i64, i64, P]
        L.orc_combine_fma.restype = None
        L.orc_combine_q_fma.argtypes = [P, P, i32, i32, P, P, i64, i32, i32, i64, i64, P]
        L.orc_combine_q_fma.restype = None
        L.orc_recv_list_fixed.argtypes = [P, i32, i32, i32, i32, P]
        L.orc_recv_list_fixed.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = i32
        for name in ("orc_bf16_from_f32_n", "orc_bf16_from_f64_n", "orc_e4m3fn_from_f32_n",
                     "orc_f32_from_e4m3fn_n"):
            getattr(L, name).argtypes = [P, P, i64]
            getattr(L, name).restype = None
        _libs[parallel] = L
    return L


def num_threads(parallel=False):
    """Threads the per-token loops run on (1 for the serial build)."""
    return int(lib(parallel).orc_num_threads())


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# ---- number formats --------------------------------------------------------

def bf16_from_f32(v):
    v = _c(v, np.float32).ravel()
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_from_f32_n(_p(v), _p(out), v.size)
    return out


def bf16_from_f64(v):
    v = _c(v, np.float64).ravel()
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_from_f64_n(_p(v), _p(out), v.size)
    return out


def f32_from_bf16(b):
    b = _c(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3fn_from_f32(v):
    v = _c(v, np.float32).ravel()
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3fn_from_f32_n(_p(v), _p(out), v.size)
    return out


def f32_from_e4m3fn(b):
    b = _c(b, np.uint8).ravel()
    out = np.empty(b.shape, np.float32)
    lib().orc_f32_from_e4m3fn_n(_p(b), _p(out), b.size)
    return out


# ---- the four stages -------------------------------------------------------

def layout(topk_idx, num_experts, num_ranks, ranks_per_node=0):
    """a1. Returns dict(num_tokens_per_rank, num_tokens_per_rdma_rank or None,
    num_tokens_per_expert, is_token_in_rank[N,R] uint8)."""
    idx = _c(topk_idx, np.int32)
    N, K = idx.shape
    E, R = num_experts, num_ranks
    per_rank = np.zeros(R, np.int32)
    per_expert = np.zeros(E, np.int32)
    in_rank = np.zeros((N, R), np.uint8)
    nodes = (R + ranks_per_node - 1) // ranks_per_node if ranks_per_node > 0 else 0
    per_node = np.zeros(max(nodes, 1), np.int32) if nodes else None
    rc = lib().orc_layout(_p(idx), N, K, E, R, ranks_per_node, _p(per_rank), _p(per_node),
                          _p(per_expert), _p(in_rank))
    if rc != 0:
        raise ValueError("topk_idx holds an id outside [-1, num_experts)")
    return dict(num_tokens_per_rank=per_rank, num_tokens_per_rdma_rank=per_node,
                num_tokens_per_expert=per_expert, is_token_in_rank=in_rank)


def max_slots(N, K, E, A):
    """Receive rows needed in the worst case: every pair plus full padding."""
    return N * K + E * (A - 1)


def slots(topk_idx, num_experts, num_ranks, expert_alignment=1):
    """a2. Returns dict(S, psum_expert, psum_rank, num_unaligned, slot_idx[N,K],
    src_meta[S,2])."""
    idx = _c(topk_idx, np.int32)
    N, K = idx.shape
    E, R, A = num_experts, num_ranks, expert_alignment
    cap = max_slots(N, K, E, A)
    psum_e = np.zeros(E + 1, np.int32)
    psum_r = np.zeros(R + 1, np.int32)
    unal = np.zeros(E, np.int32)
    slot = np.zeros((N, K), np.int32)
    meta = np.zeros((max(cap, 1), 2), np.int32)
    S = lib().orc_slots(_p(idx), N, K, E, R, A, _p(psum_e), _p(psum_r), _p(unal), _p(slot),
                        _p(meta), cap)
    if S == -1:
        raise ValueError("topk_idx holds an id outside [-1, num_experts)")
    if S < 0:
        raise RuntimeError("receive-row capacity exceeded")
    return dict(S=int(S), psum_expert=psum_e, psum_rank=psum_r, num_unaligned=unal,
                slot_idx=slot, src_meta=meta[:S].copy())


def slots_fixed(topk_idx, num_experts, num_ranks, capacity):
    """Fixed-capacity receive layout.  Returns dict(S = E*capacity,
    dropped, psum_expert, psum_rank, num_unaligned, slot_idx, src_meta)."""
    idx = _c(topk_idx, np.int32)
    N, K = idx.shape
    E, R = num_experts, num_ranks
    psum_e = np.zeros(E + 1, np.int32)
    psum_r = np.zeros(R + 1, np.int32)
    unal = np.zeros(E, np.int32)
    slot = np.zeros((N, K), np.int32)
    meta = np.zeros((max(E * capacity, 1), 2), np.int32)
    d = lib().orc_slots_fixed(_p(idx), N, K, E, R, capacity, _p(psum_e), _p(psum_r), _p(unal),
                              _p(slot), _p(meta))
    if d < 0:
        raise ValueError("topk_idx holds an id outside [-1, num_experts)")
    return dict(S=E * capacity, dropped=int(d), psum_expert=psum_e, psum_rank=psum_r,
                num_unaligned=unal, slot_idx=slot, src_meta=meta[:E * capacity].copy())


def slots_nonexpand(topk_idx, num_experts, num_ranks):
    """Non-expand layout: dict(S = rows, psum_rank [R+1], slot_idx [N,K],
    src_meta [S,2])."""
    idx = _c(topk_idx, np.int32)
    N, K = idx.shape
    psum_r = np.zeros(num_ranks + 1, np.int32)
    slot = np.zeros((N, K), np.int32)
    meta = np.zeros((max(N * min(K, num_ranks), 1), 2), np.int32)
    S = lib().orc_slots_nonexpand(_p(idx), N, K, num_experts, num_ranks, _p(psum_r), _p(slot),
                                  _p(meta))
    if S < 0:
        raise ValueError("topk_idx holds an id outside [-1, num_experts)")
    return dict(S=int(S), psum_rank=psum_r, slot_idx=slot, src_meta=meta[:S].copy())


def recv_topk(topk_idx, topk_weights, src_meta, num_experts, num_ranks):
    """recv_topk_idx int32 [rows,K] and recv_topk_weights fp32 [rows,K] of
    the non-expand layout."""
    idx = _c(topk_idx, np.int32)
    w = _c(topk_weights, np.float32)
    meta = _c(src_meta, np.int32)
    rows, K = meta.shape[0], idx.shape[1]
    ri = np.zeros((rows, K), np.int32)
    rw = np.zeros((rows, K), np.float32)
    lib().orc_recv_topk(_p(idx), _p(w), _p(meta), rows, K, num_experts, num_ranks, _p(ri), _p(rw))
    return ri, rw


def source_counts(topk_idx, num_experts, num_ranks, num_sources):
    """Per-source receive quantities of a batch of num_sources stacked source
    ranks.  Returns dict(psum_source_rank [R, P+1], expert_source_base [P, E])."""
    idx = _c(topk_idx, np.int32)
    N, K = idx.shape
    E, R, P = num_experts, num_ranks, num_sources
    psr = np.zeros((R, P + 1), np.int32)
    base = np.zeros((P, E), np.int32)
    rc = lib().orc_source_counts(_p(idx), N, K, E, R, P, _p(psr), _p(base))
    if rc == -1:
        raise ValueError("topk_idx holds an id outside [-1, num_experts)")
    if rc != 0:
        raise ValueError("num_tokens must be a multiple of num_sources")
    return dict(psum_source_rank=psr, expert_source_base=base)


def recv_list(psum_expert, num_experts, num_ranks, counts_as_prefix):
    pe = _c(psum_expert, np.int32)
    out = np.zeros(num_experts, np.int32)
    lib().orc_recv_list(_p(pe), num_experts, num_ranks, int(bool(counts_as_prefix)), _p(out))
    return out


def recv_list_fixed(num_unaligned, num_experts, num_ranks, capacity, counts_as_prefix):
    """Host list of the fixed-capacity layout: min(count, capacity) per
    expert, or its inclusive prefix restarting per rank."""
    cnt = _c(num_unaligned, np.int32)
    out = np.zeros(num_experts, np.int32)
    lib().orc_recv_list_fixed(_p(cnt), num_experts, num_ranks, capacity,
                              int(bool(counts_as_prefix)), _p(out))
    return out


QUANT_NONE, QUANT_FP8, QUANT_INT8, QUANT_MXFP4 = 0, 1, 2, 3
SCALE_FP32, SCALE_POW2, SCALE_UE8M0 = 0, 1, 2


def e2m1_from_f32(v):
    return np.array([lib().orc_e2m1_from_f32(float(a)) for a in np.ravel(v)], np.uint8)


def f32_from_e2m1(c):
    return np.array([lib().orc_f32_from_e2m1(int(a)) for a in np.ravel(c)], np.float32)


def f32_from_e8m0(b):
    return np.array([lib().orc_f32_from_e8m0(int(a)) for a in np.ravel(b)], np.float32)


def row_bytes(H, quant):
    return 2 * H if quant == QUANT_NONE else (H // 2 if quant == QUANT_MXFP4 else H)


def scale_dtype(quant, scale_mode):
    return np.uint8 if quant == QUANT_MXFP4 or scale_mode == SCALE_UE8M0 else np.float32


def dispatch(x_bits, slot_idx, num_rows, quant=QUANT_NONE, group=None, t_begin=0, t_end=None,
             recv_x=None, recv_scales=None, scale_mode=SCALE_FP32, parallel=False):
    """a3. x_bits: uint16 [N,H] bf16 bit patterns.  Returns (recv_x, recv_scales):
    bf16 bits, or code bytes [rows, H] (FP8 / int8) or [rows, H/2] (MXFP4); scales
    fp32 or E8M0 bytes [rows, G]."""
    x = _c(x_bits, np.uint16)
    sl = _c(slot_idx, np.int32)
    N, H = x.shape
    K = sl.shape[1]
    t_end = N if t_end is None else t_end
    if quant == QUANT_NONE:
        group = H
        if recv_x is None:
            recv_x = np.zeros((num_rows, H), np.uint16)
    else:
        group = 32 if quant == QUANT_MXFP4 else (H if group is None else group)
        G = H // group
        if recv_x is None:
            cdt = np.int8 if quant == QUANT_INT8 else np.uint8
            recv_x = np.zeros((num_rows, row_bytes(H, quant)), cdt)
        if recv_scales is None:
            recv_scales = np.zeros((num_rows, G), scale_dtype(quant, scale_mode))
    assert recv_x.flags.c_contiguous
    lib(parallel).orc_dispatch(_p(x), N, H, _p(sl), K, quant, group, scale_mode, t_begin, t_end,
                       _p(recv_x), _p(recv_scales))
    return recv_x, recv_scales


def quantize_rows(x_bits, quant, group=None, scale_mode=SCALE_FP32):
    """Quantises every row on its own (dispatch with row t sent to receive row t)."""
    x = _c(x_bits, np.uint16)
    ident = np.arange(x.shape[0], dtype=np.int32)[:, None]
    return dispatch(x, ident, x.shape[0], quant=quant, group=group, scale_mode=scale_mode)


def combine_q(y_codes, y_scales, quant, group, topk_weights, slot_idx, t_begin=0, t_end=None,
              out=None, fp32=False, parallel=False):
    """a4 over quantised expert outputs: y_codes [S,H] (E4M3FN bytes or int8),
    y_scales fp32 [S, H/group].  Returns uint16 bf16 bits [N,H]: the exact sum
    rounded once, or with fp32 the fp32 fused multiply-add chain."""
    yc = _c(y_codes, np.uint8 if quant == QUANT_FP8 else np.int8)
    ys = _c(y_scales, np.float32)
    w = _c(topk_weights, np.float32)
    sl = _c(slot_idx, np.int32)
    N, K = sl.shape
    H = yc.shape[1]
    t_end = N if t_end is None else t_end
    if out is None:
        out = np.zeros((N, H), np.uint16)
    L = lib(parallel)
    fn = L.orc_combine_q_fma if fp32 else L.orc_combine_q
    fn(_p(yc), _p(ys), quant, group, _p(w), _p(sl), N, K, H, t_begin, t_end, _p(out))
    return out


def combine(y_bits, topk_weights, slot_idx, t_begin=0, t_end=None, out=None, fp32=False,
            parallel=False):
    """a4. y_bits uint16 [S,H]; topk_weights fp32 [N,K].  Returns uint16 [N,H]:
    the exact weighted sum rounded once to bf16, or with fp32 the fp32 fused
    multiply-add chain over k ascending (combine_fma)."""
    y = _c(y_bits, np.uint16)
    w = _c(topk_weights, np.float32)
    sl = _c(slot_idx, np.int32)
    N, K = sl.shape
    H = y.shape[1]
    t_end = N if t_end is None else t_end
    if out is None:
        out = np.zeros((N, H), np.uint16)
    assert out.flags.c_contiguous
    L = lib(parallel)
    fn = L.orc_combine_fma if fp32 else L.orc_combine
    fn(_p(y), _p(w), _p(sl), N, K, H, t_begin, t_end, _p(out))
    return out


def combine_fma(y_bits, topk_weights, slot_idx, **kw):
    """The combine in fp32: k ascending, one fused multiply-add per term."""
    return combine(y_bits, topk_weights, slot_idx, fp32=True, **kw)


def combine_q_fma(y_codes, y_scales, quant, group, topk_weights, slot_idx, **kw):
    return combine_q(y_codes, y_scales, quant, group, topk_weights, slot_idx, fp32=True, **kw)
