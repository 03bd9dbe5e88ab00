"""Thin Python binding of libep_amd.so (include/ep.h), over torch tensors.

Argument marshalling only: every stage runs in the HIP kernels of the
library.  torch supplies device memory and the current HIP stream.  The
functions carry the C names; each returns what the C call writes.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_amd.so")

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_WORKSPACE, EP_ERR_CAPACITY, EP_ERR_DEVICE_INDEX, EP_ERR_HIP, \
    EP_ERR_STATE = range(7)
EP_QUANT_NONE, EP_QUANT_FP8_E4M3, EP_QUANT_INT8, EP_QUANT_MXFP4 = 0, 1, 2, 3
EP_SCALE_FP32, EP_SCALE_POW2, EP_SCALE_UE8M0 = 0, 1, 2
EP_FLAG_BAD_EXPERT_ID, EP_FLAG_RECV_CAPACITY, EP_FLAG_Y_ROWS = 1, 2, 4

# Every symbol include/ep.h declares.
SYMBOLS = ("ep_workspace_size", "ep_recv_capacity", "ep_handle_init", "ep_handle_init_static",
           "ep_handle_free",
           "ep_get_layout", "ep_dispatch", "ep_layout_dispatch", "ep_dispatch_topk",
           "ep_combine", "ep_dispatch_overlap", "ep_combine_overlap", "ep_quantize_rows",
           "ep_set_kernel_events", "ep_handle_view", "ep_handle_get_view", "ep_check_error",
           "ep_status_str", "ep_last_error_message")


class ep_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_topk", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_ranks", ctypes.c_int32),
                ("ranks_per_node", ctypes.c_int32), ("expert_alignment", ctypes.c_int32),
                ("quant", ctypes.c_int32), ("quant_group", ctypes.c_int32),
                ("counts_as_prefix", ctypes.c_int32), ("expert_capacity", ctypes.c_int32),
                ("num_sources", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("combine_quant", ctypes.c_int32), ("combine_group", ctypes.c_int32),
                ("non_expand", ctypes.c_int32)]


class ep_handle_view_t(ctypes.Structure):
    _fields_ = [("psum_expert", ctypes.c_void_p), ("psum_rank", ctypes.c_void_p),
                ("num_unaligned", ctypes.c_void_p), ("slot_idx", ctypes.c_void_p),
                ("src_meta", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int64), ("max_tokens", ctypes.c_int64),
                ("max_slots", ctypes.c_int64), ("num_recv_slots", ctypes.c_int64),
                ("num_sources", ctypes.c_int64), ("psum_source_rank", ctypes.c_void_p),
                ("expert_source_base", ctypes.c_void_p)]


class EpError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built (there is no
    fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.ep_workspace_size.argtypes = [P, I64, P]
        L.ep_recv_capacity.argtypes = [P, I64, P]
        L.ep_handle_init.argtypes = [P, I64, P, I64, P, P]
        L.ep_handle_init_static.argtypes = [P, I64, P, P]
        L.ep_handle_free.argtypes = [P]
        L.ep_handle_free.restype = None
        L.ep_get_layout.argtypes = [P, P, I64, P, P, P, P, I32, P, P, P]
        L.ep_dispatch.argtypes = [P, P, I64, I64, P, P, I64, P]
        L.ep_layout_dispatch.argtypes = [P, P, I64, P, P, P, P, P, P, P, I64, P]
        L.ep_combine.argtypes = [P, P, P, I64, P, I64, I64, P, P]
        L.ep_quantize_rows.argtypes = [P, P, I64, P, P, P]
        L.ep_dispatch_topk.argtypes = [P, P, I64, I64, P, P, I64, P]
        L.ep_dispatch_overlap.argtypes = [P, P, I64, I64, P, P, I64, P, P, I64, P, P, P, P, P]
        L.ep_combine_overlap.argtypes = [P, P, P, I64, P, I64, I64, P, P, P]
        L.ep_set_kernel_events.argtypes = [P, P, P]
        L.ep_handle_view.argtypes = [P, P]
        L.ep_handle_get_view.argtypes = [P, P]
        L.ep_check_error.argtypes = [P, P, P]
        L.ep_status_str.argtypes = [I32]
        L.ep_status_str.restype = ctypes.c_char_p
        L.ep_last_error_message.argtypes = []
        L.ep_last_error_message.restype = ctypes.c_char_p
        for name in ("ep_workspace_size", "ep_recv_capacity", "ep_handle_init",
                     "ep_handle_init_static", "ep_get_layout",
                     "ep_dispatch", "ep_layout_dispatch", "ep_combine", "ep_quantize_rows",
                     "ep_dispatch_topk", "ep_dispatch_overlap", "ep_combine_overlap",
                     "ep_set_kernel_events", "ep_handle_view", "ep_handle_get_view",
                     "ep_check_error"):
            getattr(L, name).restype = I32
        _lib = L
    return _lib


def status_name(st):
    return lib().ep_status_str(st).decode()


def _check(st):
    if st != EP_OK:
        raise EpError(st, lib().ep_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("tensors passed to the library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class Config:
    hidden: int
    num_topk: int
    num_experts: int
    num_ranks: int
    ranks_per_node: int = 0
    expert_alignment: int = 1
    quant: int = EP_QUANT_NONE
    quant_group: int = 0
    counts_as_prefix: bool = False
    expert_capacity: int = 0
    num_sources: int = 1
    scale_mode: int = EP_SCALE_FP32
    combine_quant: int = EP_QUANT_NONE
    combine_group: int = 0
    non_expand: bool = False

    def c(self):
        return ep_config(self.hidden, self.num_topk, self.num_experts, self.num_ranks,
                         self.ranks_per_node, self.expert_alignment, self.quant, self.quant_group,
                         int(bool(self.counts_as_prefix)), self.expert_capacity, self.num_sources,
                         self.scale_mode, self.combine_quant, self.combine_group,
                         int(bool(self.non_expand)))

    @property
    def num_nodes(self):
        return -(-self.num_ranks // self.ranks_per_node) if self.ranks_per_node > 0 else 0

    @property
    def num_groups(self):
        return self.hidden // self.quant_group if self.quant else 0

    @property
    def recv_row_elems(self):
        """Elements (bytes for codes) of one receive row."""
        return self.hidden // 2 if self.quant == EP_QUANT_MXFP4 else self.hidden

    @property
    def recv_dtype(self):
        return {EP_QUANT_NONE: torch.bfloat16, EP_QUANT_FP8_E4M3: torch.uint8,
                EP_QUANT_INT8: torch.int8, EP_QUANT_MXFP4: torch.uint8}[self.quant]

    @property
    def scales_dtype(self):
        if self.quant == EP_QUANT_MXFP4 or self.scale_mode == EP_SCALE_UE8M0:
            return torch.uint8
        return torch.float32


def ep_workspace_size(cfg: Config, max_tokens: int) -> int:
    out = ctypes.c_int64()
    c = cfg.c()
    _check(lib().ep_workspace_size(ctypes.byref(c), max_tokens, ctypes.byref(out)))
    return out.value


def ep_recv_capacity(cfg: Config, num_tokens: int) -> int:
    out = ctypes.c_int64()
    c = cfg.c()
    _check(lib().ep_recv_capacity(ctypes.byref(c), num_tokens, ctypes.byref(out)))
    return out.value


class Handle:
    """Owns the C handle and keeps its workspace tensor alive (None for the
    library's static handle, whose workspace is the library's own)."""

    def __init__(self, cfg: Config, max_tokens: int, workspace: Optional[torch.Tensor], ptr: int,
                 device=None):
        self.cfg = cfg
        self.max_tokens = max_tokens
        self.workspace = workspace
        self._device = workspace.device if workspace is not None else torch.device(device)
        self._ptr = ctypes.c_void_p(ptr)

    @property
    def device(self):
        return self._device

    @property
    def ptr(self):
        if not self._ptr:
            raise RuntimeError("handle was freed")
        return self._ptr

    def free(self):
        if self._ptr:
            lib().ep_handle_free(self._ptr)
            self._ptr = ctypes.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def ep_handle_init(cfg: Config, max_tokens: int, workspace: Optional[torch.Tensor] = None,
                   device="cuda") -> Handle:
    """Creates a handle; allocates the workspace with torch when none is
    passed (uint8, on `device`)."""
    nbytes = ep_workspace_size(cfg, max_tokens)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    out = ctypes.c_void_p()
    c = cfg.c()
    _check(lib().ep_handle_init(ctypes.byref(c), max_tokens, _ptr(workspace),
                                workspace.numel() * workspace.element_size(),
                                _stream(workspace.device), ctypes.byref(out)))
    return Handle(cfg, max_tokens, workspace, out.value)


def ep_handle_init_static(cfg: Config, max_tokens: int, device="cuda") -> Handle:
    """The handle whose workspace is the library's static device array (one
    per GPU; allocates nothing).  Every call on a device returns the same C
    handle, set up again: the previous one's layout is gone."""
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    out = ctypes.c_void_p()
    c = cfg.c()
    with torch.cuda.device(dev):
        _check(lib().ep_handle_init_static(ctypes.byref(c), max_tokens, _stream(dev),
                                           ctypes.byref(out)))
    return Handle(cfg, max_tokens, None, out.value, device=dev)


def ep_handle_free(h: Handle):
    h.free()


def _check_tensor(name, t, dtypes, shape, device):
    """t must have one of dtypes, exactly `shape`, and live on `device`."""
    if t is None:
        return
    if t.dtype not in dtypes or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError(f"{name} must be {'/'.join(map(str, dtypes))} {list(shape)} on {device} "
                         f"(got {t.dtype} {list(t.shape)} on {t.device})")


def _layout_outputs(cfg, topk_idx, per_rank, per_rdma, per_expert, in_rank, alloc):
    if (topk_idx is None or topk_idx.dtype != torch.int32 or topk_idx.dim() != 2
            or topk_idx.shape[1] != cfg.num_topk):
        raise ValueError("topk_idx must be int32 [N, num_topk]")
    N = topk_idx.shape[0]
    dev = topk_idx.device
    if alloc:
        if per_rank is None:
            per_rank = torch.empty(cfg.num_ranks, dtype=torch.int32, device=dev)
        if per_expert is None:
            per_expert = torch.empty(cfg.num_experts, dtype=torch.int32, device=dev)
        if in_rank is None:
            in_rank = torch.empty((N, cfg.num_ranks), dtype=torch.bool, device=dev)
        if per_rdma is None and cfg.num_nodes:
            per_rdma = torch.empty(cfg.num_nodes, dtype=torch.int32, device=dev)
    # caller-supplied outputs: the library writes exactly these extents
    _check_tensor("num_tokens_per_rank", per_rank, (torch.int32,), (cfg.num_ranks,), dev)
    _check_tensor("num_tokens_per_expert", per_expert, (torch.int32,), (cfg.num_experts,), dev)
    _check_tensor("is_token_in_rank", in_rank, (torch.bool, torch.uint8), (N, cfg.num_ranks), dev)
    if per_rdma is not None:
        if not cfg.num_nodes:
            raise ValueError("num_tokens_per_rdma_rank needs ranks_per_node > 0")
        _check_tensor("num_tokens_per_rdma_rank", per_rdma, (torch.int32,), (cfg.num_nodes,), dev)
    return per_rank, per_rdma, per_expert, in_rank


def _check_dispatch_tensors(cfg, x, recv_x, recv_scales, token_begin=0, token_end=None):
    """Dtypes and shapes of a dispatch's tensors; returns the token range
    (token_end defaults to the rows of x)."""
    if x is None or x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != cfg.hidden:
        raise ValueError("x must be bf16 [N, hidden]")
    want = {EP_QUANT_NONE: (torch.bfloat16,), EP_QUANT_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn),
            EP_QUANT_INT8: (torch.int8,), EP_QUANT_MXFP4: (torch.uint8,)}[cfg.quant]
    if (recv_x is None or recv_x.dtype not in want or recv_x.dim() != 2
            or recv_x.shape[1] != cfg.recv_row_elems):
        raise ValueError(f"recv_x must be {want} [rows, {cfg.recv_row_elems}]")
    if cfg.quant:
        if (recv_scales is None or recv_scales.dtype != cfg.scales_dtype
                or recv_scales.shape != (recv_x.shape[0], cfg.num_groups)):
            raise ValueError(f"recv_scales must be {cfg.scales_dtype} [rows, hidden/quant_group]")
    elif recv_scales is not None:
        raise ValueError("recv_scales must be None without quantisation")
    if recv_x.device != x.device or (recv_scales is not None and recv_scales.device != x.device):
        raise ValueError("x, recv_x and recv_scales must be on one device")
    token_end = x.shape[0] if token_end is None else token_end
    if not 0 <= token_begin <= token_end <= x.shape[0]:
        raise ValueError("token range outside x")
    return token_begin, token_end


def ep_get_layout(h: Handle, topk_idx: torch.Tensor, num_tokens_per_rank=None,
                  num_tokens_per_rdma_rank=None, num_tokens_per_expert=None,
                  is_token_in_rank=None, do_cpu_sync=False, alloc_outputs=True):
    """a1 + a2.  topk_idx: int32 [N,K] on the device.  Outputs are allocated
    (torch.empty) when not given and alloc_outputs is set.  Returns a dict of
    the outputs; with do_cpu_sync also the host list and S."""
    cfg = h.cfg
    num_tokens_per_rank, num_tokens_per_rdma_rank, num_tokens_per_expert, is_token_in_rank = \
        _layout_outputs(cfg, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                        num_tokens_per_expert, is_token_in_rank, alloc_outputs)
    N = topk_idx.shape[0]
    dev = topk_idx.device
    host_list = None
    S = ctypes.c_int64(-1)
    if do_cpu_sync:
        host_list = (ctypes.c_int32 * cfg.num_experts)()
    _check(lib().ep_get_layout(h.ptr, _ptr(topk_idx), N, _ptr(num_tokens_per_rank),
                               _ptr(num_tokens_per_rdma_rank), _ptr(num_tokens_per_expert),
                               _ptr(is_token_in_rank), int(bool(do_cpu_sync)),
                               host_list, ctypes.byref(S) if do_cpu_sync else None,
                               _stream(dev)))
    out = dict(num_tokens_per_rank=num_tokens_per_rank,
               num_tokens_per_rdma_rank=num_tokens_per_rdma_rank,
               num_tokens_per_expert=num_tokens_per_expert, is_token_in_rank=is_token_in_rank)
    if do_cpu_sync:
        out["num_recv_tokens_per_expert_list"] = list(host_list)
        out["num_recv_slots"] = S.value
    return out


def ep_dispatch(h: Handle, x: torch.Tensor, recv_x: torch.Tensor,
                recv_scales: Optional[torch.Tensor] = None, token_begin=0, token_end=None):
    """a3.  x bf16 [N,H]; recv_x [rows,H] bf16 / uint8 (E4M3FN) / int8;
    recv_scales fp32 [rows,G] when quantised."""
    token_begin, token_end = _check_dispatch_tensors(h.cfg, x, recv_x, recv_scales, token_begin,
                                                     token_end)
    _check(lib().ep_dispatch(h.ptr, _ptr(x), token_begin, token_end, _ptr(recv_x),
                             _ptr(recv_scales), recv_x.shape[0], _stream(x.device)))
    return recv_x, recv_scales


def ep_layout_dispatch(h: Handle, topk_idx: torch.Tensor, x: torch.Tensor, recv_x: torch.Tensor,
                       recv_scales: Optional[torch.Tensor] = None, num_tokens_per_rank=None,
                       num_tokens_per_rdma_rank=None, num_tokens_per_expert=None,
                       is_token_in_rank=None, alloc_outputs=True):
    """a1 + a2 + a3 in one call, no host sync.  Same arguments as
    ep_get_layout and ep_dispatch over the whole batch.  Returns the layout
    outputs dict; recv_x / recv_scales are filled in place."""
    cfg = h.cfg
    outs = _layout_outputs(cfg, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                           num_tokens_per_expert, is_token_in_rank, alloc_outputs)
    _check_dispatch_tensors(cfg, x, recv_x, recv_scales)
    if x.shape[0] != topk_idx.shape[0] or x.device != topk_idx.device:
        raise ValueError("x and topk_idx disagree on the number of tokens or the device")
    _check(lib().ep_layout_dispatch(h.ptr, _ptr(topk_idx), topk_idx.shape[0], *map(_ptr, outs),
                                    _ptr(x), _ptr(recv_x), _ptr(recv_scales), recv_x.shape[0],
                                    _stream(x.device)))
    return dict(num_tokens_per_rank=outs[0], num_tokens_per_rdma_rank=outs[1],
                num_tokens_per_expert=outs[2], is_token_in_rank=outs[3])


def _check_y(cfg, y, y_scales):
    if cfg.combine_quant == EP_QUANT_NONE:
        if y.dtype != torch.bfloat16 or y.dim() != 2 or y.shape[1] != cfg.hidden:
            raise ValueError("y must be bf16 [rows, hidden]")
        if y_scales is not None:
            raise ValueError("y_scales must be None without combine_quant")
        return
    want = torch.int8 if cfg.combine_quant == EP_QUANT_INT8 else (torch.uint8,
                                                                   torch.float8_e4m3fn)
    want = want if isinstance(want, tuple) else (want,)
    if y.dtype not in want or y.dim() != 2 or y.shape[1] != cfg.hidden:
        raise ValueError(f"y must be {want} codes [rows, hidden]")
    G = cfg.hidden // cfg.combine_group
    if y_scales is None or y_scales.dtype != torch.float32 or y_scales.shape != (y.shape[0], G):
        raise ValueError("y_scales must be fp32 [rows, hidden/combine_group]")


def _check_combine_tensors(cfg, y, y_scales, topk_weights, out, token_begin, token_end):
    """Dtypes and shapes of a combine's tensors; returns the token range
    (token_end defaults to the rows of out).  The library reads weights and
    writes out rows [token_begin, token_end) only, so both must hold them."""
    _check_y(cfg, y, y_scales)
    if topk_weights is not None and (topk_weights.dtype != torch.float32
                                     or topk_weights.dim() != 2
                                     or topk_weights.shape[1] != cfg.num_topk):
        raise ValueError("topk_weights must be fp32 [N, num_topk] or None (weights of 1)")
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.shape[1] != cfg.hidden:
        raise ValueError("out must be bf16 [N, hidden]")
    for t in (y, y_scales, topk_weights):
        if t is not None and t.device != out.device:
            raise ValueError("y, y_scales, topk_weights and out must be on one device")
    token_end = out.shape[0] if token_end is None else token_end
    n_w = out.shape[0] if topk_weights is None else topk_weights.shape[0]
    if not 0 <= token_begin <= token_end <= min(out.shape[0], n_w):
        raise ValueError("token range outside out / topk_weights")
    return token_begin, token_end


def ep_combine(h: Handle, y: torch.Tensor, topk_weights: torch.Tensor, out: torch.Tensor,
               token_begin=0, token_end=None, y_scales: Optional[torch.Tensor] = None):
    """a4.  y bf16 [rows,H] (or codes with y_scales under combine_quant);
    topk_weights fp32 [N,K]; out bf16 [N,H]."""
    token_begin, token_end = _check_combine_tensors(h.cfg, y, y_scales, topk_weights, out,
                                                    token_begin, token_end)
    _check(lib().ep_combine(h.ptr, _ptr(y), _ptr(y_scales), y.shape[0], _ptr(topk_weights),
                            token_begin, token_end, _ptr(out), _stream(out.device)))
    return out


def ep_dispatch_overlap(h: Handle, x: torch.Tensor, recv_x: torch.Tensor,
                        recv_scales: Optional[torch.Tensor] = None, token_begin=0, token_end=None,
                        h_next: Optional[Handle] = None, topk_next: Optional[torch.Tensor] = None,
                        num_tokens_per_rank=None, num_tokens_per_rdma_rank=None,
                        num_tokens_per_expert=None, is_token_in_rank=None, alloc_outputs=True):
    """ep_dispatch of h's batch and, with h_next, the start (or all) of the
    next batch's layout in the same launch.  Returns the next batch's layout
    outputs (None without h_next); they are final after the ep_combine_overlap
    that names h_next."""
    token_begin, token_end = _check_dispatch_tensors(h.cfg, x, recv_x, recv_scales, token_begin,
                                                     token_end)
    outs = (None, None, None, None)
    n_next = 0
    if h_next is not None:
        outs = _layout_outputs(h_next.cfg, topk_next, num_tokens_per_rank,
                               num_tokens_per_rdma_rank, num_tokens_per_expert, is_token_in_rank,
                               alloc_outputs)
        n_next = topk_next.shape[0]
    _check(lib().ep_dispatch_overlap(h.ptr, _ptr(x), token_begin, token_end, _ptr(recv_x),
                                     _ptr(recv_scales), recv_x.shape[0],
                                     h_next.ptr if h_next is not None else None, _ptr(topk_next),
                                     n_next, *map(_ptr, outs), _stream(x.device)))
    if h_next is None:
        return None
    return dict(num_tokens_per_rank=outs[0], num_tokens_per_rdma_rank=outs[1],
                num_tokens_per_expert=outs[2], is_token_in_rank=outs[3])


def ep_combine_overlap(h: Handle, y: torch.Tensor, topk_weights: Optional[torch.Tensor],
                       out: torch.Tensor, token_begin=0, token_end=None,
                       y_scales: Optional[torch.Tensor] = None, h_next: Optional[Handle] = None):
    """ep_combine of h's batch and the rest of h_next's layout, if it waits."""
    token_begin, token_end = _check_combine_tensors(h.cfg, y, y_scales, topk_weights, out,
                                                    token_begin, token_end)
    _check(lib().ep_combine_overlap(h.ptr, _ptr(y), _ptr(y_scales), y.shape[0], _ptr(topk_weights),
                                    token_begin, token_end, _ptr(out),
                                    h_next.ptr if h_next is not None else None, _stream(out.device)))
    return out


def ep_dispatch_topk(h: Handle, topk_weights: Optional[torch.Tensor], recv_topk_idx=None,
                     recv_topk_weights=None, token_begin=0, token_end=None, rows=None):
    """Non-expand: per received row the local expert ids (int32 [rows, K]) and
    weights (fp32 [rows, K]).  Allocates the outputs (rows = the receive
    capacity of the handle's last batch) unless given."""
    cfg = h.cfg
    N = ep_handle_view(h)["num_tokens"]
    dev = h.device
    rows = ep_recv_capacity(cfg, N) if rows is None else rows
    if recv_topk_idx is None:
        recv_topk_idx = torch.empty((rows, cfg.num_topk), dtype=torch.int32, device=dev)
    if recv_topk_weights is None and topk_weights is not None:
        recv_topk_weights = torch.empty((rows, cfg.num_topk), dtype=torch.float32, device=dev)
    cap = recv_topk_idx.shape[0]
    _check_tensor("recv_topk_idx", recv_topk_idx, (torch.int32,), (cap, cfg.num_topk), dev)
    _check_tensor("recv_topk_weights", recv_topk_weights, (torch.float32,), (cap, cfg.num_topk),
                  dev)
    token_end = N if token_end is None else token_end
    if not 0 <= token_begin <= token_end <= N:
        raise ValueError("token range outside the handle's batch")
    if topk_weights is not None and (topk_weights.dtype != torch.float32 or topk_weights.dim() != 2
                                     or topk_weights.shape[1] != cfg.num_topk
                                     or topk_weights.shape[0] < token_end
                                     or topk_weights.device != dev):
        raise ValueError("topk_weights must be fp32 [>= token_end, num_topk] on the handle's device")
    _check(lib().ep_dispatch_topk(h.ptr, _ptr(topk_weights), token_begin, token_end,
                                  _ptr(recv_topk_idx), _ptr(recv_topk_weights), cap, _stream(dev)))
    return recv_topk_idx, recv_topk_weights


def ep_quantize_rows(cfg: Config, x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None):
    """Quantises bf16 rows x [rows, H] into the (codes, fp32 scales) form
    ep_combine reads under cfg.combine_quant.  Allocates missing outputs."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != cfg.hidden:
        raise ValueError("x must be bf16 [rows, hidden]")
    if cfg.combine_quant == EP_QUANT_NONE:
        raise ValueError("ep_quantize_rows needs combine_quant")
    rows = x.shape[0]
    if codes is None:
        codes = torch.empty((rows, cfg.hidden), device=x.device,
                            dtype=torch.int8 if cfg.combine_quant == EP_QUANT_INT8 else torch.uint8)
    if scales is None:
        scales = torch.empty((rows, cfg.hidden // cfg.combine_group), dtype=torch.float32,
                             device=x.device)
    _check_y(cfg, codes, scales)
    c = cfg.c()
    _check(lib().ep_quantize_rows(ctypes.byref(c), _ptr(x), rows, _ptr(codes), _ptr(scales),
                                  _stream(x.device)))
    return codes, scales


def ep_set_kernel_events(h: Handle, start_event=None, stop_event=None):
    """Arms raw hipEvent_t handles (ints or None) to take the start / end
    timestamps of the next call's first / last kernel."""
    _check(lib().ep_set_kernel_events(h.ptr, start_event, stop_event))


def ep_handle_view(h: Handle):
    """Device arrays of the handle as int32 tensor views of its workspace.
    For the static handle (no workspace tensor) each array is given as
    (device address, int32 element count) instead."""
    v = ep_handle_view_t()
    _check(lib().ep_handle_view(h.ptr, ctypes.byref(v)))
    ws = h.workspace
    cfg = h.cfg

    class _Raw:
        def __init__(self, p, n):
            self.addr, self.numel = p, n

        def view(self, *shape):
            self.shape = shape
            return self

    def arr(p, n):
        if ws is None:
            return _Raw(p, n)
        off = p - ws.data_ptr()
        return ws[off:off + 4 * n].view(torch.int32)

    N = max(v.num_tokens, 0)
    P = v.num_sources
    src = {}
    if v.psum_source_rank:
        src = dict(psum_source_rank=arr(v.psum_source_rank,
                                        cfg.num_ranks * (P + 1)).view(cfg.num_ranks, P + 1),
                   expert_source_base=arr(v.expert_source_base,
                                          P * cfg.num_experts).view(P, cfg.num_experts))
    return dict(**src, num_sources=P,
                psum_expert=arr(v.psum_expert, cfg.num_experts + 1),
                psum_rank=arr(v.psum_rank, cfg.num_ranks + 1),
                num_unaligned=arr(v.num_unaligned, cfg.num_experts),
                slot_idx=arr(v.slot_idx, N * cfg.num_topk).view(N, cfg.num_topk),
                src_meta=arr(v.src_meta, 2 * v.max_slots).view(v.max_slots, 2),
                topk_idx=arr(v.topk_idx, N * cfg.num_topk).view(N, cfg.num_topk),
                num_tokens=v.num_tokens, max_tokens=v.max_tokens, max_slots=v.max_slots,
                num_recv_slots=v.num_recv_slots)


ep_handle_get_view = ep_handle_view


def ep_check_error(h: Handle, raise_on_error=False):
    """Waits for the stream; returns (status, flags) and clears the flags."""
    flags = ctypes.c_uint32()
    st = lib().ep_check_error(h.ptr, _stream(h.device), ctypes.byref(flags))
    if raise_on_error:
        _check(st)
    return st, flags.value


# ---- pre-bound calls: pointers converted once, one ctypes call per launch --


def _bound(h, fn, *args):
    """call(events=None): issues fn(*args); events = (start, stop) raw
    hipEvent_t handles are armed first (ep_set_kernel_events)."""
    arm = lib().ep_set_kernel_events
    hp = h.ptr

    def call(events=None):
        if events is not None:
            arm(hp, events[0], events[1])
        st = fn(*args)
        if st != EP_OK:
            _check(st)
    return call


def bind_get_layout(h: Handle, topk_idx, num_tokens_per_rank=None, num_tokens_per_rdma_rank=None,
                    num_tokens_per_expert=None, is_token_in_rank=None, stream=None):
    """A callable issuing ep_get_layout (no CPU sync) with these tensors."""
    _layout_outputs(h.cfg, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                    num_tokens_per_expert, is_token_in_rank, False)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(topk_idx.device)
    return _bound(h, lib().ep_get_layout, h.ptr, _ptr(topk_idx), topk_idx.shape[0],
                  _ptr(num_tokens_per_rank), _ptr(num_tokens_per_rdma_rank),
                  _ptr(num_tokens_per_expert), _ptr(is_token_in_rank), 0, None, None, s)


def bind_dispatch(h: Handle, x, recv_x, recv_scales, token_begin, token_end, stream=None):
    """A callable issuing ep_dispatch with these tensors and token range."""
    token_begin, token_end = _check_dispatch_tensors(h.cfg, x, recv_x, recv_scales, token_begin,
                                                     token_end)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(x.device)
    return _bound(h, lib().ep_dispatch, h.ptr, _ptr(x), token_begin, token_end, _ptr(recv_x),
                  _ptr(recv_scales), recv_x.shape[0], s)


def bind_layout_dispatch(h: Handle, topk_idx, x, recv_x, recv_scales, num_tokens_per_rank=None,
                         num_tokens_per_rdma_rank=None, num_tokens_per_expert=None,
                         is_token_in_rank=None, stream=None):
    """A callable issuing ep_layout_dispatch with these tensors."""
    _layout_outputs(h.cfg, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                    num_tokens_per_expert, is_token_in_rank, False)
    _check_dispatch_tensors(h.cfg, x, recv_x, recv_scales)
    if x.shape[0] != topk_idx.shape[0] or x.device != topk_idx.device:
        raise ValueError("x and topk_idx disagree on the number of tokens or the device")
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(x.device)
    return _bound(h, lib().ep_layout_dispatch, h.ptr, _ptr(topk_idx), topk_idx.shape[0],
                  _ptr(num_tokens_per_rank), _ptr(num_tokens_per_rdma_rank),
                  _ptr(num_tokens_per_expert), _ptr(is_token_in_rank), _ptr(x), _ptr(recv_x),
                  _ptr(recv_scales), recv_x.shape[0], s)


def bind_dispatch_overlap(h: Handle, x, recv_x, recv_scales, token_begin, token_end, h_next,
                          topk_next, num_tokens_per_rank=None, num_tokens_per_rdma_rank=None,
                          num_tokens_per_expert=None, is_token_in_rank=None, stream=None):
    """A callable issuing ep_dispatch_overlap with these tensors."""
    token_begin, token_end = _check_dispatch_tensors(h.cfg, x, recv_x, recv_scales, token_begin,
                                                     token_end)
    _layout_outputs(h_next.cfg, topk_next, num_tokens_per_rank, num_tokens_per_rdma_rank,
                    num_tokens_per_expert, is_token_in_rank, False)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(x.device)
    return _bound(h, lib().ep_dispatch_overlap, h.ptr, _ptr(x), token_begin, token_end,
                  _ptr(recv_x), _ptr(recv_scales), recv_x.shape[0], h_next.ptr, _ptr(topk_next),
                  topk_next.shape[0], _ptr(num_tokens_per_rank), _ptr(num_tokens_per_rdma_rank),
                  _ptr(num_tokens_per_expert), _ptr(is_token_in_rank), s)


def bind_combine_overlap(h: Handle, y, topk_weights, out, token_begin, token_end, h_next,
                         stream=None, y_scales=None):
    """A callable issuing ep_combine_overlap with these tensors."""
    token_begin, token_end = _check_combine_tensors(h.cfg, y, y_scales, topk_weights, out,
                                                    token_begin, token_end)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(out.device)
    return _bound(h, lib().ep_combine_overlap, h.ptr, _ptr(y), _ptr(y_scales), y.shape[0],
                  _ptr(topk_weights), token_begin, token_end, _ptr(out), h_next.ptr, s)


def bind_combine(h: Handle, y, topk_weights, out, token_begin, token_end, stream=None,
                 y_scales=None):
    """A callable issuing ep_combine with these tensors and token range."""
    token_begin, token_end = _check_combine_tensors(h.cfg, y, y_scales, topk_weights, out,
                                                    token_begin, token_end)
    s = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(out.device)
    return _bound(h, lib().ep_combine, h.ptr, _ptr(y), _ptr(y_scales), y.shape[0],
                  _ptr(topk_weights), token_begin, token_end, _ptr(out), s)
