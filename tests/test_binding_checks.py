"""CPU checks of the binding's argument validation: shapes, dtypes, devices
and token ranges are rejected with ValueError before anything reaches the C
library (which knows only the handle's token count, not the tensors' sizes).

The handles here have no C handle behind them: a check that failed to fire
would reach Handle.ptr and raise RuntimeError, never call into the library.
"""
import ctypes

import pytest
import torch

from combine_get_dispatch_layout_amd import ep

CFG = ep.Config(hidden=256, num_topk=4, num_experts=32, num_ranks=8)


def _handle(cfg=CFG, n=16):
    h = ep.Handle.__new__(ep.Handle)
    h.cfg, h.max_tokens, h.workspace = cfg, n, torch.empty(0, dtype=torch.uint8)
    h._device = torch.device("cpu")
    h._ptr = ctypes.c_void_p()          # no C handle: .ptr raises RuntimeError
    return h


def _combine_tensors(n_out=16, n_w=16, rows=64):
    y = torch.zeros((rows, 256), dtype=torch.bfloat16)
    w = torch.zeros((n_w, 4), dtype=torch.float32)
    out = torch.zeros((n_out, 256), dtype=torch.bfloat16)
    return y, w, out


@pytest.mark.parametrize("fn", ["ep_combine", "ep_combine_overlap", "bind_combine",
                                "bind_combine_overlap"])
def test_combine_range_beyond_weights_or_out(fn):
    h = _handle()
    y, w, out = _combine_tensors(n_out=16, n_w=8)
    call = getattr(ep, fn)
    with pytest.raises(ValueError, match="token range"):
        if fn.startswith("bind"):
            args = (h, y, w, out, 0, 16) + ((h,) if "overlap" in fn else ())
            call(*args)
        else:
            call(h, y, w, out)                  # token_end defaults to out's 16 rows
    y, w, out = _combine_tensors(n_out=8, n_w=16)
    with pytest.raises(ValueError, match="token range"):
        if fn.startswith("bind"):
            call(*((h, y, w, out, 0, 12) + ((h,) if "overlap" in fn else ())))
        else:
            call(h, y, w, out, 0, 12)


@pytest.mark.parametrize("fn", ["ep_combine", "ep_combine_overlap"])
def test_combine_dtypes_and_shapes(fn):
    h = _handle()
    call = getattr(ep, fn)
    y, w, out = _combine_tensors()
    with pytest.raises(ValueError, match="out must be"):
        call(h, y, w, out.float())
    with pytest.raises(ValueError, match="topk_weights must be"):
        call(h, y, w[:, :3].contiguous(), out)
    with pytest.raises(ValueError, match="topk_weights must be"):
        call(h, y, w.double(), out)
    with pytest.raises(ValueError, match="y must be"):
        call(h, y[:, :128].contiguous(), w, out)
    with pytest.raises(ValueError, match="y_scales must be None"):
        call(h, y, w, out, y_scales=torch.zeros((64, 2)))


def test_layout_outputs_checked():
    topk = torch.zeros((16, 4), dtype=torch.int32)
    bad = [dict(num_tokens_per_rank=torch.zeros(7, dtype=torch.int32)),
           dict(num_tokens_per_rank=torch.zeros(8, dtype=torch.int64)),
           dict(num_tokens_per_expert=torch.zeros(31, dtype=torch.int32)),
           dict(is_token_in_rank=torch.zeros((15, 8), dtype=torch.bool)),
           dict(is_token_in_rank=torch.zeros((16, 8), dtype=torch.int32)),
           dict(num_tokens_per_rdma_rank=torch.zeros(1, dtype=torch.int32))]   # no nodes
    for kw in bad:
        with pytest.raises(ValueError):
            ep.ep_get_layout(_handle(), topk, **kw)
        with pytest.raises(ValueError):
            ep.bind_get_layout(_handle(), topk, **{f"{k}": v for k, v in kw.items()})
    with pytest.raises(ValueError, match="topk_idx"):
        ep.ep_get_layout(_handle(), topk[:, :3].contiguous())
    cfg = ep.Config(hidden=256, num_topk=4, num_experts=32, num_ranks=8, ranks_per_node=4)
    with pytest.raises(ValueError, match="rdma"):
        ep.ep_get_layout(_handle(cfg), topk,
                         num_tokens_per_rdma_rank=torch.zeros(3, dtype=torch.int32))


def test_dispatch_ranges_and_shapes():
    h = _handle()
    x = torch.zeros((16, 256), dtype=torch.bfloat16)
    recv = torch.zeros((64, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="token range"):
        ep.bind_dispatch(h, x, recv, None, 0, 17)
    with pytest.raises(ValueError, match="token range"):
        ep.ep_dispatch_overlap(h, x, recv, None, 4, 2)
    with pytest.raises(ValueError, match="recv_x must be"):
        ep.ep_dispatch(h, x, recv[:, :128].contiguous())
    with pytest.raises(ValueError, match="recv_scales must be None"):
        ep.ep_dispatch(h, x, recv, torch.zeros((64, 2)))
    with pytest.raises(ValueError, match="topk_idx"):
        ep.ep_dispatch_overlap(h, x, recv, None, h_next=_handle(), topk_next=None)
    with pytest.raises(ValueError, match="number of tokens"):
        ep.ep_layout_dispatch(h, torch.zeros((15, 4), dtype=torch.int32), x, recv)


def test_host_tensors_rejected():
    with pytest.raises(ValueError, match="on the GPU"):
        ep._ptr(torch.zeros(4))
    assert ep._ptr(None) is None
