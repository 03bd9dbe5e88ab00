"""The allocation-free handle (ep_handle_init_static, workspace = the
library's static device array) against the handle over a caller workspace
(ep_handle_init): the same layout outputs, host list, handle arrays, receive
rows, scales and combine output, bit for bit, on calls in a row whose second
batch is smaller -- with the static handle set up again for each batch, and
kept from the first batch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from combine_get_dispatch_layout_amd import ep
from shuffle_check import bits16, config_of

pytestmark = pytest.mark.gpu

_HIP = None


def _copy_i32(addr, numel):
    """int32 array at a device address, copied into host memory."""
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    out = np.empty(numel, np.int32)
    torch.cuda.synchronize()
    assert _HIP.hipMemcpy(out.ctypes.data, addr, 4 * numel, 2) == 0    # device to host
    return out


def _arrays(h, S):
    """The handle's arrays as host numpy, for either kind of handle."""
    v = ep.ep_handle_view(h)
    out = {}
    for k in ("psum_expert", "psum_rank", "num_unaligned", "slot_idx", "topk_idx", "src_meta"):
        a = v[k]
        if isinstance(a, torch.Tensor):
            a = a.reshape(-1).cpu().numpy()
        else:
            a = _copy_i32(a.addr, a.numel)
        out[k] = a[:2 * S] if k == "src_meta" else a
    out["num_tokens"] = v["num_tokens"]
    out["num_recv_slots"] = v["num_recv_slots"]
    return out


def _run(h, w, idx, wts, x, y):
    cfg = config_of(w)
    N = idx.shape[0]
    topk = torch.from_numpy(idx).cuda()
    wd = torch.from_numpy(wts).cuda()
    lay = ep.ep_get_layout(h, topk, do_cpu_sync=True)
    S = lay["num_recv_slots"]
    cap = ep.ep_recv_capacity(cfg, N)
    recv = torch.zeros((cap, cfg.recv_row_elems), dtype=cfg.recv_dtype, device="cuda")
    scales = (torch.zeros((cap, cfg.num_groups), dtype=cfg.scales_dtype, device="cuda")
              if w.quant else None)
    rounds = W.round_ranges(N, w.rounds)
    for b, e in rounds:
        ep.ep_dispatch(h, x, recv, scales, b, e)
    out = torch.zeros((N, w.hidden), dtype=torch.bfloat16, device="cuda")
    for b, e in rounds:
        ep.ep_combine(h, y, wd, out, b, e)
    assert ep.ep_check_error(h) == (ep.EP_OK, 0)
    res = {k: v.cpu().numpy() for k, v in lay.items() if isinstance(v, torch.Tensor)}
    res["host_list"] = np.array(lay["num_recv_tokens_per_expert_list"])
    res["S"] = S
    res["recv"] = recv[:S].view(torch.uint8).cpu().numpy()
    if scales is not None:
        res["scales"] = scales[:S].view(torch.uint8).cpu().numpy()
    res["out"] = bits16(out)
    res.update({"view_" + k: v for k, v in _arrays(h, S).items()})
    return res


def _inputs(w, n, seed):
    wb = w.scaled(num_tokens=n, seed=seed)
    idx, wts = W.routing(wb)
    x = W.activations(n, w.hidden, seed * 3 + 1, device="cuda")
    cap = ep.ep_recv_capacity(config_of(w), n)
    y = W.activations(cap, w.hidden, seed * 3 + 2, device="cuda")
    return wb, idx, wts, x, y


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert np.array_equal(a[k], b[k]), k
        else:
            assert a[k] == b[k], k


CASES = [
    # (workload, token counts of the calls in a row)
    ("qwen3_30b_a3b_prefill", [4096, 777]),
    ("deepseek_v3_prefill", [3000, 1531]),          # alignment 128, masking, Zipf
    ("long_seq_int8", [8192, 2050]),                # int8 per row, 4 rounds
    ("ll_decode_fp8", [128, 57]),                   # FP8 groups of 128
]


@pytest.mark.parametrize("name,sizes", CASES)
@pytest.mark.parametrize("reinit", [True, False])
def test_static_handle_matches_workspace_handle(name, sizes, reinit):
    w = W.WORKLOADS[name]
    cfg = config_of(w)
    print(f"[no-alloc] {name} sizes={sizes} reinit={reinit}", flush=True)
    hs = None
    for i, n in enumerate(sizes):
        wb, idx, wts, x, y = _inputs(w, n, 40 + i)
        if reinit or hs is None:
            hs = ep.ep_handle_init_static(cfg, n if reinit else max(sizes))
        hw = ep.ep_handle_init(cfg, n, device="cuda")
        got = _run(hs, wb, idx, wts, x, y)
        want = _run(hw, wb, idx, wts, x, y)
        _same(got, want)
        assert got["S"] > 0 and got["view_num_tokens"] == n
    ep.ep_handle_free(hs)           # a no-op for the static handle


def test_static_handle_is_one_per_device():
    cfg = config_of(W.WORKLOADS["tiny"])
    a = ep.ep_handle_init_static(cfg, 128)
    b = ep.ep_handle_init_static(cfg, 64)
    assert a.ptr.value == b.ptr.value
    a.free()
    b.free()
