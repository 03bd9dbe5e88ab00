"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/ep.h declares, and rejects invalid arguments on the host before any
HIP call (no compute call is made without a GPU)."""
import ctypes
import os
import re

import pytest

from combine_get_dispatch_layout_amd import ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "ep.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(ep.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = ep.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    # the boundary's calls by their contract names
    for name in ("ep_workspace_size", "ep_handle_init", "ep_handle_free", "ep_get_layout",
                 "ep_dispatch", "ep_combine", "ep_handle_view", "ep_check_error",
                 "ep_status_str", "ep_last_error_message"):
        assert name in _declared_functions() and hasattr(L, name), name


def test_every_call_cites_a_passage():
    """Each declaration in include/ep.h is preceded by a comment that names
    the page passage ([P2] ... [P5]) defining the operation."""
    with open(os.path.join(ROOT, "include", "ep.h")) as f:
        text = f.read()
    body = text.split('extern "C" {', 1)[1]
    decls = list(re.finditer(r"^(?:ep_status|void|const char\*) (ep_[a-z_]+)\(", body, flags=re.M))
    assert len(decls) == len(ep.SYMBOLS)
    missing, prev = [], 0
    for m in decls:
        before = body[prev:m.start()]
        prev = m.end()
        if m.group(1) == "ep_handle_get_view":
            continue                      # the alias of ep_handle_view
        if m.group(1) == "ep_handle_init_static":
            # not an operation of the pages: its comment names its callers
            assert "cannot allocate" in before
            continue
        if not re.search(r"\[P[2-5]\]", before):
            missing.append(m.group(1))
    assert not missing, missing


def test_status_strings():
    assert ep.status_name(ep.EP_OK) == "EP_OK"
    assert ep.status_name(ep.EP_ERR_CAPACITY) == "EP_ERR_CAPACITY"
    assert ep.status_name(99) == "EP_ERR_UNKNOWN"


GOOD = dict(hidden=2048, num_topk=8, num_experts=128, num_ranks=16)


@pytest.mark.parametrize("bad", [
    dict(hidden=0), dict(hidden=2047), dict(hidden=(1 << 24) + 8), dict(num_topk=0), dict(num_topk=17),
    dict(num_experts=0), dict(num_experts=1025), dict(num_ranks=0), dict(num_ranks=3),
    dict(num_ranks=2048, num_experts=1024), dict(ranks_per_node=-1), dict(expert_alignment=0),
    dict(quant=3), dict(quant=1, quant_group=64), dict(quant=2, quant_group=128, hidden=2056),
    dict(quant=2, quant_group=16384, hidden=16384), dict(num_sources=-1),
    dict(num_sources=1025), dict(quant=3, quant_group=128), dict(quant=3, quant_group=32, hidden=2056),
    dict(quant=4), dict(scale_mode=3), dict(combine_quant=3, combine_group=128),
    dict(combine_quant=1, combine_group=64), dict(combine_quant=2, combine_group=128, hidden=2056),
])
def test_invalid_configs_rejected(bad):
    cfg = ep.Config(**{**GOOD, **bad})
    with pytest.raises(ep.EpError) as ei:
        ep.ep_workspace_size(cfg, 4096)
    assert ei.value.status == ep.EP_ERR_INVALID_ARG
    assert ".cpp:" in str(ei.value)        # "file:line reason"


def test_workspace_and_capacity_sizes():
    cfg = ep.Config(**GOOD, expert_alignment=128)
    assert ep.ep_recv_capacity(cfg, 4096) == 4096 * 8 + 128 * 127
    b = ep.ep_workspace_size(cfg, 4096)
    # at least the slot, clone and metadata arrays
    assert b >= 4096 * 8 * 4 * 2 + 8 * ep.ep_recv_capacity(cfg, 4096)
    assert b % 256 == 0
    with pytest.raises(ep.EpError):
        ep.ep_workspace_size(cfg, -1)
    with pytest.raises(ep.EpError):
        ep.ep_workspace_size(cfg, 1 << 29)      # receive rows beyond 2^31


def test_quantize_rows_host_checks():
    L = ep.lib()
    c = ep.Config(**GOOD).c()            # combine_quant none: rejected
    assert L.ep_quantize_rows(ctypes.byref(c), None, 4, None, None, None) == ep.EP_ERR_INVALID_ARG
    c = ep.Config(**GOOD, combine_quant=1, combine_group=128).c()
    assert L.ep_quantize_rows(ctypes.byref(c), None, 0, None, None, None) == ep.EP_OK   # no rows
    assert L.ep_quantize_rows(ctypes.byref(c), None, 4, None, None, None) == ep.EP_ERR_INVALID_ARG
    c = ep.Config(hidden=16384, num_topk=8, num_experts=128, num_ranks=16, combine_quant=2,
                  combine_group=16384).c()    # one row is too long for one wave's scale
    assert L.ep_quantize_rows(ctypes.byref(c), None, 4, None, None, None) == ep.EP_ERR_INVALID_ARG


def test_workspace_grows_with_sources():
    one = ep.ep_workspace_size(ep.Config(**GOOD), 4096)
    p16 = ep.ep_workspace_size(ep.Config(**GOOD, num_sources=16), 4096)
    # accumulators [P, E+R], bases [P, E], prefix [R, P+1], each 256-byte aligned
    assert p16 - one >= 4 * (16 * (128 + 16) + 16 * 128 + 16 * 17)
    assert ep.ep_workspace_size(ep.Config(**GOOD, num_sources=1), 4096) == one


def _init(cfg, max_tokens, ptr, nbytes):
    out = ctypes.c_void_p()
    c = cfg.c()
    return ep.lib().ep_handle_init(ctypes.byref(c), max_tokens, ctypes.c_void_p(ptr), nbytes, None,
                                   ctypes.byref(out)), out


def test_handle_init_workspace_errors():
    cfg = ep.Config(**GOOD)
    need = ep.ep_workspace_size(cfg, 1024)
    st, out = _init(cfg, 1024, 0, need)
    assert st == ep.EP_ERR_WORKSPACE and not out.value
    st, out = _init(cfg, 1024, 0x1000 + 16, need)          # misaligned
    assert st == ep.EP_ERR_WORKSPACE
    st, out = _init(cfg, 1024, 0x1000, need - 1)           # too small
    assert st == ep.EP_ERR_WORKSPACE
    assert "needs" in ep.lib().ep_last_error_message().decode()


def test_calls_on_null_handle_rejected():
    L = ep.lib()
    assert L.ep_get_layout(None, None, 0, None, None, None, None, 0, None, None, None) == \
        ep.EP_ERR_INVALID_ARG
    assert L.ep_dispatch(None, None, 0, 0, None, None, 0, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_combine(None, None, None, 0, None, 0, 0, None, None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_layout_dispatch(None, None, 0, None, None, None, None, None, None, None, 0,
                                None) == ep.EP_ERR_INVALID_ARG
    assert L.ep_check_error(None, None, None) == ep.EP_ERR_INVALID_ARG
    L.ep_handle_free(None)


def test_static_handle_rejects_workspace_beyond_its_limit():
    """ep_handle_init_static refuses, before any HIP call, a handle whose
    workspace would not fit the library's static array."""
    cfg = ep.Config(**GOOD)
    need = ep.ep_workspace_size(cfg, 1 << 18)
    assert need > (4 << 20)
    out = ctypes.c_void_p()
    c = cfg.c()
    st = ep.lib().ep_handle_init_static(ctypes.byref(c), 1 << 18, None, ctypes.byref(out))
    assert st == ep.EP_ERR_WORKSPACE and not out.value
    msg = ep.lib().ep_last_error_message().decode()
    assert str(need) in msg and str(4 << 20) in msg
    c = ep.Config(**{**GOOD, "num_topk": 0}).c()
    assert ep.lib().ep_handle_init_static(ctypes.byref(c), 16, None, ctypes.byref(out)) == \
        ep.EP_ERR_INVALID_ARG


_I32 = (-2 ** 31, 2 ** 31 - 1)


def _cfg_strategy():
    from hypothesis import strategies as st

    def near(vals):
        return st.one_of(st.sampled_from(vals), st.integers(*_I32))
    return st.builds(
        ep.Config,
        hidden=near([8, 128, 2048, 7168, 8192, 1 << 24]),
        num_topk=near([1, 8, 16, 17]),
        num_experts=near([1, 16, 128, 256, 1024]),
        num_ranks=near([1, 4, 16, 1024]),
        ranks_per_node=near([0, 1, 8]),
        expert_alignment=near([1, 128]),
        quant=near([0, 1, 2, 3]),
        quant_group=near([0, 32, 128, 2048]),
        counts_as_prefix=st.booleans(),
        expert_capacity=near([0, 1, 64]),
        num_sources=near([0, 1, 16, 1024]),
        scale_mode=near([0, 1, 2]),
        combine_quant=near([0, 1, 2]),
        combine_group=near([0, 128, 2048]),
        non_expand=st.booleans())


def test_sizes_never_misbehave_on_arbitrary_configs():
    """The host-side size calls, on arbitrary configurations and token counts
    (any int32 field, any int64 count): a status of EP_OK or
    EP_ERR_INVALID_ARG, never a crash; an accepted size is positive, a
    multiple of 256 and holds the receive rows, which stay below 2^31."""
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=400, deadline=None, derandomize=True)
    @given(_cfg_strategy(), st.one_of(st.sampled_from([0, 1, 4096, 1 << 20]),
                                      st.integers(-2 ** 63, 2 ** 63 - 1)))
    def check(cfg, n):
        L = ep.lib()
        c = cfg.c()
        out = ctypes.c_int64(-7)
        st_ws = L.ep_workspace_size(ctypes.byref(c), n, ctypes.byref(out))
        assert st_ws in (ep.EP_OK, ep.EP_ERR_INVALID_ARG)
        if st_ws == ep.EP_OK:
            assert out.value > 0 and out.value % 256 == 0
        cap = ctypes.c_int64(-7)
        st_cap = L.ep_recv_capacity(ctypes.byref(c), n, ctypes.byref(cap))
        assert st_cap in (ep.EP_OK, ep.EP_ERR_INVALID_ARG)
        if st_cap == ep.EP_OK:
            assert 0 <= cap.value < 2 ** 31
        if st_ws == ep.EP_OK:
            assert st_cap == ep.EP_OK and out.value >= 8 * cap.value
    check()
