"""Shared parity machinery: run the HIP path through the C ABI and compare
every output with the CPU oracle on the same seeded inputs.

Parity bars (written out here, used by every GPU test):
  * layout outputs, psum/count arrays, slot indices, source metadata and
    bf16 dispatched rows: bit-exact;
  * FP8 E4M3FN / int8 codes: at most one step apart on the ordered code line
    (the kernels decide codes in fp32 exactly as the oracle does, so the
    observed difference is expected to be zero), fp32 scales bit-exact;
  * combine: bit-exact against the oracle's fp32 reduction (k ascending, one
    fused multiply-add per term, then bf16), which is the reduction the path
    states; that is inside the one-ulp bar |got - ref| <= 2^-7 * |ref|.
    Against the oracle's exact sum (fp64, rounded once) every element must
    lie within 2^-7 * max(|ref|, |got|) plus the error bound of a K-term fp32
    chain, K * 2^-23 * sum_k |w_k y_k| (K * u * sum|terms|, u = 2^-24,
    doubled); the elements beyond the strict 2^-7 * |ref| bar there are
    counted (cancellation: the sum is far below its terms).
"""
import numpy as np
import torch

import oracle
import workloads as W
from combine_get_dispatch_layout_amd import ep


def bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def config_of(w: W.Workload, counts_as_prefix=False):
    return ep.Config(hidden=w.hidden, num_topk=w.num_topk, num_experts=w.num_experts,
                     num_ranks=w.num_ranks, ranks_per_node=w.ranks_per_node,
                     expert_alignment=w.expert_alignment, quant=w.quant,
                     quant_group=w.quant_group if w.quant else 0,
                     counts_as_prefix=counts_as_prefix, expert_capacity=w.expert_capacity,
                     num_sources=w.num_sources, scale_mode=w.scale_mode,
                     combine_quant=w.combine_quant, combine_group=w.combine_group,
                     non_expand=w.non_expand)


def oracle_slots(w: W.Workload, idx):
    """The oracle's slot assignment for the workload's layout mode (the
    receive rows: per (token, rank) with non_expand)."""
    if w.non_expand:
        return oracle.slots_nonexpand(idx, w.num_experts, w.num_ranks)
    if w.expert_capacity > 0:
        return oracle.slots_fixed(idx, w.num_experts, w.num_ranks, w.expert_capacity)
    return oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment)


def expected_host_list(w: W.Workload, ref_slots, counts_as_prefix=False):
    if w.expert_capacity > 0:
        return oracle.recv_list_fixed(ref_slots["num_unaligned"], w.num_experts, w.num_ranks,
                                      w.expert_capacity, counts_as_prefix).tolist()
    return oracle.recv_list(ref_slots["psum_expert"], w.num_experts, w.num_ranks,
                            counts_as_prefix).tolist()




class GpuRun:
    """All device-side buffers of one run of the path."""

    def __init__(self, w: W.Workload, idx, wts, x, y_rows=None, device="cuda", rounds=None):
        self.w = w
        self.cfg = config_of(w)
        N = idx.shape[0]
        self.h = ep.ep_handle_init(self.cfg, N, device=device)
        self.topk = torch.from_numpy(idx).to(device)
        self.wts = torch.from_numpy(wts).to(device)
        self.x = x.to(device)
        self.cap = ep.ep_recv_capacity(self.cfg, N)
        self.recv = torch.zeros((self.cap, self.cfg.recv_row_elems), dtype=self.cfg.recv_dtype,
                                device=device)
        self.scales = (torch.zeros((self.cap, self.cfg.num_groups), dtype=self.cfg.scales_dtype,
                                   device=device) if w.quant else None)
        self.out = torch.zeros((N, w.hidden), dtype=torch.bfloat16, device=device)
        self.rounds = rounds or W.round_ranges(N, w.rounds)
        self.y_rows = self.cap if y_rows is None else y_rows

    def layout(self, do_cpu_sync=True):
        self.lay = ep.ep_get_layout(self.h, self.topk, do_cpu_sync=do_cpu_sync)
        return self.lay

    def layout_dispatch(self):
        """Layout and dispatch of the whole batch in one ep_layout_dispatch call."""
        assert len(self.rounds) == 1
        self.lay = ep.ep_layout_dispatch(self.h, self.topk, self.x, self.recv, self.scales)
        return self.lay

    def dispatch(self):
        for b, e in self.rounds:
            ep.ep_dispatch(self.h, self.x, self.recv, self.scales, b, e)

    def combine(self, y, y_scales=None):
        for b, e in self.rounds:
            ep.ep_combine(self.h, y, self.wts, self.out, b, e, y_scales=y_scales)


def compare_layout(run: GpuRun, idx, ref_lay, ref_slots, host_sync=True):
    w = run.w
    lay = run.lay
    assert np.array_equal(lay["num_tokens_per_expert"].cpu().numpy(), ref_lay["num_tokens_per_expert"])
    assert np.array_equal(lay["num_tokens_per_rank"].cpu().numpy(), ref_lay["num_tokens_per_rank"])
    assert np.array_equal(lay["is_token_in_rank"].cpu().numpy().astype(np.uint8),
                          ref_lay["is_token_in_rank"])
    if ref_lay["num_tokens_per_rdma_rank"] is not None:
        assert np.array_equal(lay["num_tokens_per_rdma_rank"].cpu().numpy(),
                              ref_lay["num_tokens_per_rdma_rank"])
    v = ep.ep_handle_view(run.h)
    S = ref_slots["S"]
    # per-expert arrays: the expert-level layout (the receive layout itself
    # with expand)
    ref_exp = oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment) \
        if w.non_expand else ref_slots
    if host_sync:
        assert lay["num_recv_slots"] == S == v["num_recv_slots"]
    else:
        assert v["num_recv_slots"] == -1
    assert np.array_equal(v["psum_expert"].cpu().numpy(), ref_exp["psum_expert"])
    assert np.array_equal(v["psum_rank"].cpu().numpy(), ref_slots["psum_rank"])
    assert np.array_equal(v["num_unaligned"].cpu().numpy(), ref_exp["num_unaligned"])
    assert np.array_equal(v["slot_idx"].cpu().numpy(), ref_slots["slot_idx"])
    assert np.array_equal(v["src_meta"][:S].cpu().numpy(), ref_slots["src_meta"])
    assert np.array_equal(v["topk_idx"].cpu().numpy(), idx)
    assert v["num_sources"] == max(w.num_sources, 1)
    if w.num_sources > 1:
        ref_src = oracle.source_counts(idx, w.num_experts, w.num_ranks, w.num_sources)
        assert np.array_equal(v["psum_source_rank"].cpu().numpy(), ref_src["psum_source_rank"])
        assert np.array_equal(v["expert_source_base"].cpu().numpy(),
                              ref_src["expert_source_base"])
    else:
        assert "psum_source_rank" not in v
    if host_sync:
        assert lay["num_recv_tokens_per_expert_list"] == expected_host_list(w, ref_exp)


def ordered_code(c, quant):
    c = c.astype(np.int32)
    if quant == W.QUANT_FP8:
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    return np.where(c > 127, c - 256, c)    # int8 viewed as uint8


def compare_dispatch(run: GpuRun, ref_recv, ref_scales, ref_slots):
    """Returns the number of quantised codes that differ (0 for bf16).
    MXFP4 codes and every scale (fp32 words or E8M0 bytes) must match
    exactly; FP8 / int8 codes within one step."""
    meta = ref_slots["src_meta"]
    real = meta[:, 0] >= 0
    S = ref_slots["S"]
    if run.w.quant == W.QUANT_NONE:
        got = bits16(run.recv[:S])
        assert np.array_equal(got[real], ref_recv[:S][real])
        return 0
    got = run.recv[:S].view(torch.uint8).cpu().numpy()[real]
    ref = ref_recv[:S].view(np.uint8)[real]
    gs = run.scales[:S].cpu().numpy()[real]
    rs = ref_scales[:S][real]
    if gs.dtype == np.uint8:
        assert np.array_equal(gs, rs.view(np.uint8))
    else:
        assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))
    if run.w.quant == W.QUANT_MXFP4:
        assert np.array_equal(got, ref)
        return 0
    d = np.abs(ordered_code(got, run.w.quant) - ordered_code(ref, run.w.quant))
    assert d.max(initial=0) <= 1, f"codes differ by {d.max()} steps"
    return int((d != 0).sum())


def combine_refs(y_bits, wts, slot_idx):
    """The oracle's combine of bf16 expert outputs: (fp32 chain, exact sum)."""
    return oracle.combine_fma(y_bits, wts, slot_idx), oracle.combine(y_bits, wts, slot_idx)


def combine_q_refs(codes, scales, quant, group, wts, slot_idx):
    """The same for quantised expert outputs."""
    return (oracle.combine_q_fma(codes, scales, quant, group, wts, slot_idx),
            oracle.combine_q(codes, scales, quant, group, wts, slot_idx))


def compare_combine(got_bits, refs, yval, wts, slot_idx, K):
    """Checks the combine bars against refs = (fp32 chain, exact sum).
    Returns dict(not_bit_identical: elements differing from the exact sum,
    beyond_strict_bar: of those, the ones with |got - ref| > 2^-7 * |ref|).
    yval(s, h): the value of expert-output element (s, h), for the chain
    bound of the elements beyond the strict bar."""
    ref_chain, ref_exact = refs
    off = got_bits != ref_chain
    if off.any():
        t, h = np.argwhere(off)[0]
        raise AssertionError(f"{int(off.sum())} combine elements differ from the fp32 chain; "
                             f"first ({t},{h}): got {got_bits[t, h]:#06x} want {ref_chain[t, h]:#06x}")
    got = oracle.f32_from_bf16(got_bits).astype(np.float64)
    ref = oracle.f32_from_bf16(ref_exact).astype(np.float64)
    d = np.abs(got - ref)
    beyond = np.argwhere(d > 2.0 ** -7 * np.abs(ref))
    for t, hcol in beyond:
        terms = [abs(float(wts[t, k])) * abs(yval(slot_idx[t, k], hcol))
                 for k in range(K) if slot_idx[t, k] >= 0]
        bar = 2.0 ** -7 * max(abs(ref[t, hcol]), abs(got[t, hcol])) + K * 2.0 ** -23 * sum(terms)
        assert d[t, hcol] <= bar, (t, hcol, got[t, hcol], ref[t, hcol], bar)
    return dict(not_bit_identical=int((got_bits != ref_exact).sum()),
                beyond_strict_bar=int(len(beyond)))


def bf16_values(y_bits):
    return lambda s, h: float(oracle.f32_from_bf16(y_bits[s, h:h + 1])[0])


def quantised_values(codes, scales, quant, group):
    def val(s, h):
        c = codes[s, h:h + 1]          # uint8 (E4M3FN) or int8
        v = (float(oracle.f32_from_e4m3fn(c)[0]) if quant == W.QUANT_FP8 else float(c[0]))
        return v * float(scales[s, h // group])
    return val


def run_and_check(w: W.Workload, device="cuda", rounds=None, seed_x=None, seed_y=None,
                  check_combine=True, idx=None, wts=None, fused=False):
    """Full path for workload `w` on the device and on the oracle; asserts
    the parity bars.  Returns a dict of statistics.  fused: layout and
    dispatch through the one-call ep_layout_dispatch (no host sync)."""
    if idx is None:
        idx, wts = W.routing(w)
    N = idx.shape[0]
    x = W.activations(N, w.hidden, seed_x if seed_x is not None else W.x_seed(w), device=device)
    run = GpuRun(w, idx, wts, x, device=device, rounds=rounds)
    if fused:
        run.layout_dispatch()
    else:
        run.layout()
        run.dispatch()
    ref_lay = oracle.layout(idx, w.num_experts, w.num_ranks, w.ranks_per_node)
    ref_slots = oracle_slots(w, idx)
    st, flags = ep.ep_check_error(run.h)
    if ref_slots.get("dropped", 0) > 0:    # full fixed-capacity segments
        assert st == ep.EP_ERR_CAPACITY and flags == ep.EP_FLAG_RECV_CAPACITY
    else:
        assert st == ep.EP_OK and flags == 0
    compare_layout(run, idx, ref_lay, ref_slots, host_sync=not fused)
    x_bits = bits16(x)
    ref_recv, ref_scales = oracle.dispatch(x_bits, ref_slots["slot_idx"], run.cap, quant=w.quant,
                                           group=w.quant_group or None, scale_mode=w.scale_mode)
    ncode = compare_dispatch(run, ref_recv, ref_scales, ref_slots)
    stats = dict(S=ref_slots["S"], code_diffs=ncode)
    if w.non_expand:
        ri, rw = ep.ep_dispatch_topk(run.h, run.wts, rows=run.cap)
        ref_ri, ref_rw = oracle.recv_topk(idx, wts, ref_slots["src_meta"], w.num_experts,
                                          w.num_ranks)
        S = ref_slots["S"]
        assert np.array_equal(ri[:S].cpu().numpy(), ref_ri)
        assert np.array_equal(rw[:S].cpu().numpy().view(np.uint32), ref_rw.view(np.uint32))
        assert ep.ep_check_error(run.h) == (ep.EP_OK, 0)
    if check_combine:
        S = ref_slots["S"]
        y = W.activations(max(S, 1), w.hidden,
                          seed_y if seed_y is not None else W.y_seed(w), device=device)
        y_bits = bits16(y)
        if w.combine_quant:
            # expert outputs as codes + fp32 scales, quantised by the oracle
            cq, cs = oracle.quantize_rows(y_bits, w.combine_quant, group=w.combine_group,
                                          scale_mode=min(w.scale_mode, 1))
            run.combine(torch.from_numpy(cq).to(device), torch.from_numpy(cs).to(device))
            refs = combine_q_refs(cq, cs, w.combine_quant, w.combine_group, wts,
                                  ref_slots["slot_idx"])
            yval = quantised_values(cq, cs, w.combine_quant, w.combine_group)
        elif w.non_expand:
            # rank rows already weighted on the expert side: unit weights
            for b, e in run.rounds:
                ep.ep_combine(run.h, y, None, run.out, b, e)
            refs = combine_refs(y_bits, np.ones_like(wts), ref_slots["slot_idx"])
            yval = bf16_values(y_bits)
        else:
            run.combine(y)
            refs = combine_refs(y_bits, wts, ref_slots["slot_idx"])
            yval = bf16_values(y_bits)
        st, flags = ep.ep_check_error(run.h)
        assert st == ep.EP_OK and flags == 0
        cc = compare_combine(bits16(run.out), refs, yval,
                             np.ones_like(wts) if w.non_expand else wts, ref_slots["slot_idx"],
                             w.num_topk)
        stats["combine_not_bit_identical"] = cc["not_bit_identical"]
        stats["combine_beyond_strict_bar"] = cc["beyond_strict_bar"]
    stats["run"] = run
    return stats


def run_overlap_sequence(w: W.Workload, sizes, seeds, device="cuda"):
    """Batches of the given sizes through the merged calls (ep_dispatch_overlap
    / ep_combine_overlap over two handles): batch i+1 is laid out inside batch
    i's launches.  Checks every batch's rows and combine output, and every
    next batch's layout, against the oracle.  Returns the two handles."""
    cfg = config_of(w)
    nmax = max(sizes)
    hs = [ep.ep_handle_init(cfg, nmax, device=device), ep.ep_handle_init(cfg, nmax, device=device)]
    batches = []
    for n, sd in zip(sizes, seeds):
        wb = w.scaled(num_tokens=n, seed=sd)
        idx, wts = W.routing(wb)
        x = W.activations(n, w.hidden, sd * 7 + 1, device=device)
        cap = ep.ep_recv_capacity(cfg, n)
        b = dict(w=wb, idx=idx, wts=wts, topk=torch.from_numpy(idx).to(device),
                 wts_d=torch.from_numpy(wts).to(device), x=x,
                 recv=torch.zeros((cap, cfg.recv_row_elems), dtype=cfg.recv_dtype, device=device),
                 scales=(torch.zeros((cap, cfg.num_groups), dtype=cfg.scales_dtype, device=device)
                         if w.quant else None),
                 out=torch.zeros((n, w.hidden), dtype=torch.bfloat16, device=device), cap=cap)
        batches.append(b)
    lay = ep.ep_get_layout(hs[0], batches[0]["topk"])
    for i, b in enumerate(batches):
        h, hn = hs[i % 2], hs[(i + 1) % 2]
        nxt = batches[i + 1] if i + 1 < len(batches) else None
        if nxt is not None:
            nlay = ep.ep_dispatch_overlap(h, b["x"], b["recv"], b["scales"], h_next=hn,
                                          topk_next=nxt["topk"])
        else:
            ep.ep_dispatch_overlap(h, b["x"], b["recv"], b["scales"])
        S = oracle_slots(b["w"], b["idx"])["S"]
        y = W.activations(max(S, 1), w.hidden, 900 + i, device=device)
        ep.ep_combine_overlap(h, y, b["wts_d"], b["out"], h_next=hn if nxt is not None else None)
        st, flags = ep.ep_check_error(h)
        # the finished batch: rows and combine
        ref_slots = oracle_slots(b["w"], b["idx"])
        dropped = ref_slots.get("dropped", 0) > 0
        assert st == (ep.EP_ERR_CAPACITY if dropped else ep.EP_OK), (i, st, flags)

        class R:
            pass
        run = R()
        run.w, run.recv, run.scales = b["w"], b["recv"], b["scales"]
        ref_recv, ref_scales = oracle.dispatch(bits16(b["x"]), ref_slots["slot_idx"], b["cap"],
                                               quant=w.quant, group=w.quant_group or None,
                                               scale_mode=w.scale_mode)
        compare_dispatch(run, ref_recv, ref_scales, ref_slots)
        y_bits = bits16(y)
        compare_combine(bits16(b["out"]), combine_refs(y_bits, b["wts"], ref_slots["slot_idx"]),
                        bf16_values(y_bits), b["wts"], ref_slots["slot_idx"], w.num_topk)
        if w.non_expand and ref_slots["S"] > 0:
            ri, rw = ep.ep_dispatch_topk(h, b["wts_d"], rows=b["cap"])
            ref_ri, ref_rw = oracle.recv_topk(b["idx"], b["wts"], ref_slots["src_meta"],
                                              w.num_experts, w.num_ranks)
            S = ref_slots["S"]
            assert np.array_equal(ri[:S].cpu().numpy(), ref_ri)
            assert np.array_equal(rw[:S].cpu().numpy().view(np.uint32), ref_rw.view(np.uint32))
        # the next batch's layout, complete after this combine
        if nxt is not None:
            run.lay, run.h = nlay, hn
            ref_lay = oracle.layout(nxt["idx"], w.num_experts, w.num_ranks, w.ranks_per_node)
            compare_layout(run, nxt["idx"], ref_lay, oracle_slots(nxt["w"], nxt["idx"]),
                           host_sync=False)
    return hs
