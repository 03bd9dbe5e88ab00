"""Benchmark of the MoE token shuffle on one MI355X.

One step = the whole hot path over one batch: routing layout + slot
assignment (ep_get_layout), dispatch (ep_dispatch, per round) and combine
(ep_combine, per round), all through the C ABI with inputs resident in HBM.
Default workload: the Qwen3-30B-A3B-shaped prefill (4096 tokens, hidden 2048
bf16, 128 experts over 16 simulated ranks, top-8).

Prints one JSON line.  `value` is tokens/s over whole steps; the roofline
entry is for the kernel with the largest share of the step, with its
achieved bandwidth = algorithmic bytes per launch / mean launch time taken
from HIP events recorded on the launch stream inside the timed region.
Buffers rotate over several independent sets so each step streams memory
that the 256 MB Infinity Cache does not hold.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s (AMD public figure)


def algorithmic_bytes(w, V, S):
    """Bytes each stage must move (padding rows excluded), per step.

    layout:   topk read 4NK, clone + in-block rank + slot writes/reads 16NK,
              is_token_in_rank NR, metadata 8V
    dispatch: x read 2NH, slot read 4NK, receive rows V*(b*H + 4G)
    combine:  y rows read 2VH, weights + slots read 8NK, out write 2NH
    """
    N, H, K, R = w.num_tokens, w.hidden, w.num_topk, w.num_ranks
    b = 2 if w.quant == 0 else 1
    G = (H // w.quant_group) if w.quant else 0
    layout = 4 * N * K + 16 * N * K + N * R + 8 * V
    dispatch = 2 * N * H + 4 * N * K + V * (b * H + 4 * G)
    combine = 2 * V * H + 8 * N * K + 2 * N * H
    return dict(layout=layout, dispatch=dispatch, combine=combine)


def kernel_source_hash(kernel):
    src = {"dispatch": "dispatch.hip", "combine": "combine.hip", "layout": "layout.hip"}[kernel]
    with open(os.path.join(ROOT, "combine_get_dispatch_layout_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, idx, wts, budget_s=12.0):
    """The oracle, as it stands (serial C), on the same workload: repeated
    full passes (layout, slots, dispatch, combine) until budget_s is spent."""
    import numpy as np
    import oracle
    import workloads as W
    import torch
    N = w.num_tokens
    x = W.activations(N, w.hidden, W.x_seed(w)).view(torch.int16).numpy().view(np.uint16)
    s0 = oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment)
    y = W.activations(max(s0["S"], 1), w.hidden, W.y_seed(w)).view(torch.int16).numpy() \
        .view(np.uint16)
    cap = oracle.max_slots(N, w.num_topk, w.num_experts, w.expert_alignment)
    recv = np.zeros((cap, w.hidden), np.uint16 if w.quant == 0 else np.uint8)
    scales = np.zeros((cap, w.hidden // w.quant_group), np.float32) if w.quant else None
    out = np.zeros((N, w.hidden), np.uint16)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.layout(idx, w.num_experts, w.num_ranks, w.ranks_per_node)
        s = oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment)
        for b, e in W.round_ranges(N, w.rounds):
            oracle.dispatch(x, s["slot_idx"], cap, quant=w.quant, group=w.quant_group or None,
                            t_begin=b, t_end=e, recv_x=recv, recv_scales=scales)
        for b, e in W.round_ranges(N, w.rounds):
            oracle.combine(y, wts, s["slot_idx"], t_begin=b, t_end=e, out=out)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=N * reps / el, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{reps} full pass(es) of the {w.name} workload ({N} tokens: layout, "
                       f"slots, dispatch, combine), serial C, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_30b_a3b_prefill")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this path runs on "
              "one GPU's share of an EP step, with destination ranks simulated as partitions "
              "of one HBM buffer.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    from combine_get_dispatch_layout_amd import ep

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    idx, wts = W.routing(w)
    N, H = w.num_tokens, w.hidden
    V = int((idx >= 0).sum())
    cfg = ep.Config(hidden=H, num_topk=w.num_topk, num_experts=w.num_experts,
                    num_ranks=w.num_ranks, ranks_per_node=w.ranks_per_node,
                    expert_alignment=w.expert_alignment, quant=w.quant,
                    quant_group=w.quant_group if w.quant else 0)
    cap = ep.ep_recv_capacity(cfg, N)
    rdt = {0: torch.bfloat16, 1: torch.uint8, 2: torch.int8}[w.quant]
    G = cfg.num_groups
    rounds = W.round_ranges(N, w.rounds)

    # bytes touched per set; rotate sets so one cycle is >= 1 GiB
    per_set = 2 * N * H * 2 + cap * H * (2 if w.quant == 0 else 1) + cap * H * 2
    nsets = args.sets or max(2, min(8, -(-(1 << 30) // per_set)))
    sets = []
    topk_d = torch.from_numpy(idx).to(dev)
    wts_d = torch.from_numpy(wts).to(dev)
    for i in range(nsets):
        s = dict(h=ep.ep_handle_init(cfg, N, device=dev),
                 topk=topk_d.clone(), wts=wts_d.clone(),
                 x=W.activations(N, H, W.x_seed(w) + i, device=dev),
                 y=W.activations(cap, H, W.y_seed(w) + i, device=dev),
                 recv=torch.empty((cap, H), dtype=rdt, device=dev),
                 scales=torch.empty((cap, G), dtype=torch.float32, device=dev) if w.quant else None,
                 out=torch.empty((N, H), dtype=torch.bfloat16, device=dev),
                 per_rank=torch.empty(w.num_ranks, dtype=torch.int32, device=dev),
                 per_expert=torch.empty(w.num_experts, dtype=torch.int32, device=dev),
                 per_node=(torch.empty(cfg.num_nodes, dtype=torch.int32, device=dev)
                           if cfg.num_nodes else None),
                 in_rank=torch.empty((N, w.num_ranks), dtype=torch.bool, device=dev))
        sets.append(s)
    # S from one synced layout (for the byte counts)
    S = ep.ep_get_layout(sets[0]["h"], sets[0]["topk"], do_cpu_sync=True)["num_recv_slots"]
    nbytes = algorithmic_bytes(w, V, S)
    stream = torch.cuda.current_stream()
    for s in sets:
        s["calls"] = (
            [ep.bind_get_layout(s["h"], s["topk"], s["per_rank"], s["per_node"], s["per_expert"],
                                s["in_rank"], stream=stream)],
            [ep.bind_dispatch(s["h"], s["x"], s["recv"], s["scales"], b, e, stream=stream)
             for b, e in rounds],
            [ep.bind_combine(s["h"], s["y"], s["wts"], s["out"], b, e, stream=stream)
             for b, e in rounds])

    def step(i, ev=None):
        lay_calls, dis_calls, com_calls = sets[i % nsets]["calls"]
        if ev is not None:
            ev[0].record(stream)
        for c in lay_calls:
            c()
        if ev is not None:
            ev[1].record(stream)
        for c in dis_calls:
            c()
        if ev is not None:
            ev[2].record(stream)
        for c in com_calls:
            c()
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    lay = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    dis = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    com = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    ms_per_step = wall / args.steps * 1e3
    value = N * args.steps / wall
    t_dc = float(np.mean(dis) + np.mean(com))

    # per-launch means (one dispatch/combine launch per round)
    nr = len(rounds)
    stages = dict(layout=(float(np.mean(lay)), nbytes["layout"], 1),
                  dispatch=(float(np.mean(dis)), nbytes["dispatch"], nr),
                  combine=(float(np.mean(com)), nbytes["combine"], nr))
    dom = max(("dispatch", "combine"), key=lambda k: stages[k][0])
    t_dom, b_dom, launches = stages[dom]
    achieved = b_dom / t_dom / 1e9
    traffic = traffic_from_profiles(dom, w.name)

    # achievable reference: a plain 1 GiB device copy
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    bb = torch.empty_like(a)
    for _ in range(3):
        bb.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        bb.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, bb

    line = {
        "metric": "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), "
                  "Qwen3-30B-A3B shape",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {0: "bf16", 1: "bf16->fp8_e4m3fn", 2: "bf16->int8"}[w.quant],
        "data": "synthetic (seeded routing and N(0,1) activations)",
        "config": {"workload": w.name, "num_tokens": N, "hidden": H,
                   "num_experts": w.num_experts, "num_ranks": w.num_ranks,
                   "num_topk": w.num_topk, "expert_alignment": w.expert_alignment,
                   "rounds": len(rounds), "buffer_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": b_dom / launches,
                     "launches_per_step": launches},
        "stages_us": {k: v[0] * 1e6 for k, v in stages.items()},
        "stages_GBps": {k: v[1] / v[0] / 1e9 for k, v in stages.items()},
        "dispatch_combine": {"tokens_per_s": N / t_dc,
                             "GBps": (nbytes["dispatch"] + nbytes["combine"]) / t_dc / 1e9,
                             "frac_of_peak": (nbytes["dispatch"] + nbytes["combine"]) / t_dc / 1e9
                             / HBM_PEAK_GBS},
        "device_copy_GBps": copy_gbs,
        "recv_rows": S, "valid_pairs": V,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, idx, wts)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
