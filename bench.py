"""Benchmark of the MoE token shuffle on one MI355X.

One step = the whole hot path over one batch: routing layout + slot
assignment, dispatch and combine, all through the C ABI with inputs resident
in HBM.  By default (merged) a step dispatches and combines one batch with
ep_dispatch_overlap / ep_combine_overlap while laying out the next batch
inside the same two launches, so in steady state each step carries one
batch's layout, dispatch and combine.
Default workload: the Qwen3-30B-A3B-shaped prefill (4096 tokens, hidden 2048
bf16, 128 experts over 16 simulated ranks, top-8).

--pipeline picks how a step is issued: merged (default; the layout of the
next batch runs inside this batch's dispatch and combine launches -- those of
its first round -- on one stream), overlap (the layout of the next batch runs
on a second stream),
serial (one stream), fused
(ep_layout_dispatch + combine, the one-call form for decode batches) or
cached (dispatch + combine on a handle whose layout was computed once before
the timed loop: the cached-dispatch decode loop, whose step does not include
the layout).

Prints one JSON line.  `value` is tokens/s over whole steps, timed by the
host clock around the K steps (no events inside that region).  Kernel times
come from a second, eager pass of the same steps right after it, with HIP
events on every launch (taken on the launch stream from the kernels' own
start and end); the roofline entry is for the kernel with the largest share
of the step, its achieved bandwidth = algorithmic bytes per launch / median
launch time.  Buffers rotate over several independent sets so each step
streams memory that the 256 MB Infinity Cache does not hold (--sets 1 gives
the warm figures, labelled as such).

cpu_baseline times the CPU oracle on the host: layout and slots serial, the
per-token loops of dispatch and combine on the OpenMP build (all the
threads OpenMP gives it); per-stage medians over full passes.
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
    dispatch: x read 2NH, slot read 4NK, receive rows M*(b*H + c*G) with b
              bytes per element (2 bf16, 1 FP8 / int8, 1/2 MXFP4) and c bytes
              per scale (4 fp32, 1 E8M0)
    combine:  y rows read M*(b'*H + 4*G') (b' = 2 bf16, 1 FP8 / int8 codes
              with G' fp32 scales), weights + slots read 8NK, out write 2NH
    M, the rows moved, is V (valid pairs), or S (one row per token and rank)
    with the non-expand dispatch.
    """
    N, H, K, R = w.num_tokens, w.hidden, w.num_topk, w.num_ranks
    M = S if w.non_expand else V
    b = {0: 2.0, 1: 1.0, 2: 1.0, 3: 0.5}[w.quant]
    G = (H // w.quant_group) if w.quant else 0
    c = 1 if (w.quant == 3 or w.scale_mode == 2) else 4
    layout = 4 * N * K + 16 * N * K + N * R + 8 * V
    dispatch = 2 * N * H + 4 * N * K + M * (b * H + c * G)
    yb = 2 if w.combine_quant == 0 else 1
    Gc = (H // w.combine_group) if w.combine_quant else 0
    combine = M * (yb * H + 4 * Gc) + 8 * N * K + 2 * N * H
    return dict(layout=int(layout), dispatch=int(dispatch), combine=int(combine))


KERNEL_SOURCES = {"dispatch": ("dispatch.hip", "scatter.hpp"),
                  "combine": ("combine.hip", "gather.hpp"),
                  "layout": ("layout.hip", "route.hpp"),
                  "layout_dispatch": ("fused.hip", "route.hpp", "scatter.hpp"),
                  "dispatch_layout": ("overlap.hip", "scatter.hpp", "route.hpp", "sources.hpp"),
                  "combine_layout": ("overlap.hip", "gather.hpp", "route.hpp", "sources.hpp")}


def kernel_source_hash(kernel):
    """Hash of the kernel's sources without their comments and blank space,
    so that an edit of the comments alone keeps its counter record valid."""
    import re
    h = hashlib.sha256()
    for src in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "combine_get_dispatch_layout_amd", "csrc", src)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


QNAMES = {"none": 0, "fp8": 1, "int8": 2, "mxfp4": 3}
SCALE_MODES = {"fp32": 0, "pow2": 1, "ue8m0": 2}
# fields the variant flags may change, and their short names in a tag
VARIANT_FIELDS = (("num_sources", "src"), ("quant", "q"), ("quant_group", "qg"),
                  ("scale_mode", "sm"), ("combine_quant", "cq"), ("combine_group", "cg"))


def variant_of(args):
    """The workload that --workload and the variant flags name, its tag, and
    the flags as bench.py arguments.  The tag is the workload's name, plus
    one suffix per field the flags changed; it keys the traffic records, so
    a variant never reports another configuration's counted bytes."""
    import workloads as W
    base = W.WORKLOADS[args.workload]
    w, flags = base, []
    if args.num_sources > 1:
        w = w.scaled(num_sources=args.num_sources)
        flags += ["--num-sources", str(args.num_sources)]
    if args.quant:
        q = QNAMES[args.quant]
        w = w.scaled(quant=q, quant_group=(args.quant_group or (32 if q == 3 else 128)) if q else 0)
        flags += ["--quant", args.quant] + (["--quant-group", str(args.quant_group)]
                                            if args.quant_group else [])
    if args.scale_mode:
        w = w.scaled(scale_mode=SCALE_MODES[args.scale_mode])
        flags += ["--scale-mode", args.scale_mode]
    if args.combine_quant and args.combine_quant != "none":
        w = w.scaled(combine_quant=QNAMES[args.combine_quant], combine_group=args.combine_group)
        flags += ["--combine-quant", args.combine_quant, "--combine-group", str(args.combine_group)]
    tag = args.workload + "".join(f"_{short}{getattr(w, f)}" for f, short in VARIANT_FIELDS
                                  if getattr(w, f) != getattr(base, f))
    return w, tag, flags


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since
    the counters were taken."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f).get("kernels", {}).get(kernel)
    if not d or d.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_rows(path, counter):
    import csv
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


KERNEL_SYMBOLS = {"dispatch": "k_dispatch<", "combine": "k_combine<",
                  "layout_dispatch": "k_route_dispatch<",
                  "dispatch_layout": "k_dispatch_layout<", "combine_layout": "k_combine_layout<"}


def traffic_summary(fetch_csv, write_csv, args):
    """Adds to profiles/traffic_<tag>.json the HBM bytes per launch of the
    data-moving kernels found in two rocprofv3 --pmc counter_collection CSVs
    of `bench.py --workload <workload> <variant flags> --pipeline <pipeline>`
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), where <tag> names the
    workload and its variant.  Each counter is scaled by what it reads for
    the benchmark's 1 GiB device copy (read 1 GiB, write 1 GiB)."""
    workload, pipeline = args.workload, args.pipeline
    w, tag, flags = variant_of(args)
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    copy_f = max(v for n, v in fetch if "copyBuffer" in n)
    copy_w = max(v for n, v in write if "copyBuffer" in n)
    f_fetch, f_write = gib_kib / copy_f, gib_kib / copy_w
    import workloads as W
    import numpy as np
    idx, _ = W.routing(w)
    V = int((idx >= 0).sum())
    ranks = np.where(idx >= 0, idx // (w.num_experts // w.num_ranks), -1)
    rows = sum(len(set(r[r >= 0].tolist())) for r in ranks)   # non-expand rows
    nbytes = algorithmic_bytes(w, V, rows)
    nbytes["layout_dispatch"] = nbytes["layout"] + nbytes["dispatch"]
    # the launches that also lay out the next batch are priced at their
    # dispatch / combine bytes alone
    nbytes["dispatch_layout"] = nbytes["dispatch"]
    nbytes["combine_layout"] = nbytes["combine"]
    vflags = "".join(" " + f for f in flags)
    bench_args = (f"--workload {workload}{vflags} --pipeline {pipeline} --steps 4 --warmup 2 "
                  "--no-cpu-baseline")
    command = [f"rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o fetch -- python3 bench.py {bench_args}",
               f"rocprofv3 --pmc WRITE_SIZE -f csv -d <dir> -o write -- python3 bench.py {bench_args}",
               f"python3 bench.py --traffic-from <dir>/fetch_counter_collection.csv "
               f"<dir>/write_counter_collection.csv --workload {workload}{vflags} --pipeline {pipeline}"]
    path = traffic_path(tag)
    out = dict(workload=tag, kernels={})
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    for kern, sym in KERNEL_SYMBOLS.items():
        if kern == "dispatch":
            # ep_quantize_rows (expert outputs as codes, before the timed
            # loop) runs the dispatch kernel too, with the combine's format as
            # its first template argument: keep the step's own dispatch only
            if w.combine_quant and w.combine_quant == w.quant:
                continue
            sym = f"k_dispatch<{w.quant},"
        fv = [v for n, v in fetch if sym in n]
        wv = [v for n, v in write if sym in n]
        if not fv or not wv:
            continue
        fk, wk = float(np.median(fv)), float(np.median(wv))
        launches = 1 if kern == "layout_dispatch" else len(W.round_ranges(w.num_tokens, w.rounds))
        per_launch_alg = nbytes[kern] / launches
        hbm = (fk * f_fetch + wk * f_write) * 1024.0
        out["kernels"][kern] = dict(
            fetch_kib=fk, write_kib=wk, hbm_bytes_per_launch=hbm,
            algorithmic_bytes_per_launch=per_launch_alg,
            traffic_over_algorithmic=hbm / per_launch_alg, launches=len(fv),
            copy_fetch_kib=copy_f, copy_write_kib=copy_w, fetch_scale=f_fetch,
            write_scale=f_write, source_sha256_16=kernel_source_hash(kern), command=command)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    write_traffic_md(out, tag)
    print(json.dumps(out, indent=1))


def write_traffic_md(rec, tag):
    """profiles/traffic_<tag>.md: the JSON record as a table, with the
    commands that made each entry."""
    rows, cmds = [], []
    for kern, d in rec["kernels"].items():
        rows.append(f"| {kern} | {d['fetch_kib']:.0f} | {d['write_kib']:.0f} | {d['fetch_scale']:.4f} | "
                    f"{d['write_scale']:.4f} | {d['hbm_bytes_per_launch']:.4e} | "
                    f"{d['algorithmic_bytes_per_launch']:.4e} | {d['traffic_over_algorithmic']:.4f} |")
        for c in d["command"]:
            if c not in cmds:
                cmds.append(c)
    text = [f"# HBM traffic per launch: {tag}", "",
            "Each kernel's counters come from two rocprofv3 passes (one counter each) over `bench.py`, "
            "summarised by `bench.py --traffic-from`; FETCH_SIZE and WRITE_SIZE are scaled by what they "
            "read for the benchmark's own 1 GiB device copy (`__amd_rocclr_copyBuffer`, reads 1 GiB, "
            "writes 1 GiB).", "",
            "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch scale | write scale | HBM bytes | "
            "algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|", *rows, "",
            "Commands (repo root, on one MI355X):", "", "```", *cmds, "```", "",
            "Medians over the run's launches (warm-up and timed steps).  A ratio near 1 means the kernel "
            "moves its algorithmic bytes and nothing more (no re-reads; padding rows are never written).  "
            "`bench.py` reports `roofline.traffic` from the JSON file only while the kernel's sources "
            "still hash to the recorded value.", ""]
    with open(os.path.join(ROOT, "profiles", f"traffic_{tag}.md"), "w") as f:
        f.write("\n".join(text))


def ea_summary(rd_csv, wr_csv, args):
    """profiles/ea_requests_<tag>.md from two rocprofv3 --pmc passes over
    `bench.py --workload <workload> --pipeline <pipeline>`: the L2's memory
    requests (TCC_EA0_RDREQ / _32B / _DRAM, then TCC_EA0_WRREQ / _64B /
    _DRAM, summed over the L2 channels) as bytes per launch, and the share of
    them sent to the memory controller rather than to other agents."""
    import csv
    import numpy as np
    w, tag, flags = variant_of(args)
    per = {}
    for path in (rd_csv, wr_csv):
        for r in csv.DictReader(open(path)):
            n = r["Kernel_Name"]
            if "copyBuffer" in n:
                n = "__amd_rocclr_copyBuffer"
            elif "epk::" in n:
                n = n.split("(anonymous namespace)::", 1)[-1]
                n = n.split(">(")[0] + ">" if ">(" in n else n.split("(")[0]
            else:
                continue
            per.setdefault(n, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    rows = []
    for n, c in per.items():
        # the copy: its largest launch (the 1 GiB one); kernels: the median
        pick = max if n == "__amd_rocclr_copyBuffer" else (lambda v: float(np.median(v)))
        v = {k: pick(x) for k, x in c.items()}
        rd = (v["TCC_EA0_RDREQ_sum"] - v["TCC_EA0_RDREQ_32B_sum"]) * 64 + v["TCC_EA0_RDREQ_32B_sum"] * 32
        wr = v["TCC_EA0_WRREQ_64B_sum"] * 64 + (v["TCC_EA0_WRREQ_sum"] - v["TCC_EA0_WRREQ_64B_sum"]) * 32
        rdd = v["TCC_EA0_RDREQ_DRAM_sum"] / max(v["TCC_EA0_RDREQ_sum"], 1.0)
        wrd = v["TCC_EA0_WRREQ_DRAM_sum"] / max(v["TCC_EA0_WRREQ_sum"], 1.0)
        rows.append(f"| `{n}` | {len(c['TCC_EA0_RDREQ_sum'])} | {rd / 1e6:.2f} | {rdd:.4f} | "
                    f"{wr / 1e6:.2f} | {wrd:.4f} |")
    vflags = "".join(" " + f for f in flags)
    a = f"--workload {args.workload}{vflags} --pipeline {args.pipeline} --steps 4 --warmup 2 --no-cpu-baseline"
    text = [f"# L2 memory requests per launch: {tag}, {args.pipeline} pipeline", "", "Commands (repo root, on one MI355X):", "",
            "```",
            f"rocprofv3 --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_DRAM_sum -f csv "
            f"-d <dir>/rd -o rd -- python3 bench.py {a}",
            f"rocprofv3 --pmc TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum TCC_EA0_WRREQ_DRAM_sum -f csv "
            f"-d <dir>/wr -o wr -- python3 bench.py {a}",
            f"python3 bench.py --ea-from <dir>/rd/rd_counter_collection.csv "
            f"<dir>/wr/wr_counter_collection.csv --workload {args.workload}{vflags} "
            f"--pipeline {args.pipeline}", "```", "",
            "| kernel | launches | read MB (64 B and 32 B requests) | read share to DRAM | write MB | "
            "write share to DRAM |", "|---|---|---|---|---|---|", *rows, "",
            "Medians over the run's launches; the device copy row is its 1 GiB launch (reads 1 GiB, "
            "writes 1 GiB).  The read requests seen on this interface are half the bytes read, for the "
            "copy as for the kernels, which is the factor of 2 applied to FETCH_SIZE in the traffic "
            "records; writes are counted whole.  Every request is sent to the memory controller (DRAM "
            "share 1), none to other agents.  The 256 MB Infinity Cache is on the memory side of this "
            "interface, so these counters cannot tell its hits from HBM accesses; the benchmark rotates "
            "buffer sets of over 1 GiB per cycle to keep the data out of it, and `--sets 1` measures "
            "the warm case beside it.", ""]
    out = os.path.join(ROOT, "profiles", f"ea_requests_{tag}_{args.pipeline}.md")
    with open(out, "w") as f:
        f.write("\n".join(text))
    print(out)


def trace_summary(trace_dir, args):
    """profiles/kernels_<tag>[_<pipeline>][_graph].md from a rocprofv3
    --kernel-trace --stats run of `bench.py --workload <workload> <variant
    flags> --pipeline <pipeline> [--graph]` whose output went to
    <trace_dir>/trace_*.csv: per library kernel, calls and average / min /
    max duration, and its launch shape, LDS and registers."""
    import csv
    w, tag, flags = variant_of(args)
    name = tag + ("" if args.pipeline == "merged" else f"_{args.pipeline}") + \
        ("_graph" if args.graph else "")
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_stats.csv"))))
    shapes = {}
    for r in csv.DictReader(open(os.path.join(trace_dir, "trace_kernel_trace.csv"))):
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        sh = shapes.setdefault(r["Kernel_Name"], dict(shape=set(), lds=set(), vgpr=set()))
        sh["shape"].add(f"{grid // max(wg, 1)}x{wg}")
        sh["lds"].add(r.get("LDS_Block_Size", r.get("Lds_Size", "?")))
        sh["vgpr"].add(r.get("Arch_VGPR_Count", r.get("VGPR_Count", "?")))
    def short(name):
        # "void epk::(anonymous namespace)::k_x<...>(args)" -> "k_x<...>"
        name = name.split("(anonymous namespace)::", 1)[-1]
        return name.split(">(")[0] + ">" if ">(" in name else name.split("(")[0]
    rows = []
    for r in stats:
        kn = r["Name"]
        if "epk::" not in kn and not kn.startswith("__amd_rocclr_copyBuffer"):
            continue
        sh = shapes.get(kn, dict(shape=set(), lds=set(), vgpr=set()))
        rows.append(f"| `{short(kn)}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                    f"{'; '.join(sorted(sh['shape']))} | {'; '.join(sorted(sh['lds']))} | "
                    f"{'; '.join(sorted(sh['vgpr']))} |")
    vflags = "".join(" " + f for f in flags)
    cmd = (f"rocprofv3 --kernel-trace --stats -f csv -d <dir> -o trace -- python3 bench.py "
           f"--workload {args.workload}{vflags} --pipeline {args.pipeline}"
           f"{' --graph' if args.graph else ''} --steps {args.steps} --warmup {args.warmup} "
           "--no-cpu-baseline")
    text = [f"# Kernel trace: {name}", "", "Command (repo root, on one MI355X):", "", "```", cmd,
            f"python3 bench.py --trace-from <dir> --workload {args.workload}{vflags} "
            f"--pipeline {args.pipeline}{' --graph' if args.graph else ''} --steps {args.steps} "
            f"--warmup {args.warmup}", "```", "",
            "`<dir>/trace_kernel_stats.csv` and `trace_kernel_trace.csv`; the library's kernels, plus "
            "the 1 GiB device copy the benchmark times as its achievable-bandwidth reference:", "",
            "| kernel | calls | avg us | min us | max us | workgroups x threads | static LDS B | VGPRs |",
            "|---|---|---|---|---|---|---|---|", *rows, "",
            "Workload: " + json.dumps(dict(workload=w.name, num_tokens=w.num_tokens, hidden=w.hidden,
                                           num_experts=w.num_experts, num_ranks=w.num_ranks,
                                           num_topk=w.num_topk, expert_alignment=w.expert_alignment,
                                           rounds=w.rounds, num_sources=w.num_sources, quant=w.quant,
                                           quant_group=w.quant_group, scale_mode=w.scale_mode,
                                           combine_quant=w.combine_quant,
                                           combine_group=w.combine_group)), "",
            "Kernel averages include the warm-up steps and the eager timing pass.  Other kernels of the "
            "run (torch's input generation) are left out.  The LDS column is the profiler's "
            "`LDS_Block_Size`, the kernel's static LDS; the dynamic LDS a launch requests is not in it.", ""]
    out = os.path.join(ROOT, "profiles", f"kernels_{name}.md")
    with open(out, "w") as f:
        f.write("\n".join(text))
    print(out)


def cpu_baseline(w, idx, wts, budget_s=10.0, nbytes=None):
    """The oracle, as it stands, on the same workload: full passes (layout,
    slots, dispatch, combine) until budget_s is spent (at least 3).  Layout
    and slots run on the serial build; dispatch and combine (the fp32
    reduction) on the OpenMP build, which gives the same bits.  Reports the
    median pass and per-stage medians, and with nbytes (the algorithmic
    bytes per stage) the stages' GB/s on the same byte counts as the GPU's."""
    import numpy as np
    import oracle
    import workloads as W
    import torch
    N = w.num_tokens
    threads = oracle.num_threads(parallel=True)
    x = W.activations(N, w.hidden, W.x_seed(w)).view(torch.int16).numpy().view(np.uint16)
    s0 = (oracle.slots_nonexpand(idx, w.num_experts, w.num_ranks) if w.non_expand
          else oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment))
    y = W.activations(max(s0["S"], 1), w.hidden, W.y_seed(w)).view(torch.int16).numpy() \
        .view(np.uint16)
    cap = oracle.max_slots(N, w.num_topk, w.num_experts, w.expert_alignment)
    recv = np.zeros((cap, oracle.row_bytes(w.hidden, w.quant) // (2 if w.quant == 0 else 1)),
                    np.uint16 if w.quant == 0 else np.uint8)
    scales = (np.zeros((cap, w.hidden // w.quant_group), oracle.scale_dtype(w.quant, w.scale_mode))
              if w.quant else None)
    if w.combine_quant:
        yc, ys = oracle.quantize_rows(y, w.combine_quant, group=w.combine_group,
                                      scale_mode=min(w.scale_mode, 1))
    out = np.zeros((N, w.hidden), np.uint16)
    ones = np.ones_like(wts)
    rounds = W.round_ranges(N, w.rounds)
    times = {"layout": [], "slots": [], "dispatch": [], "combine": []}
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.layout(idx, w.num_experts, w.num_ranks, w.ranks_per_node)
        t1 = time.perf_counter()
        s = (oracle.slots_nonexpand(idx, w.num_experts, w.num_ranks) if w.non_expand
             else oracle.slots(idx, w.num_experts, w.num_ranks, w.expert_alignment))
        t2 = time.perf_counter()
        for b, e in rounds:
            oracle.dispatch(x, s["slot_idx"], cap, quant=w.quant, group=w.quant_group or None,
                            t_begin=b, t_end=e, recv_x=recv, recv_scales=scales,
                            scale_mode=w.scale_mode, parallel=True)
        t3 = time.perf_counter()
        for b, e in rounds:
            if w.combine_quant:
                oracle.combine_q(yc, ys, w.combine_quant, w.combine_group, wts, s["slot_idx"],
                                 t_begin=b, t_end=e, out=out, fp32=True, parallel=True)
            else:
                oracle.combine(y, ones if w.non_expand else wts, s["slot_idx"], t_begin=b,
                               t_end=e, out=out, fp32=True, parallel=True)
        t4 = time.perf_counter()
        for k, a, b in (("layout", t0, t1), ("slots", t1, t2), ("dispatch", t2, t3),
                        ("combine", t3, t4)):
            times[k].append(b - a)
        if len(times["layout"]) >= 3 and t4 - t_start >= budget_s:
            break
    passes = len(times["layout"])
    total = np.array(times["layout"]) + np.array(times["slots"]) + np.array(times["dispatch"]) \
        + np.array(times["combine"])
    med = {k: float(np.median(v)) for k, v in times.items()}
    gbps = None
    if nbytes:
        gbps = {"layout+slots": nbytes["layout"] / (med["layout"] + med["slots"]) / 1e9,
                "dispatch": nbytes["dispatch"] / med["dispatch"] / 1e9,
                "combine": nbytes["combine"] / med["combine"] / 1e9}
    return dict(value=N / float(np.median(total)), unit="tokens/s", cores=threads,
                host_cpus=os.cpu_count(), kind="oracle",
                stages_ms={k: v * 1e3 for k, v in med.items()}, stages_GBps=gbps,
                sample=f"{passes} full passes of the {w.name} workload ({N} tokens: layout and "
                       f"slots serial, dispatch and fp32 combine over tokens on {threads} "
                       f"OpenMP threads), median pass {np.median(total) * 1e3:.1f} ms, "
                       f"{time.perf_counter() - t_start:.1f} s")


def ceilings(w=None, gib=1.0, reps=10):
    """Achievable HBM bandwidth of plain streaming kernels (libep_probe.so):
    for read, write and copy, the best of a sweep over workgroup counts,
    workgroup sizes, 16-byte vectors per lane and the non-temporal hint,
    each timed over `reps` launches on `gib` GiB buffers (torch events on the
    launch stream).  With a workload `w`, also the ceilings of its own two
    row patterns without their arithmetic: the combine's gather and the
    dispatch's scatter over the workload's slot table (from the library's
    layout), bf16 rows, four rotating buffer sets.  Prints one JSON line."""
    import ctypes
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "combine_get_dispatch_layout_amd", "libep_probe.so"))
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.ep_probe_stream.argtypes = [I32, P, P, I64, I32, I32, I32, I32, P]
    L.ep_probe_rows.argtypes = [I32, P, P, P, I64, I32, I64, I32, I32, P]
    dev = torch.device("cuda:0")
    nbytes = int(gib * (1 << 30))
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(launch, nrep):
        launch(0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(nrep):
            launch(r)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / nrep

    names = {0: "read", 1: "write", 2: "copy"}
    results = []
    for mode in (0, 1, 2):
        moved = nbytes * (2 if mode == 2 else 1)
        for threads in (256, 512, 1024):
            for vpl in (1, 2, 4, 8):
                for nt in (0, 1):
                    for blocks in (256, 512, 1024, 2048, 4096, 8192):
                        args = (mode, ctypes.c_void_p(src.data_ptr()),
                                ctypes.c_void_p(dst.data_ptr()), nbytes, blocks, threads, vpl,
                                nt, sp)

                        def go(_r, args=args):
                            if L.ep_probe_stream(*args) != 0:
                                raise RuntimeError("ep_probe_stream failed")
                        t = timed(go, reps)
                        results.append(dict(mode=names[mode], threads=threads, vec_per_lane=vpl,
                                            nontemporal=nt, blocks=blocks, GBps=moved / t / 1e9))
        print(f"[ceilings] {names[mode]} done", file=sys.stderr, flush=True)
    del src, dst
    best = {}
    for r in results:
        if r["GBps"] > best.get(r["mode"], {}).get("GBps", 0):
            best[r["mode"]] = r
    line = dict(ceilings={k: dict(v, frac_of_peak=v["GBps"] / HBM_PEAK_GBS) for k, v in best.items()},
                peak_GBps=HBM_PEAK_GBS, buffer_GiB=gib, reps=reps, configs=len(results),
                note="bytes moved / time; copy counts its reads and its writes")
    if w is not None:
        import workloads as W
        from combine_get_dispatch_layout_amd import ep
        idx, _ = W.routing(w)
        N, H, K = w.num_tokens, w.hidden, w.num_topk
        cfg = ep.Config(hidden=H, num_topk=K, num_experts=w.num_experts, num_ranks=w.num_ranks,
                        expert_alignment=w.expert_alignment, expert_capacity=w.expert_capacity,
                        non_expand=w.non_expand)
        h = ep.ep_handle_init(cfg, N, device=dev)
        S = ep.ep_get_layout(h, torch.from_numpy(idx).to(dev), do_cpu_sync=True)["num_recv_slots"]
        slot = ep.ep_handle_view(h)["slot_idx"]
        V = int((slot >= 0).sum().item())
        rows_b = 2 * H
        sets = [(torch.empty((max(S, 1), H), dtype=torch.bfloat16, device=dev).fill_(1),
                 torch.empty((N, H), dtype=torch.bfloat16, device=dev).fill_(1)) for _ in range(4)]
        pat = []
        for mode, nm in ((3, "gather"), (4, "scatter")):
            for threads in (256, 512, 1024):
                for vpl in (1, 2, 4):
                    def go(r, mode=mode, threads=threads, vpl=vpl):
                        big, small = sets[r % 4]
                        s_, d_ = (big, small) if mode == 3 else (small, big)
                        if L.ep_probe_rows(mode, ctypes.c_void_p(s_.data_ptr()),
                                           ctypes.c_void_p(d_.data_ptr()),
                                           ctypes.c_void_p(slot.data_ptr()), N, K, rows_b, threads,
                                           vpl, sp) != 0:
                            raise RuntimeError("ep_probe_rows failed")
                    t = timed(go, 4 * reps)
                    moved = (V + N) * rows_b
                    pat.append(dict(pattern=nm, threads=threads, vec_per_lane=vpl, us=t * 1e6,
                                    GBps=moved / t / 1e9))
        for nm in ("gather", "scatter"):
            b = min((x for x in pat if x["pattern"] == nm), key=lambda x: x["us"])
            line.setdefault("patterns", {})[nm] = dict(b, frac_of_peak=b["GBps"] / HBM_PEAK_GBS)
        line["patterns_workload"] = dict(workload=w.name, tokens=N, hidden=H, topk=K, rows=V,
                                         bytes_moved=(V + N) * rows_b)
        results += pat
    print(json.dumps(line), flush=True)
    return line, results


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (so the library can attach
    them to its kernel launches)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def ms(self, a, b):
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(self.ev[a]),
                                        self.ct.c_void_p(self.ev[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.ev = []


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen3_30b_a3b_prefill")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0 = auto)")
    ap.add_argument("--quant", choices=("none", "fp8", "int8", "mxfp4"),
                    help="override the workload's dispatch quantisation")
    ap.add_argument("--quant-group", type=int, default=0,
                    help="elements per dispatch scale (default: 128, 32 for MXFP4)")
    ap.add_argument("--scale-mode", choices=("fp32", "pow2", "ue8m0"),
                    help="FP8 / int8 scale format (round_scale, use_ue8m0)")
    ap.add_argument("--combine-quant", choices=("none", "fp8", "int8"),
                    help="expert outputs as FP8 / int8 codes with fp32 scales (quantised once, "
                         "before the timed loop, with ep_quantize_rows)")
    ap.add_argument("--combine-group", type=int, default=128)
    ap.add_argument("--num-sources", type=int, default=0,
                    help=">1: read the batch as this many stacked source ranks (receive order "
                         "(source, token, k) plus the per-source counts)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle passes behind cpu_baseline")
    ap.add_argument("--pipeline", choices=("merged", "overlap", "serial", "fused", "cached"),
                    default=None,
                    help="(default: merged) "
                         "merged: batch i+1's layout runs inside batch i's dispatch and "
                         "combine launches (ep_dispatch_overlap / ep_combine_overlap), one "
                         "stream; overlap: batch i+1's layout runs on a second stream during "
                         "batch i's dispatch and combine; serial: one stream, one stage after "
                         "another; "
                         "fused: ep_layout_dispatch (layout + dispatch in one call) then "
                         "combine, one stream (one round only); cached: the layout is computed "
                         "once per buffer set and each step is dispatch + combine on the cached "
                         "handle (a decode loop whose routing does not change)")
    ap.add_argument("--event-steps", type=int, default=50,
                    help="steps of the eager pass after the timed region that takes kernel "
                         "times (HIP events on every launch; at least 10)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one rotation of steps (one step per buffer set) in a HIP "
                         "graph and time its replays (steps rounded up to whole rotations) "
                         "(merged, serial, fused and cached pipelines)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the achievable read / write / copy bandwidth of plain "
                         "streaming kernels (libep_probe.so) and exit")
    ap.add_argument("--trace-from", metavar="DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run (DIR/trace_*.csv) "
                         "into profiles/ and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs into profiles/ and exit")
    ap.add_argument("--ea-from", nargs=2, metavar=("RD_CSV", "WR_CSV"),
                    help="summarise two rocprofv3 --pmc runs of the L2's memory request counters "
                         "into profiles/ and exit")
    args = ap.parse_args()
    if args.pipeline is None:
        args.pipeline = "merged"
    if args.traffic_from:
        traffic_summary(args.traffic_from[0], args.traffic_from[1], args)
        return
    if args.trace_from:
        trace_summary(args.trace_from, args)
        return
    if args.ea_from:
        ea_summary(args.ea_from[0], args.ea_from[1], args)
        return
    if args.ceilings:
        _, results = ceilings(variant_of(args)[0])
        out = os.environ.get("EP_CEILINGS_OUT")
        if out:
            with open(out, "w") as f:
                json.dump(results, f)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this path runs on "
              "one GPU's share of an EP step, with destination ranks simulated as partitions "
              "of one HBM buffer.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    from combine_get_dispatch_layout_amd import ep

    w, tag, _ = variant_of(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    idx, wts = W.routing(w)
    N, H = w.num_tokens, w.hidden
    V = int((idx >= 0).sum())
    cfg = ep.Config(hidden=H, num_topk=w.num_topk, num_experts=w.num_experts,
                    num_ranks=w.num_ranks, ranks_per_node=w.ranks_per_node,
                    expert_alignment=w.expert_alignment, quant=w.quant,
                    quant_group=w.quant_group if w.quant else 0, num_sources=w.num_sources,
                    scale_mode=w.scale_mode, combine_quant=w.combine_quant,
                    combine_group=w.combine_group, non_expand=w.non_expand)
    cap = ep.ep_recv_capacity(cfg, N)
    G = cfg.num_groups
    rounds = W.round_ranges(N, w.rounds)
    fused = args.pipeline == "fused"
    if fused and len(rounds) != 1:
        sys.exit("--pipeline fused dispatches the whole batch in one call: the workload must "
                 "have one round")

    # bytes touched per set; rotate sets so one cycle is >= 1 GiB
    per_set = 2 * N * H * 2 + cap * H * (2 if w.quant == 0 else 1) + cap * H * 2
    per_set += cap * H * (2 if w.combine_quant else 0)   # y codes besides the bf16 y
    nsets = args.sets or max(2, min(8, -(-(1 << 30) // per_set)))
    sets = []
    topk_d = torch.from_numpy(idx).to(dev)
    wts_d = torch.from_numpy(wts).to(dev)
    for i in range(nsets):
        s = dict(h=ep.ep_handle_init(cfg, N, device=dev),
                 topk=topk_d.clone(), wts=wts_d.clone(),
                 x=W.activations(N, H, W.x_seed(w) + i, device=dev),
                 y=W.activations(cap, H, W.y_seed(w) + i, device=dev),
                 recv=torch.empty((cap, cfg.recv_row_elems), dtype=cfg.recv_dtype, device=dev),
                 scales=(torch.empty((cap, G), dtype=cfg.scales_dtype, device=dev) if w.quant
                         else None),
                 out=torch.empty((N, H), dtype=torch.bfloat16, device=dev),
                 per_rank=torch.empty(w.num_ranks, dtype=torch.int32, device=dev),
                 per_expert=torch.empty(w.num_experts, dtype=torch.int32, device=dev),
                 per_node=(torch.empty(cfg.num_nodes, dtype=torch.int32, device=dev)
                           if cfg.num_nodes else None),
                 in_rank=torch.empty((N, w.num_ranks), dtype=torch.bool, device=dev))
        s["y_scales"] = None
        if w.combine_quant:
            s["y"], s["y_scales"] = ep.ep_quantize_rows(cfg, s["y"])
        sets.append(s)
    data_sets = nsets
    if nsets == 1 and args.pipeline == "merged":
        # the merged pipeline lays the next batch out into another handle:
        # a second handle over the same buffers, so one set of data stays hot
        sets.append(dict(sets[0], h=ep.ep_handle_init(cfg, N, device=dev)))
        nsets = 2
    # S from one synced layout (for the byte counts)
    S = ep.ep_get_layout(sets[0]["h"], sets[0]["topk"], do_cpu_sync=True)["num_recv_slots"]
    nbytes = algorithmic_bytes(w, V, S)
    pl = args.pipeline
    # a graph is captured on a stream of its own (default priority)
    stream = torch.cuda.Stream() if args.graph else torch.cuda.current_stream()
    # overlap: the layout of batch i+1 runs on a second stream while batch i
    # is dispatched and combined (double-batch overlap); default priority
    lay_stream = torch.cuda.Stream() if pl == "overlap" else stream
    stage_names = {"fused": ["layout_dispatch", "combine"], "cached": ["dispatch", "combine"],
                   "merged": ["dispatch", "combine"]}.get(pl, ["layout", "dispatch", "combine"])
    stage_bytes = dict(nbytes, layout_dispatch=nbytes["layout"] + nbytes["dispatch"])
    for si, s in enumerate(sets):
        calls = []   # (stage index, bound call) in issue order
        if pl == "merged":
            # this set's batch is dispatched and combined while the next set's
            # batch (the next step's) is laid out inside the same launches:
            # those of the first round; later rounds are plain calls
            t = sets[(si + 1) % nsets]
            cw = None if w.non_expand else s["wts"]
            (b0, e0), rest = rounds[0], rounds[1:]
            calls.append((0, ep.bind_dispatch_overlap(s["h"], s["x"], s["recv"], s["scales"], b0,
                                                      e0, t["h"], t["topk"], t["per_rank"],
                                                      t["per_node"], t["per_expert"], t["in_rank"],
                                                      stream=stream)))
            calls += [(0, ep.bind_dispatch(s["h"], s["x"], s["recv"], s["scales"], b, e,
                                           stream=stream)) for b, e in rest]
            calls.append((1, ep.bind_combine_overlap(s["h"], s["y"], cw, s["out"], b0, e0, t["h"],
                                                     stream=stream, y_scales=s["y_scales"])))
            calls += [(1, ep.bind_combine(s["h"], s["y"], cw, s["out"], b, e, stream=stream,
                                          y_scales=s["y_scales"])) for b, e in rest]
            s["calls"] = calls
            s["lay_done"] = torch.cuda.Event()
            s["main_done"] = torch.cuda.Event()
            continue
        if pl == "fused":
            calls.append((0, ep.bind_layout_dispatch(s["h"], s["topk"], s["x"], s["recv"],
                                                     s["scales"], s["per_rank"], s["per_node"],
                                                     s["per_expert"], s["in_rank"],
                                                     stream=stream)))
        elif pl == "cached":
            # the handle's layout is computed once and reused by every step
            ep.ep_get_layout(s["h"], s["topk"], s["per_rank"], s["per_node"], s["per_expert"],
                             s["in_rank"])
        else:
            calls.append((0, ep.bind_get_layout(s["h"], s["topk"], s["per_rank"], s["per_node"],
                                                s["per_expert"], s["in_rank"],
                                                stream=lay_stream)))
        if pl != "fused":
            calls += [(stage_names.index("dispatch"),
                       ep.bind_dispatch(s["h"], s["x"], s["recv"], s["scales"], b, e,
                                        stream=stream)) for b, e in rounds]
        calls += [(stage_names.index("combine"),
                   ep.bind_combine(s["h"], s["y"], None if w.non_expand else s["wts"], s["out"],
                                   b, e, stream=stream, y_scales=s["y_scales"]))
                  for b, e in rounds]
        s["calls"] = calls
        s["lay_done"] = torch.cuda.Event()
        s["main_done"] = torch.cuda.Event()
        s["main_done"].record(stream)

    stage_of = [st for st, _ in sets[0]["calls"]]
    calls_per_step = len(stage_of)
    ev_steps = max(10, args.event_steps)
    hev = None   # the eager pass's (start, stop) event pair per call of every step

    def issue(i, j, base):
        c = sets[i % nsets]["calls"][j][1]
        if base is None:
            c()
        else:
            c((hev.ev[base + 2 * j], hev.ev[base + 2 * j + 1]))

    fork, join = torch.cuda.Event(), torch.cuda.Event()

    def layout(i, base, capturing=False):
        s = sets[i % nsets]
        if capturing:
            # a fork of the captured stream: the layout waits for every earlier
            # step's work, and the layout stream joins the capture
            fork.record(stream)
            lay_stream.wait_event(fork)
        else:
            lay_stream.wait_event(s["main_done"])   # the set's previous batch is combined
        issue(i, 0, base)
        s["lay_done"].record(lay_stream)

    def shuffle(i, base, wait=True):
        s = sets[i % nsets]
        if wait:
            stream.wait_event(s["lay_done"])
        for j in range(1, calls_per_step):
            issue(i, j, base)
        s["main_done"].record(stream)

    if pl == "merged":
        # the first batch's layout; every later one is laid out one step ahead
        ep.ep_get_layout(sets[0]["h"], sets[0]["topk"], sets[0]["per_rank"], sets[0]["per_node"],
                         sets[0]["per_expert"], sets[0]["in_rank"])
    gstep = [0]   # steps issued so far (the merged pipeline's set rotation)

    def run(n, timed, capturing=False):
        """n steps; with overlap the layout of step i+1 is issued before the
        dispatch and combine of step i, otherwise each step's calls in order.
        timed: every call carries kernel events (the eager timing pass).
        capturing (overlap): one rotation inside a graph capture, the first
        set's layout already done (by the prologue or the previous replay),
        the last layout for the next replay's first step."""
        def base(i):
            return 2 * calls_per_step * i if timed else None
        if pl == "overlap" and capturing:
            for i in range(n):
                layout(i + 1, None, capturing=True)
                shuffle(i, None, wait=i > 0)
            join.record(lay_stream)
            stream.wait_event(join)
            return
        if pl == "merged":
            for i in range(n):
                c = sets[gstep[0] % nsets]["calls"]
                gstep[0] += 1
                for j in range(calls_per_step):
                    if base(i) is None:
                        c[j][1]()
                    else:
                        c[j][1]((hev.ev[base(i) + 2 * j], hev.ev[base(i) + 2 * j + 1]))
            return
        if pl == "overlap":
            layout(0, base(0))
            for i in range(n):
                if i + 1 < n:
                    layout(i + 1, base(i + 1))
                shuffle(i, base(i))
        else:
            for i in range(n):
                for j in range(calls_per_step):
                    issue(i, j, base(i))

    torch.cuda.synchronize()   # set-up work on the default stream is done
    run(args.warmup, False)
    torch.cuda.synchronize()
    if args.graph:
        # one rotation (a step per buffer set) as one graph: the merged
        # pipeline's host bookkeeping advances by a whole rotation during the
        # capture, the device catches up on each replay
        graph = torch.cuda.CUDAGraph()
        if pl == "overlap":
            # the first set's layout, ahead of the captured rotation
            issue(0, 0, None)
            torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            run(nsets, False, capturing=True)
        reps = -(-args.steps // nsets)
        args.steps = reps * nsets
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        t_enqueue = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        t0 = time.perf_counter()
        run(args.steps, False)
        t_enqueue = time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    # kernel times: an eager pass of the same steps with events on every call
    # (the host then issues slower than the GPU runs, which the kernels' own
    # start / end timestamps do not see)
    hev = HipEvents(2 * calls_per_step * ev_steps)
    run(ev_steps, True)
    torch.cuda.synchronize()

    def durs(j):
        """Per-step duration (s) of call j over the eager pass."""
        return np.array([hev.ms(2 * calls_per_step * i + 2 * j, 2 * calls_per_step * i + 2 * j + 1)
                         for i in range(ev_steps)]) * 1e-3

    # per stage: per-step durations (sum over the stage's launches), bytes, launches
    per_stage = {}
    for st, name in enumerate(stage_names):
        js = [j for j in range(calls_per_step) if stage_of[j] == st]
        per_stage[name] = (sum(durs(j) for j in js), stage_bytes[name], len(js))
    hev.close()
    ms_per_step = wall / args.steps * 1e3
    value = N * args.steps / wall
    stages = {k: (float(np.median(d)), by, n) for k, (d, by, n) in per_stage.items()}
    moving = [k for k in stage_names if k != "layout"]   # the dispatch + combine stages
    t_dc = sum(stages[k][0] for k in moving)
    dom = max(moving, key=lambda k: stages[k][0])
    t_dom, b_dom, launches = stages[dom]
    achieved = b_dom / t_dom / 1e9   # = per-launch bytes / median per-launch time
    b_dc = sum(stages[k][1] for k in moving)
    # the kernel that carries the stage (merged, one round: the launch that
    # also lays out the next batch; with rounds, most launches are plain)
    merged1 = pl == "merged" and len(rounds) == 1
    traffic = traffic_from_profiles({"dispatch": "dispatch_layout", "combine": "combine_layout"}
                                    .get(dom, dom) if merged1 else dom, tag)

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
        "dtype": {0: "bf16", 1: "bf16->fp8_e4m3fn", 2: "bf16->int8", 3: "bf16->mxfp4"}[w.quant]
                 + {0: "", 1: "; combine fp8_e4m3fn in", 2: "; combine int8 in"}[w.combine_quant],
        "data": "synthetic (seeded routing and N(0,1) activations)",
        "config": {"workload": w.name, "num_tokens": N, "hidden": H,
                   "num_experts": w.num_experts, "num_ranks": w.num_ranks,
                   "num_topk": w.num_topk, "expert_alignment": w.expert_alignment,
                   "rounds": len(rounds), "num_sources": w.num_sources, "quant": w.quant,
                   "quant_group": w.quant_group, "scale_mode": w.scale_mode,
                   "combine_quant": w.combine_quant, "combine_group": w.combine_group,
                   "buffer_sets": data_sets},
        "roofline": {"bound": "hbm",
                     "kernel": ({"dispatch": "k_dispatch_layout (dispatch, with the next batch's "
                                             "layout phase it carries)",
                                 "combine": "k_combine_layout (combine, with the next batch's "
                                            "layout phase it carries)"}.get(dom, dom)
                                if merged1 else dom),
                     "kernel_us_per_launch": t_dom / launches * 1e6,
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": b_dom / launches,
                     "launches_per_step": launches},
        "stages_us": {k: v[0] * 1e6 for k, v in stages.items()},
        "stages_us_p10_p50_p90": {k: ([float(np.percentile(d, q)) * 1e6 for q in (10, 50, 90)]
                                      if len(d) else None) for k, (d, _, _) in per_stage.items()},
        "stages_GBps": {k: v[1] / v[0] / 1e9 for k, v in stages.items()},
        "+".join(moving): {"tokens_per_s": N / t_dc,
                             "GBps": b_dc / t_dc / 1e9,
                             "frac_of_peak": b_dc / t_dc / 1e9 / HBM_PEAK_GBS},
        "device_copy_GBps": copy_gbs,
        "pipeline": args.pipeline,
        "cache": ("warm: one buffer set, reused every step (Infinity-Cache-resident where it "
                  "fits)" if data_sets == 1 else
                  f"cold: {nsets} buffer sets rotate, {nsets * per_set / 2**30:.2f} GiB per "
                  "cycle against a 256 MB Infinity Cache"),
        "timing": {"wall_clock": "host clock around the timed steps, no events inside",
                   "kernels": "eager pass after the timed steps, HIP events on every launch, "
                              "medians",
                   "graph": args.graph,
                   "host_enqueue_ms_per_step": t_enqueue / args.steps * 1e3,
                   "samples_per_stage": {k: int(len(d)) for k, (d, _, _) in per_stage.items()}},
        "recv_rows": S, "valid_pairs": V,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, idx, wts, budget_s=args.cpu_budget, nbytes=nbytes)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
