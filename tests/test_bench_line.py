"""The benchmark's command-line contract: `python bench.py` prints one JSON
line with the metric, the roofline of the dominant kernel and the oracle's
CPU baseline; more than one GPU is refused with a message."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_refused():
    r = _run(["--gpus", "2"], 120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.gpu
def test_default_line_has_the_contract_fields():
    # the default workload and pipeline, few steps, a short oracle budget
    print("bench.py --steps 20 --warmup 5 --cpu-budget 2", flush=True)
    r = _run(["--steps", "20", "--warmup", "5", "--cpu-budget", "2"], 300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 5
    assert line["value"] > 0 and line["config"]["workload"] == "qwen3_30b_a3b_prefill"
    rf = line["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["achieved"] < rf["peak"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert rf["traffic"] is None or rf["traffic"] > 0
    # kernel times from an eager pass with every launch timed: medians of
    # at least 10 samples per stage
    assert all(n >= 10 for n in line["timing"]["samples_per_stage"].values())
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["host_cpus"] >= 1 and set(cb["stages_ms"]) == {"layout", "slots", "dispatch",
                                                             "combine"}
    assert set(cb["stages_GBps"]) == {"layout+slots", "dispatch", "combine"}
    assert cb["unit"] == line["unit"] and cb["sample"]


@pytest.mark.gpu
@pytest.mark.parametrize("args,check", [
    (["--workload", "qwen3_30b_a3b_prefill", "--sets", "1"],
     lambda l: l["config"]["buffer_sets"] == 1 and l["cache"].startswith("warm")),
    (["--workload", "tiny", "--pipeline", "overlap", "--graph"],
     lambda l: l["pipeline"] == "overlap" and l["timing"]["graph"]),
    (["--workload", "ll_decode_fp8", "--pipeline", "merged", "--graph"],
     lambda l: l["timing"]["graph"] and l["roofline"]["kernel_us_per_launch"] > 0),
], ids=["warm", "overlap-graph", "merged-graph"])
def test_bench_modes(args, check):
    """The warm mode (one buffer set, two handles for the merged pipeline)
    and the graph-captured overlap and merged pipelines each print a line."""
    print("bench.py", *args, flush=True)
    r = _run([*args, "--steps", "8", "--warmup", "4", "--no-cpu-baseline"], 300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["value"] > 0 and check(line), line


def _variant(**kw):
    import argparse
    sys.path.insert(0, ROOT) if ROOT not in sys.path else None
    import bench
    a = dict(workload="qwen3_30b_a3b_prefill", num_sources=0, quant=None, quant_group=0,
             scale_mode=None, combine_quant=None, combine_group=128)
    a.update(kw)
    return bench, bench.variant_of(argparse.Namespace(**a))


def test_variant_flags_key_their_own_traffic(tmp_path, monkeypatch):
    """A run with variant flags is priced and looked up under its own tag:
    it never reports the plain workload's counted bytes, and a record whose
    kernel sources changed is not used."""
    bench, (w, tag, flags) = _variant()
    assert tag == "qwen3_30b_a3b_prefill" and flags == [] and w.quant == 0
    _, (w, tag, flags) = _variant(quant="mxfp4")
    assert (w.quant, w.quant_group) == (3, 32)
    assert tag == "qwen3_30b_a3b_prefill_q3_qg32" and flags == ["--quant", "mxfp4"]
    _, (w, tag, _) = _variant(num_sources=16, combine_quant="fp8")
    assert tag == "qwen3_30b_a3b_prefill_src16_cq1_cg128" and w.combine_group == 128
    # flags that restate the workload's own settings keep its tag
    _, (_, tag, _) = _variant(workload="ll_decode_fp8", quant="fp8")
    assert tag == "ll_decode_fp8"
    # lookups: a record for the plain workload only, in a scratch folder
    monkeypatch.setattr(bench, "traffic_path", lambda t: str(tmp_path / f"traffic_{t}.json"))
    rec = dict(workload="qwen3_30b_a3b_prefill", kernels=dict(
        combine=dict(hbm_bytes_per_launch=1.5e8,
                     source_sha256_16=bench.kernel_source_hash("combine")),
        dispatch=dict(hbm_bytes_per_launch=1.5e8, source_sha256_16="0000000000000000")))
    (tmp_path / "traffic_qwen3_30b_a3b_prefill.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("combine", "qwen3_30b_a3b_prefill") == 1.5e8
    assert bench.traffic_from_profiles("combine", "qwen3_30b_a3b_prefill_q3_qg32") is None
    assert bench.traffic_from_profiles("dispatch", "qwen3_30b_a3b_prefill") is None   # stale
