"""Builds libep_amd.so (HIP kernels + C-ABI host runtime) for gfx950 with hipcc,
and libep_probe.so (the streaming bandwidth probes of include/ep_probe.h).

The libraries are built in-tree, next to this file.  Each source is compiled
to an object in ``_build/`` and the objects are linked into shared libraries.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libep_amd.so")
PROBE_LIB = os.path.join(PKG, "libep_probe.so")
ARCH = "gfx950"

SOURCES = ["layout.hip", "dispatch.hip", "fused.hip", "sources.hip", "nonexpand.hip",
           "combine.hip", "overlap.hip", "api.cpp"]
PROBE_SOURCES = ["probe.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-I", INCLUDE, "-I", CSRC]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src, extra):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, *extra, "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), out=LIB, verbose=False) -> str:
    """Compiles every source and links ``out`` and the probe library.
    Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs))
    _link(objs[:len(SOURCES)], out)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(out, PROBE_LIB)
    return out


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
