"""Builds the CPU oracle with gcc: ``libep_oracle.so`` (serial, the parity
reference) and ``libep_oracle_omp.so`` (the same source with OpenMP over the
tokens of dispatch and combine, used only to time the oracle on a host's
cores; its results equal the serial build's).

Test infrastructure: compiled by ``__graft_entry__.build()`` and on demand by
the tests, the smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
HDR = os.path.join(HERE, "ep_oracle.h")
LIB = os.path.join(HERE, "libep_oracle.so")
LIB_OMP = os.path.join(HERE, "libep_oracle_omp.so")

# Plain scalar code: no fast-math, no contraction of a*b+c into fma, no
# vector extensions beyond the x86-64 baseline (SSE2 keeps fp32 arithmetic in
# fp32 and fp64 in fp64).  The serial build ignores the OpenMP pragmas.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def _stale(lib):
    return (not os.path.exists(lib)
            or os.path.getmtime(lib) < max(os.path.getmtime(SRC), os.path.getmtime(HDR)))


def build(force: bool = True, openmp: bool = False) -> str:
    lib = LIB_OMP if openmp else LIB
    if not force and not _stale(lib):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    flags = CFLAGS + (["-fopenmp"] if openmp else ["-Wno-unknown-pragmas"])
    cmd = ["gcc", *flags, "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_all(force: bool = True):
    return build(force=force), build(force=force, openmp=True)


if __name__ == "__main__":
    print(build_all())
