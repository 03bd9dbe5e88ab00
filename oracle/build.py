"""Builds the CPU oracle (``libep_oracle.so``) with gcc.

Test infrastructure: compiled by ``__graft_entry__.build()`` and on demand by
the tests, the smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.c")
LIB = os.path.join(HERE, "libep_oracle.so")

# Plain scalar code: no fast-math, no contraction of a*b+c into fma, no
# vector extensions beyond the x86-64 baseline (SSE2 keeps fp32 arithmetic in
# fp32 and fp64 in fp64).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
