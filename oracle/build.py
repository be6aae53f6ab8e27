"""Compile the CPU oracle (plain C) into oracle/libmoe_oracle.so.

Test infrastructure only: the oracle is the checker, never part of the
product path.  Flags keep IEEE fp32/fp64 semantics: no fast-math, no
fused multiply-add contraction; OpenMP runs the per-token loops on threads.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB, extra=()) -> str:
    """extra: additional compiler flags (the sanitizer build of the tests)."""
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", *extra, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
