"""Compile the CPU oracle (plain C, gcc) into oracle/libcskv_oracle.so.

Strict IEEE arithmetic: no fast-math, no contraction of a*b+c into FMA (the
oracle calls fmaf explicitly where the definition fuses), no -march, so the
fp32 steps round exactly as the definitions say.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libcskv_oracle.so")
SRC = os.path.join(HERE, "cskv_oracle.c")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-fno-finite-math-only", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
