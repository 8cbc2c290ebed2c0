"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags keep the arithmetic exactly as written: no fast-math, no contraction of
a*b+c into a fused multiply-add.  OpenMP only splits output columns across
threads.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
