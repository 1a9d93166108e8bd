"""Compile the CPU oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure only.  IEEE double semantics are kept: no fast-math and no
floating-point contraction, so every machine computes the same bits.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O3", "-std=c11", "-D_GNU_SOURCE", "-fopenmp", "-ffp-contract=off",
           "-march=x86-64-v2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
