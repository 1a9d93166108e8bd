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


SAN_LIB = os.path.join(HERE, "liboracle_san.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build (any report aborts);
# a process that loads it preloads gcc's libasan (asan_runtime()).
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc"] + (SAN_FLAGS if sanitize else ["-O3"]) + [
           "-std=c11", "-D_GNU_SOURCE", "-fopenmp", "-ffp-contract=off",
           "-march=x86-64-v2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
