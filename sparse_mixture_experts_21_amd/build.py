"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m sparse_mixture_experts_21_amd.build [-v]

Objects go to _build/ at the repository root; the shared library is written
next to this file so the Python binding (and anything copied with the tree)
finds it.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_api.cpp", "router.hip", "dispatch.hip", "route_small.hip", "expert_gemm.hip",
           "combine.hip", "expert_choice.hip", "bwd_gemm.hip", "bwd.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for every device pass (the host pass
# warns that it does not know the feature; that is harmless).
COMMON = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str, verbose: bool, extra) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if verbose and r.stderr.strip():
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines), flush=True)
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


# Host-sanitizer build: moe_api.cpp (argument validation, workspace layout,
# launch sequencing) with AddressSanitizer and UndefinedBehaviorSanitizer on
# its host code only, linked with the regular kernel objects into
# libmoe_hostsan.so.  The CPU tests load it through MOE_LIB with the clang
# ASan runtime preloaded (asan_runtime()).
SAN_LIB = os.path.join(PKG, "libmoe_hostsan.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang ASan runtime that a process loading libmoe_hostsan.so preloads."""
    import glob
    root = os.path.dirname(os.path.dirname(hipcc())) if os.path.isabs(hipcc()) else "/opt/rocm"
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm llvm tree")
    return hits[-1]


def build_host_sanitized(verbose: bool = False) -> str:
    others = [os.path.join(OBJDIR, os.path.splitext(f)[0] + ".o") for f in SOURCES
              if f != "moe_api.cpp"]
    if not all(os.path.exists(o) for o in others):
        build(verbose)
    os.makedirs(OBJDIR, exist_ok=True)
    obj = os.path.join(OBJDIR, "moe_api_hostsan.o")
    cmd = [hipcc()] + COMMON + ["-g"] + SAN_HOST + ["-c", os.path.join(CSRC, "moe_api.cpp"),
                                                    "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on moe_api.cpp (host sanitizers):\n{r.stderr}")
    tmp = SAN_LIB + f".tmp{os.getpid()}"
    # the sanitizer runtime is not linked in: its symbols resolve against the
    # preloaded clang ASan runtime (which carries the UBSan handlers too)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj] + others
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
