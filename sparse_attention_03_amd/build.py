"""Builds libdsa.so (the HIP kernels and the C interface) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree.  Packed-FP32 instructions are disabled for the device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "libdsa.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "sparse_mla.hip", "cache_append.hip", "align.hip", "mla_backward.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    cmd = [HIPCC, *FLAGS, *extra_flags, *(os.path.join(CSRC, s) for s in SOURCES), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libdsa.so")
    errs = [ln for ln in res.stderr.splitlines() if "error" in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
