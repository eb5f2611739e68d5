"""Builds libdsa.so (the HIP kernels and the C interface) for gfx950 with hipcc.

The library is built in-tree, next to this file, so that it travels with the
source tree.  Each source compiles to its own object in parallel (the
kernels of one file never call into another file's device code), then the
objects are linked into the shared library.  Packed-FP32 instructions are
disabled for the device code.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
OBJ_DIR = os.path.join(LIB_DIR, "obj")
LIB = os.path.join(LIB_DIR, "libdsa.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "sparse_mla.hip", "cache_append.hip", "align.hip", "mla_backward.hip",
           "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    errs = [ln for ln in res.stderr.splitlines() if "error" in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")


# Host code (argument checks, workspace plans, launches) instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built as
# usual.  For CPU-side tests only: load it with LIBDSA_PATH and preload clang's
# ASan runtime (the command is in the library's design notes).
SANITIZED_LIB = os.path.join(LIB_DIR, "libdsa_sanitized.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def build(verbose: bool = False, extra_flags=(), sanitize: bool = False) -> str:
    obj_dir = os.path.join(LIB_DIR, "obj_sanitized" if sanitize else "obj")
    out = SANITIZED_LIB if sanitize else LIB
    flags = [*FLAGS, *(SANITIZE_FLAGS if sanitize else ()), *extra_flags]
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
    if sanitize:
        link[3:3] = ["-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"]
    _run(link, verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
