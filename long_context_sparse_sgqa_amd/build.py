"""Build libsgqa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m long_context_sparse_sgqa_amd.build          # compile + link
The library lands next to this file; objects go to _build/ (not committed).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libsgqa.so")

SOURCES = ["sgqa_api.cpp", "compress.hip", "index.hip", "topk.hip", "select_fused.hip", "attend.hip",
           "attend_split.hip", "paged.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(REPO_DIR, "include"), "-I", CSRC,
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsgqa.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that notice is harmless
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libsgqa.so; always rebuilds.  Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
