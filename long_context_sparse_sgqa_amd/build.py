"""Build libsgqa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m long_context_sparse_sgqa_amd.build          # compile + link
    python -m long_context_sparse_sgqa_amd.build --host-sanitizers
        # libsgqa_hostsan.so: the same library with AddressSanitizer and UndefinedBehaviorSanitizer
        # on the host code only (argument validation, sizing, launch set-up); the GPU code is
        # built as usual.  Run the CPU test tier against it with
        #   SGQA_LIBRARY=$PWD/long_context_sparse_sgqa_amd/libsgqa_hostsan.so \
        #   LD_PRELOAD=$(python -m long_context_sparse_sgqa_amd.build --asan-runtime) \
        #   ASAN_OPTIONS=detect_leaks=0 python -m pytest tests -m "not gpu" -q
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
           "attend_split.hip", "attend_bwd.hip", "paged.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(REPO_DIR, "include"), "-I", CSRC,
]

# Per-source flags.  The key-major dK/dV kernel needs more than the 256 architectural VGPRs; left to
# its heuristics the compiler keeps the dK/dV sums in VGPRs between steps and moves all 128 of them
# to accumulation registers for every step's products.  Matrix-core ops on VGPRs avoid that move.
SOURCE_FLAGS = {
    "attend_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


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


# host-only sanitizers: each -fsanitize= goes to the host compilation alone
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-g"]
HOSTSAN_LIB_PATH = os.path.join(PKG_DIR, "libsgqa_hostsan.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a host-sanitized library needs preloaded."""
    hipcc = _hipcc()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                       text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang AddressSanitizer runtime was not found")
    return path


def build(verbose: bool = False, host_sanitizers: bool = False) -> str:
    """Compile every source and link libsgqa.so (or libsgqa_hostsan.so with host sanitizers);
    always rebuilds.  Returns the library path."""
    hipcc = _hipcc()
    bdir = os.path.join(BUILD_DIR, "hostsan") if host_sanitizers else BUILD_DIR
    lib_path = HOSTSAN_LIB_PATH if host_sanitizers else LIB_PATH
    extra = HOST_SANITIZE if host_sanitizers else []
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
               "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    # a host-sanitized library is linked without a runtime: its sanitizer symbols resolve against
    # the AddressSanitizer runtime preloaded into the process (which carries the UBSan handlers)
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib_path)
    if verbose:
        print("built", lib_path)
    return lib_path


if __name__ == "__main__":
    if "--asan-runtime" in sys.argv:
        print(asan_runtime())
    else:
        build(verbose=True, host_sanitizers="--host-sanitizers" in sys.argv)
    sys.exit(0)
