"""Build libq4k.so (HIP, gfx950) in-tree with hipcc.

    python -m gemm_q4_super_amd.build

Each csrc/*.hip is compiled to an object under _build/ in parallel, then
linked into gemm_q4_super_amd/libq4k.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libq4k.so")
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


# Packed fp32 VALU ops are kept out of generated code on purpose; the fp32
# epilogues are written as scalar fma.  The leading 16 dwords of every
# kernel's arguments are preloaded into scalar registers at wave launch (the
# code keeps a prologue that loads them for firmware without the feature).
# Matrix-core results go to ordinary vector registers, where the fp32
# epilogue reads them without copies.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-kernarg-preload-count=16",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I" + os.path.join(ROOT, "include")]


# Q4K_GEMM_INT8=1 builds the prefill GEMM's int8 contraction instead of the
# default fp16 one (same results to fp32 rounding; kept for comparison).
if os.environ.get("Q4K_GEMM_INT8") == "1":
    COMMON.append("-DGEMM_I8=true")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc()] + COMMON + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
