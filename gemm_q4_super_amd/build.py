"""Build libq4k.so (HIP, gfx950) in-tree with hipcc.

    python -m gemm_q4_super_amd.build

Each csrc/*.hip is compiled to an object under _build/ in parallel, then
linked into gemm_q4_super_amd/libq4k.so next to this file.  A second library,
libq4k_gemm_int8.so, is the same objects with the prefill GEMM compiled for
its int8 contraction (v_mfma_i32_32x32x32_i8 on the quants and codes) instead
of the default fp16 one: the comparison the default was chosen by, kept built
and tested.
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

LIB_GEMM_INT8 = os.path.join(HERE, "libq4k_gemm_int8.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, suffix: str = "", defs=()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + suffix + ".o")
    cmd = [hipcc()] + COMMON + list(defs) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    gemm_src = os.path.join(CSRC, "gemm.hip")
    jobs = [(src, "", ()) for src in srcs] + [(gemm_src, "_int8", ("-DGEMM_I8=true",))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    base, int8_gemm = objs[:-1], objs[-1]
    _link(base, LIB)
    _link([o for o in base if os.path.basename(o) != "gemm.o"] + [int8_gemm], LIB_GEMM_INT8)
    if verbose:
        print("built", LIB, "and", LIB_GEMM_INT8)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
