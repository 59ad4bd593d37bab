"""Build libgemmq.so for gfx950 with hipcc (in-tree, next to this file).

    python -m quant_packed_weight_amd.build

Every HIP source is compiled for gfx950 only, with:
  -ffp-contract=off      the kernels write every fused multiply-add explicitly, so
                         the f32 order of operations is exactly the source's;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                         no packed f32 instructions are generated;
and never with -ffast-math: the activation quantizer needs correctly rounded
f32 division and preserved denormals to match its definition bit for bit.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemmq.so")
SOURCES = ["abi.hip", "quantize.hip", "gemv.hip", "gemm.hip", "gemm_q4k.hip", "gemm_q6k.hip", "decode.hip",
           "repack.hip", "probe.hip", "skinny.hip", "skinny_q6k.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libgemmq.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
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
