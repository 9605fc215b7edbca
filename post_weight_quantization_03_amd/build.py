"""Build libgptq.so (HIP, gfx950) in-tree: one hipcc compile per source, then a link.

Usage: python -m post_weight_quantization_03_amd.build  (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is written next to
this file, where the Python binding loads it from.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgptq.so")

# the column sweep's instantiations (sweep_*.hip) are the slowest to compile: first, so
# that they start at once
SOURCES = ["sweep_g0.hip", "sweep_g128.hip", "sweep_misc.hip", "quantize.hip", "gptq_abi.hip", "hessian.hip",
           "gemm.hip", "prepare.hip", "pack.hip", "serve.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

# Packed fp32 VALU instructions (v_pk_*_f32) are disabled for every kernel; all fp32
# arithmetic is issued as scalar-lane VALU or MFMA instructions.
CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the column sweep keeps a 128-column row block in registers: its loops must unroll fully
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
