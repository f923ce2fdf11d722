"""Compile libparo.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m rotated_linear_amd._build`` (also called by ``__graft_entry__.build``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libparo.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}",
    # keep packed-FP32 VALU instructions out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# per-file extras: the build-time pack must round every float64 product and sum on its own
# the GEMM keeps its accumulators in architectural registers (the per-group rescale multiplies them)
EXTRA = {"pack.hip": ["-ffp-contract=off"], "gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "skinny.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["paro_api.cpp", "schedule.cpp", "pack.hip", "rotate.hip", "decode.hip", "gemm.hip", "skinny.hip", "noalloc.hip"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libparo")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
