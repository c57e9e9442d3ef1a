"""Build libmx.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

Usage: python -m microscaling_precision_gemm_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmx.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = [
    os.path.join(CSRC, "api.cpp"),
    os.path.join(CSRC, "kernels", "quantize.hip"),
    os.path.join(CSRC, "kernels", "requant.hip"),
    os.path.join(CSRC, "kernels", "gemm_mx.hip"),
    os.path.join(CSRC, "kernels", "gemm_staged.hip"),
    os.path.join(CSRC, "kernels", "gemm_tiled.hip"),
    os.path.join(CSRC, "kernels", "gemm_nvpipe.hip"),
    os.path.join(CSRC, "kernels", "gemm_any.hip"),
    os.path.join(CSRC, "kernels", "gemm_f6.hip"),
    os.path.join(CSRC, "kernels", "stats.hip"),
    os.path.join(CSRC, "kernels", "gemm_qa.hip"),
]

# -ffp-contract=off: the quantizers' FP32 scale arithmetic must round once per
# operation, exactly as written.  Packed FP32 instructions are disabled.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-x", "hip", "-c", src, "-o", obj, "-I", os.path.join(ROOT, "include")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libmx.so next to this file."""
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
