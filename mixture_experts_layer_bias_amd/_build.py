"""Build libmoe_zc.so in-tree for gfx950 with hipcc (no GPU needed).

    python -m mixture_experts_layer_bias_amd._build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_zc.so")
SOURCES = ["route.hip", "gemm_mfma.hip", "gemm_packed.hip", "gemm_fp8.hip", "gemm_simt.hip",
           "backward.hip", "api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU ops stay off: hipcc would otherwise form them from
# ordinary float code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
    "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build)")


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc, "-x", "hip", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # host-pass warnings about the unknown packed-fp32 feature are expected
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe_zc.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(7, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
