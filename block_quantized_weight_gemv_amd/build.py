"""Builds libqk.so in-tree with hipcc for gfx950.

Each source compiles to its own object (the dequantiser with
-ffp-contract=off), then one shared library is linked. The library has no
RPATH to /opt/rocm: when torch is imported first, its HIP runtime (same
SONAME) is the one the library binds to.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("QK_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
    # packed fp32 VALU ops (v_pk_fma_f32 and friends) stay disabled
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
SOURCES = {
    "qk_api.hip": [],
    "qk_dequant.hip": ["-ffp-contract=off"],
    "qk_gemv.hip": [],
    "qk_gemm.hip": [],
    "qk_pass.hip": [],
    "qk_probe.hip": [],
    "qk_step.hip": [],
    "qk_gguf.cpp": [],
}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.DEVNULL)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
