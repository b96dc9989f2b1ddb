"""Build the HIP library ``libbbsa.so`` in-tree with hipcc for gfx950.

Usage: ``python -m block_sparse_long_bbsa_amd.build`` (or call ``build()``).
The library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbbsa.so")

SOURCES = ["bbsa_forward.hip", "bbsa_probs.hip", "bbsa_backward.hip", "bbsa_plan.cpp", "bbsa_host.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed FP32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Scores are always finite (the padding bias is -10000, the initial max
    # -1e30): max needs no NaN quieting, so v_max/v_max3 run without
    # canonicalising their inputs.
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbbsa.so")


def build(verbose: bool = False) -> str:
    """Compile every source into ``libbbsa.so``; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
