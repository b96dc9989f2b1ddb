"""Build the HIP library ``libbbsa.so`` in-tree with hipcc for gfx950.

Usage: ``python -m block_sparse_long_bbsa_amd.build`` (or call ``build()``).
The library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbbsa.so")

SOURCES = ["bbsa_forward.hip", "bbsa_probs.hip", "bbsa_backward.hip", "bbsa_backward_f32.hip", "bbsa_plan.cpp",
           "bbsa_host.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed FP32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Scores are always finite (the padding bias is -10000, the initial max
    # -1e30): max needs no NaN quieting, so v_max/v_max3 run without
    # canonicalising their inputs.
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-Wall", "-Wno-unused-result",
]

# Per-source additions.  The backward kernels keep their MFMA accumulators
# in ordinary VGPRs: the scores feed VALU arithmetic every step, and with
# AGPR accumulators each value would be copied out first (and the dk/dv
# kernel would not fit two waves per SIMD).
SOURCE_FLAGS = {
    "bbsa_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbbsa.so")


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link ``libbbsa.so``; returns
    the library path."""
    tmp = LIB + ".tmp"
    include = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="bbsa_build_") as work:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(work, src + ".o")
            cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *include, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, proc in procs:
            out, _ = proc.communicate()
            if proc.returncode != 0:
                sys.stderr.write(out)
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
