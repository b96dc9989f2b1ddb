"""The benchmark's useful-work and byte accounting, pinned to the oracle's
block mask: useful flops count exactly the (query block, key block) pairs the
pattern contains, at 4 * block^2 * d flops each (QK^T and PV)."""
import os
import sys

import numpy as np
import pytest

import oracle

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from block_sparse_long_bbsa_amd import workloads  # noqa: E402


@pytest.mark.parametrize("nb,r", [(12, 3), (16, 3), (64, 3), (256, 2), (30, 7)])
def test_useful_pairs_match_the_block_mask(nb, r):
    plan = oracle.plan_rand_attn(2, nb, r, 5)
    for h in range(2):
        pairs = int(oracle.block_mask(nb, plan[h]).sum())
        assert bench.useful_pairs(nb, r) == pairs


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_workload_figures(wid):
    w = workloads.WORKLOADS[wid]
    plan = oracle.plan_rand_attn(1, w.nb, w.r, w.plan_seed)
    keys = oracle.attended_key_counts(w.nb, w.block, plan[0])
    # Each attended (query, key) pair costs 2d flops for QK^T and 2d for PV.
    flops = float(keys.sum()) * w.block * 4 * w.d * w.B * w.H
    assert bench.useful_flops(w.B, w.H, w.nb, w.block, w.d, w.r) == pytest.approx(flops, rel=1e-12)
    elt = 2 if w.dtype == "bf16" else 4
    nbytes = 4 * w.B * w.H * w.L * w.d * elt + w.B * w.L * 4 + w.H * (w.nb - 2) * w.r * 4
    assert bench.algorithmic_bytes(w.B, w.H, w.L, w.d, w.nb, w.r, elt) == nbytes


def test_headline_workload_figures():
    # B4 H12 L4096 d64 block64 r3: 31.306 GFLOP of useful work, 100.738 MB moved.
    w = workloads.WORKLOADS[2]
    assert bench.useful_flops(w.B, w.H, w.nb, w.block, w.d, w.r) / 1e9 == pytest.approx(31.306, abs=5e-4)
    assert bench.algorithmic_bytes(w.B, w.H, w.L, w.d, w.nb, w.r, 2) / 1e6 == pytest.approx(100.738, abs=5e-4)


def test_multi_gpu_request_is_refused():
    import subprocess
    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
