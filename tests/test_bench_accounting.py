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


def _executed_by_rows(w, mask, plan, chunks):
    """The executed share restated row by row from the pattern itself: a
    middle row lists block 0 first; a global row's key chunks come in groups
    of four, group g covering blocks [4g nb / chunks, (4g + 4) nb / chunks),
    and chunk u of a group lists every fourth block of that range from its
    u-th; a list with a key of mask 1 drops its fully padded blocks except
    the first.  (For these workloads each 64-row tile of a query block has
    the same list.)"""
    nb, blk = w.nb, w.block
    blocks = mask.reshape(w.B, nb, blk)
    padded = (blocks == 0).all(axis=2)
    one = (blocks == 1).any(axis=2)
    total = executed = 0

    def add(b, lst):
        nonlocal total, executed
        total += len(lst)
        drop = sum(padded[b, x] for x in lst[1:]) if any(one[b, x] for x in lst) else 0
        executed += len(lst) - drop

    for b in range(w.B):
        for h in range(w.H):
            M = oracle.block_mask(nb, plan[h])
            for i in range(nb):
                if i in (0, nb - 1):
                    for g in range(chunks // 4):
                        lo, hi = 4 * g * nb // chunks, (4 * g + 4) * nb // chunks
                        for u in range(4):
                            add(b, list(range(lo + u, hi, 4)))
                else:
                    keys = [int(x) for x in np.nonzero(M[i])[0]]
                    add(b, [0] + [x for x in keys if x != 0])
    return executed / total


@pytest.mark.parametrize("wid,chunks", [(2, 4), (3, 4), (4, 16), (5, 8)])
def test_executed_pair_fraction(wid, chunks):
    """bench.executed_pair_fraction (the library's work map plus the mask)
    against the same rule applied to the pattern's block mask."""
    from block_sparse_long_bbsa_amd import bbsa
    w = workloads.WORKLOADS[wid]
    x = workloads.make_inputs(wid)
    plan = bbsa.bbsa_plan_rand_attn(w.H, w.nb, w.r, w.plan_seed)
    got = bench.executed_pair_fraction(w, x["mask"], plan, bbsa)
    assert got == pytest.approx(_executed_by_rows(w, x["mask"], plan, chunks), rel=1e-12)
    if wid == 4:
        assert got == 1.0     # no padding: nothing is left out
    else:
        assert 0.6 < got < 0.9


class _FakeCuda:
    @staticmethod
    def synchronize():
        pass


class _FakeTorch:
    cuda = _FakeCuda()


class _FakeRun:
    torch = _FakeTorch()

    def step(self, i):
        pass


def test_clock_reading_parses_amd_smi(monkeypatch):
    # The mean of the gfx_* clocks of the one GPU listed; other clock domains
    # are ignored.
    out = ('{"gpu_data": [{"gpu": 0, "clock": {"gfx_0": {"clk": {"value": 2000, "unit": "MHz"}}, '
           '"gfx_1": {"clk": {"value": 2100, "unit": "MHz"}}, "mem_0": {"clk": {"value": 1300, "unit": "MHz"}}}}]}')
    monkeypatch.setattr(bench.subprocess, "run",
                        lambda *a, **k: bench.subprocess.CompletedProcess(a, 0, stdout=out, stderr=""))
    res = bench.Runner.clock_under_load(_FakeRun(), 0.2)
    assert res is not None and res["mhz"] == 2050.0 and res["readings"] >= 1


@pytest.mark.parametrize("stdout", ["", "not json", '{"gpu_data": []}',
                                    '{"gpu_data": [{"clock": {}}, {"clock": {}}]}'])
def test_clock_reading_is_none_when_unavailable(monkeypatch, stdout):
    monkeypatch.setattr(bench.subprocess, "run",
                        lambda *a, **k: bench.subprocess.CompletedProcess(a, 0, stdout=stdout, stderr=""))
    assert bench.Runner.clock_under_load(_FakeRun(), 0.1) is None


def test_clock_reading_without_the_tool(monkeypatch):
    def missing(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(bench.subprocess, "run", missing)
    assert bench.Runner.clock_under_load(_FakeRun(), 0.1) is None
