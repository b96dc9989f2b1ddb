"""Seeded sweep of shapes against the oracle: batch, heads, length, block,
number of random blocks, dtype, padding and score scale drawn per case from
a fixed generator, so that combinations the hand-picked cases miss are
exercised too (every case is reproducible from its index)."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import announce, assert_close, plans, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bbsa.lib()


def draw_case(i):
    rng = np.random.Generator(np.random.PCG64(7000 + i))
    block = int(rng.choice([64, 128]))
    r = int(rng.integers(1, 7))
    nb_min = 6 + 2 * r                      # shortest length on the sparse path
    nb_max = max(nb_min, 2048 // block)
    nb = int(rng.integers(nb_min, nb_max + 1))
    L = nb * block
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    valid = None
    if rng.random() < 0.7:
        valid = [int(rng.integers(block, L + 1)) for _ in range(B)]
    q_scale = float(rng.choice([1.0 / 8.0, 0.5, 1.0]))
    return B, H, L, block, r, dtype, valid, q_scale


@pytest.mark.parametrize("i", range(10))
def test_seeded_shape_sweep(i):
    B, H, L, block, r, dtype, valid, q_scale = draw_case(i)
    announce(f"sweep {i}: B{B} H{H} L{L} block{block} r{r} {dtype} valid={valid} q_scale={q_scale}")
    inp = workloads.make_case(B, H, L, 64, 7000 + i, dtype=dtype, valid=valid, q_scale=q_scale)
    cplan, oplan = plans(H, L // block, r, 7000 + i)
    got, st = run_gpu(inp, block, r, dtype, cplan)
    assert st == bbsa.BBSA_OK
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block)
    assert_close(got, want, dtype, f"sweep {i}")
