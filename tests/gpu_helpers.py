"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, compare to the stated tolerances."""
import sys

import numpy as np
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa

# Tolerances versus the float64 oracle.
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype).cuda()


def plans(H, nb, r, seed):
    """The library plan and the oracle plan; they must be bit-identical."""
    c = bbsa.bbsa_plan_rand_attn(H, nb, r, seed)
    o = oracle.plan_rand_attn(H, nb, r, seed)
    assert np.array_equal(c, o), "C planner and oracle planner differ"
    return c, o


def run_gpu(inp, block, r, dtype, plan, use_mask=True):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (to_dev(inp[n], tdt) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32) if use_mask else None
    ra = torch.from_numpy(plan).cuda() if plan is not None else None
    out, st = bbsa.bbsa_forward(q, k, v, mask, ra, block, r, warn_fallback=False)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st


def assert_close(got, want, dtype, what=""):
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    announce(f"{what} max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx}"
        assert mean <= BF16_MEAN_ABS, f"{what}: mean abs {mean}"
    return mx, mean


def sample_blocks(nb, extra=()):
    """Query blocks compared at full size: both global rows, both rows next to
    them, a few middle rows."""
    base = {0, 1, 2, nb // 3, nb // 2, (2 * nb) // 3, nb - 3, nb - 2, nb - 1}
    return sorted(b for b in base.union(extra) if 0 <= b < nb)


def gather_rows(out, blocks, block):
    idx = np.concatenate([np.arange(b * block, (b + 1) * block) for b in blocks])
    return out[:, :, idx]
