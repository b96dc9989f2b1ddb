"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, compare to the stated tolerances."""
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa

# Tolerances versus the float64 oracle.
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3

# (what, rows, max_abs, mean_abs) of every comparison, printed at the end of
# the session by conftest.py.
PARITY_LOG = []


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
    """One bbsa_forward call.  The output buffer is filled with NaN first, so
    a row the kernels never write shows up as non-finite."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (to_dev(inp[n], tdt) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32) if use_mask else None
    ra = torch.from_numpy(plan).cuda() if plan is not None else None
    out = torch.full_like(q, float("nan"))
    out, st = bbsa.bbsa_forward(q, k, v, mask, ra, block, r, out=out, warn_fallback=False)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st


def check_tol(mx, mean, dtype, what):
    if dtype == "f32":
        assert mx <= F32_MAX_ABS, f"{what}: max abs {mx}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx}"
        assert mean <= BF16_MEAN_ABS, f"{what}: mean abs {mean}"


def assert_close(got, want, dtype, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output (a row was not written?)"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    announce(f"{what} max_abs={mx:.3e} mean_abs={mean:.3e}")
    PARITY_LOG.append((what, int(np.prod(got.shape[:-1])), mx, mean))
    check_tol(mx, mean, dtype, what)
    return mx, mean


def sample_blocks(nb, extra=()):
    """Query blocks compared at full size: both global rows, both rows next to
    them, a few middle rows."""
    base = {0, 1, 2, nb // 3, nb // 2, (2 * nb) // 3, nb - 3, nb - 2, nb - 1}
    return sorted(b for b in base.union(extra) if 0 <= b < nb)


def varied_blocks(nb, bh, n_random=6, seed=0):
    """The fixed sample above plus ``n_random`` middle blocks drawn per
    (batch, head), so that different pairs check different rows."""
    rng = np.random.Generator(np.random.PCG64(90000 + 131 * bh + seed))
    extra = rng.choice(np.arange(1, nb - 1), size=min(n_random, nb - 2), replace=False)
    return sample_blocks(nb, extra=[int(x) for x in extra])


def gather_rows(out, blocks, block):
    idx = np.concatenate([np.arange(b * block, (b + 1) * block) for b in blocks])
    return out[..., idx, :]


def oracle_slices(inp, plan, block, jobs, threads=8):
    """Run the oracle on (batch, head) slices in a thread pool.

    jobs: list of (b, h, query_blocks or None).  Returns the list of float64
    outputs ``[rows, d]`` in the same order.  Each call is the plain oracle
    on one slice; numpy releases the interpreter lock in its matrix products
    and element-wise kernels, so the slices run in parallel."""
    from threadpoolctl import threadpool_limits

    def one(job):
        b, h, qbs = job
        return oracle.forward(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1],
                              inp["v"][b:b + 1, h:h + 1], inp["mask"][b:b + 1],
                              None if plan is None else plan[h:h + 1], block,
                              query_blocks=qbs)[0, 0]

    with threadpool_limits(1):
        with ThreadPoolExecutor(threads) as ex:
            return list(ex.map(one, jobs))


def valid_query_rows(mask, b, rows):
    """Boolean over ``rows`` (token indices): True where the query token is
    inside the valid length (mask 1)."""
    return mask[b, rows] > 0.5
