"""Dense attention probabilities (output_attentions) on MI355X against the
oracle's probabilities ("BigBirdPegasus…", section "三类注意力组合全局 局部
随机": the sparse weights scattered into a full (bsz, heads, L, L) matrix).

Every entry outside the pattern must be exactly 0 (bit for bit); inside it
the probabilities are computed in fp32 from q and k, so both dtypes are held
to the fp32 bound, max abs 1e-4 against the float64 oracle (a score's fp32
rounding over 64 products is about 1e-5 relative to sum |q_e k_e|, which the
probability carries as a relative error); row sums agree with the oracle's
within 1e-5 (they are 1 except where a ragged length's trimmed padding keys
carried weight).
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import PARITY_LOG, announce, plans, to_dev

pytestmark = pytest.mark.gpu

P_MAX_ABS = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bbsa.lib()


def run_probs(inp, block, r, dtype, plan, pad=False, qk=False):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k = (to_dev(inp[n], tdt) for n in ("q", "k"))
    mask = to_dev(inp["mask"], torch.float32)
    ra = torch.from_numpy(plan).cuda() if plan is not None else None
    B, H, L, _ = q.shape
    probs = torch.full((B, H, L, L), float("nan"), dtype=torch.float32, device="cuda")
    probs, st = bbsa.bbsa_attention_probs(q, k, mask, ra, block, r, probs=probs, pad_to_block=pad,
                                          query_key_mask=qk)
    torch.cuda.synchronize()
    return probs.cpu().numpy().astype(np.float64), st


def compare(got, want, nb, block, plan, full, what, L):
    assert np.isfinite(got).all(), f"{what}: non-finite or unwritten entries"
    H = got.shape[1]
    for h in range(H):
        M = np.ones((nb, nb), bool) if full else oracle.block_mask(nb, plan[h])
        T = np.kron(M.astype(np.int8), np.ones((block, block), np.int8)).astype(bool)[:L, :L]
        outside = got[:, h][:, ~T]
        assert (outside == 0.0).all(), f"{what}: nonzero probability outside the pattern"
    err = np.abs(got - want)
    # Row sums: 1, except where the [L, L] matrix trims away the padding keys
    # of a ragged length that carried weight (a padded query row in query x
    # key mode); the oracle's trimmed rows say how much remains.
    rs = np.abs(got.sum(axis=-1) - want.sum(axis=-1))
    announce(f"{what} P max_abs={err.max():.3e} row-sum dev={rs.max():.3e}")
    PARITY_LOG.append((what + " probs", int(np.prod(got.shape[:-1])), float(err.max()), float(err.mean())))
    assert err.max() <= P_MAX_ABS, f"{what}: {err.max()}"
    assert rs.max() <= 1e-5, f"{what}: row sums {rs.max()}"


CASES = [
    # B, H, L, block, r, dtype, valid, pad, qk, q_scale
    (2, 2, 1024, 64, 3, "bf16", (1024, 700), False, False, None),
    (2, 2, 1024, 64, 3, "f32", (1024, 700), False, False, None),
    (1, 2, 2048, 128, 2, "bf16", (1900,), False, False, None),
    (2, 2, 1536, 64, 3, "f32", (1536, 900), False, True, None),   # query x key
    (2, 2, 1000, 64, 3, "bf16", (1000, 937), True, False, None),  # ragged length
    (1, 2, 1100, 64, 3, "f32", (1050,), True, True, None),        # ragged + query x key
    (1, 2, 704, 64, 3, "bf16", (650,), False, False, None),       # short: full attention
    (1, 1, 1024, 64, 3, "f32", (0,), False, False, None),         # fully padded
    (1, 2, 2048, 64, 3, "f32", (2048,), False, False, 1.0),       # large scores
]


@pytest.mark.parametrize("B,H,L,block,r,dtype,valid,pad,qk,q_scale", CASES)
def test_probs_match_oracle(B, H, L, block, r, dtype, valid, pad, qk, q_scale):
    announce(f"probs B{B} H{H} L{L} block{block} r{r} {dtype} valid={valid} pad={pad} qk={qk}")
    inp = workloads.make_case(B, H, L, 64, 110 + L % 89, dtype=dtype, valid=valid, q_scale=q_scale)
    nb = -(-L // block)
    full = L <= (5 + 2 * r) * block
    cplan, oplan = plans(H, nb, r, 110)
    got, st = run_probs(inp, block, r, dtype, None if full else cplan, pad=pad, qk=qk)
    assert st == (bbsa.BBSA_OK_FULL_FALLBACK if full else bbsa.BBSA_OK)
    f = oracle.forward_padded if pad else oracle.forward
    _, want = f(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block, return_probs=True, query_key_mask=qk)
    compare(got, want, nb, block, oplan, full, f"probs L{L} {dtype} pad={pad} qk={qk}", L)


def test_probs_at_the_bigbird_base_length():
    # Two (batch, head) slices of the BigBird-base workload (L = 4096,
    # padded sequences): every entry compared; P V also reproduces the
    # forward output of the same inputs.
    announce("probs BigBird-base slices")
    w = workloads.WORKLOADS[2]
    full_inp = workloads.make_inputs(2)
    inp = {n: np.ascontiguousarray(full_inp[n][1:2, 3:5]) for n in ("q", "k", "v")}
    inp["mask"] = np.ascontiguousarray(full_inp["mask"][1:2])
    cplan, oplan = plans(w.H, w.nb, w.r, w.plan_seed)
    cplan, oplan = cplan[3:5].copy(), oplan[3:5].copy()
    got, st = run_probs(inp, w.block, w.r, "bf16", cplan)
    assert st == bbsa.BBSA_OK
    out, want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, w.block, return_probs=True)
    compare(got, want, w.nb, w.block, oplan, False, "probs BigBird-base B1 H2 L4096", 4096)
    pv = got @ inp["v"].astype(np.float64)
    assert np.abs(pv - out).max() <= 1e-4
