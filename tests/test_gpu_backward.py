"""Parity of the backward (bbsa_backward) with the oracle's float64
gradients on MI355X ("models 仓库中的 BigBird…", section "梯度检查点的实现方式";
"BigBirdPegasus…", section "使用限制与注意事项").

The GPU path runs bbsa_forward_ex (output and fp32 row log-sum-exp), then
bbsa_backward; the oracle differentiates the float64 definition at the same
inputs (bf16-exact for the bf16 path) and output gradient.

Tolerances, for each of dq, dk, dv with s the largest magnitude of the
oracle's gradient (at least 1):
- bf16: max abs <= 2e-2 s and mean abs <= 2e-3 s.  The GPU path's errors
  are relative to the gradient's scale: P carries the forward lse's error
  (the bf16 path sums bf16-rounded probabilities: up to 2^-9 relative),
  rowsum(dout * out) uses the forward's bf16 output (2^-9 relative per
  element), and ds and p are rounded to bf16 (2^-9) before the products
  that accumulate them in fp32.
- fp32: max abs <= 1e-4 s and mean abs <= 1e-5 s.  Everything is fp32: the
  forward output (relative error ~1e-6), the 64-term dot products and the
  sums over up to L keys (each ~1e-6 relative), and the exponentials (a few
  ulps); the row normaliser is recomputed relative to the row's bias level,
  so no -10000 cancellation enters.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import PARITY_LOG, announce, plans, to_dev

pytestmark = pytest.mark.gpu

MAX_REL = {"bf16": 2e-2, "f32": 1e-4}
MEAN_REL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bbsa.lib()


def bf16_exact(x):
    return workloads.round_to_bf16(x)


def run_backward(inp, dout, block, r, plan, pad=False, qk=False, dtype="bf16", no_mask=False):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, do = (to_dev(x, tdt) for x in (inp["q"], inp["k"], inp["v"], dout))
    mask = None if no_mask else to_dev(inp["mask"], torch.float32)
    ra = torch.from_numpy(plan).cuda() if plan is not None else None
    out, lse, st = bbsa.bbsa_forward_ex(q, k, v, mask, ra, block, r, return_lse=True, pad_to_block=pad,
                                        query_key_mask=qk, warn_fallback=False)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(q, float("nan"))
    dv = torch.full_like(q, float("nan"))
    dq, dk, dv, st2 = bbsa.bbsa_backward(q, k, v, out, do, lse, mask, ra, block, r, dq=dq, dk=dk, dv=dv,
                                         pad_to_block=pad, query_key_mask=qk)
    torch.cuda.synchronize()
    assert st == st2
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)], st


def plans_for(H, nb, r, seed, full):
    """(C plan, oracle plan).  With fewer than 5 + r blocks no plan exists and
    the call is the full-attention fallback; the oracle takes that decision
    from the plan's shape (its r), so it gets a placeholder of that shape."""
    if nb >= 5 + r:
        return plans(H, nb, r, seed)
    assert full
    return None, np.zeros((H, max(nb - 2, 0), r), dtype=np.int32)


def check(got, want, what, dtype="bf16"):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert np.isfinite(g).all(), f"{what} {name}: non-finite (unwritten?) entries"
        s = max(1.0, float(np.abs(w).max()))
        err = np.abs(g - w)
        announce(f"{what} {name}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} scale={s:.3g}")
        PARITY_LOG.append((f"{what} {name}", int(np.prod(g.shape[:-1])), float(err.max()), float(err.mean())))
        assert err.max() <= MAX_REL[dtype] * s, f"{what} {name}: max abs {err.max()} (scale {s})"
        assert err.mean() <= MEAN_REL[dtype] * s, f"{what} {name}: mean abs {err.mean()} (scale {s})"


CASES = [
    # B, H, L, block, r, valid, pad, qk, seed
    (2, 2, 1024, 64, 3, (1024, 700), False, False, 1),
    (1, 3, 2048, 128, 2, (1900,), False, False, 2),
    (2, 2, 1536, 64, 3, (1536, 900), False, True, 3),     # query x key
    (2, 2, 1000, 64, 3, (1000, 937), True, False, 4),     # ragged length
    (1, 2, 1100, 64, 3, (1050,), True, True, 5),          # ragged + query x key
    (1, 2, 704, 64, 3, (650,), False, False, 6),          # short: full attention
    (1, 2, 4096, 64, 3, (3500,), False, False, 7),        # long global rows and columns
    (1, 2, 2048, 64, 12, (2048,), False, False, 8),       # many random blocks per row
    (1, 2, 512, 64, 3, (480,), False, False, 9),          # full attention, 8 blocks in two chunks
    (1, 2, 64, 64, 3, (50,), False, False, 11),           # one block: rows not split, no merge
    (2, 3, 960, 64, 3, (960, 17), True, True, 10),        # ragged, one almost fully padded sequence
    (2, 2, 1024, 64, 3, (1024, 0), False, False, 12),     # a fully padded sequence
]


@pytest.mark.parametrize("B,H,L,block,r,valid,pad,qk,seed", CASES)
def test_backward_matches_oracle(B, H, L, block, r, valid, pad, qk, seed):
    announce(f"backward B{B} H{H} L{L} block{block} r{r} valid={valid} pad={pad} qk={qk}")
    inp = workloads.make_case(B, H, L, 64, 200 + seed, valid=valid)
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    dout = bf16_exact(rng.standard_normal((B, H, L, 64)).astype(np.float32))
    nb = -(-L // block)
    full = L <= (5 + 2 * r) * block
    cplan, oplan = plans_for(H, nb, r, seed, full)
    got, st = run_backward(inp, dout, block, r, None if full else cplan, pad=pad, qk=qk)
    assert st == (bbsa.BBSA_OK_FULL_FALLBACK if full else bbsa.BBSA_OK)
    f = oracle.backward_padded if pad else oracle.backward
    want = f(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block, dout, query_key_mask=qk)
    check(got, want, f"backward L{L} pad={pad} qk={qk}")


def test_backward_bigbird_base_workload():
    # The BigBird-base workload (B4 H12 L4096, padded sequences) through the
    # backward; every gradient row of four (batch, head) pairs on different
    # XCD lanes is compared.
    w = workloads.WORKLOADS[2]
    announce("backward BigBird-base workload")
    inp = workloads.make_inputs(2)
    rng = np.random.Generator(np.random.PCG64(400))
    dout = bf16_exact(rng.standard_normal(inp["q"].shape).astype(np.float32))
    cplan, oplan = plans(w.H, w.nb, w.r, w.plan_seed)
    got, st = run_backward(inp, dout, w.block, w.r, cplan)
    assert st == bbsa.BBSA_OK
    for g in got:
        assert np.isfinite(g).all()
    for bh in (0, 13, 30, 47):
        b, h = divmod(bh, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = oracle.backward(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["mask"][b:b + 1], oplan[h:h + 1],
                               w.block, dout[sl])
        check([g[sl] for g in got], want, f"backward {w.name} pair {bh}")


def test_backward_pegasus_workload():
    # The Pegasus-large encoder workload (B8 H16 L4096, valid lengths that
    # end inside a block, so padded and half-padded blocks both occur)
    # through the backward; every gradient row of two (batch, head) pairs on
    # different XCD lanes and batches is compared.
    w = workloads.WORKLOADS[3]
    announce("backward Pegasus-large workload")
    inp = workloads.make_inputs(3)
    rng = np.random.Generator(np.random.PCG64(402))
    dout = bf16_exact(rng.standard_normal(inp["q"].shape).astype(np.float32))
    cplan, oplan = plans(w.H, w.nb, w.r, w.plan_seed)
    got, st = run_backward(inp, dout, w.block, w.r, cplan)
    assert st == bbsa.BBSA_OK
    for g in got:
        assert np.isfinite(g).all()
    for bh in (5, 122):
        b, h = divmod(bh, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = oracle.backward(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["mask"][b:b + 1], oplan[h:h + 1],
                               w.block, dout[sl])
        check([g[sl] for g in got], want, f"backward {w.name} pair {bh}")


@pytest.mark.parametrize("wid,bh", [(4, 9), (5, 15)])
def test_backward_long_workloads(wid, bh):
    # The 16384-token workload (no mask; global rows and columns in four
    # chunks) and the 32768-token block-128 workload (padded tail, key
    # outliers, two 64-query tiles per block) through the backward; every
    # gradient row of one (batch, head) pair on an XCD lane other than 0.
    w = workloads.WORKLOADS[wid]
    announce(f"backward workload {wid} {w.name} pair {bh}")
    inp = workloads.make_inputs(wid)
    rng = np.random.Generator(np.random.PCG64(404 + wid))
    dout = bf16_exact(rng.standard_normal(inp["q"].shape).astype(np.float32))
    cplan, oplan = plans(w.H, w.nb, w.r, w.plan_seed)
    got, st = run_backward(inp, dout, w.block, w.r, cplan, no_mask=not w.masked)
    assert st == bbsa.BBSA_OK
    for g in got:
        assert np.isfinite(g).all()
    b, h = divmod(bh, w.H)
    sl = (slice(b, b + 1), slice(h, h + 1))
    want = oracle.backward(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["mask"][b:b + 1] if w.masked else None,
                           oplan[h:h + 1], w.block, dout[sl])
    check([g[sl] for g in got], want, f"backward {w.name} pair {bh}")


F32_CASES = [
    # B, H, L, block, r, valid, pad, qk, seed
    (1, 2, 1024, 64, 3, (1024,), False, False, 21),       # the fp32 workload's shape
    (2, 2, 1024, 64, 3, (1024, 0), False, False, 22),     # a fully padded sequence
    (2, 2, 1536, 64, 3, (1536, 900), False, True, 23),    # query x key
    (1, 2, 1000, 64, 3, (937,), True, False, 24),         # ragged length
    (1, 2, 2048, 128, 2, (1900,), False, False, 25),      # block 128
    (1, 2, 704, 64, 3, (650,), False, False, 26),         # short: full attention
]


@pytest.mark.parametrize("B,H,L,block,r,valid,pad,qk,seed", F32_CASES)
def test_backward_f32_matches_oracle(B, H, L, block, r, valid, pad, qk, seed):
    announce(f"backward f32 B{B} H{H} L{L} block{block} r{r} valid={valid} pad={pad} qk={qk}")
    inp = workloads.make_case(B, H, L, 64, 200 + seed, dtype="f32", valid=valid)
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    dout = rng.standard_normal((B, H, L, 64)).astype(np.float32)
    nb = -(-L // block)
    full = L <= (5 + 2 * r) * block
    cplan, oplan = plans_for(H, nb, r, seed, full)
    got, st = run_backward(inp, dout, block, r, None if full else cplan, pad=pad, qk=qk, dtype="f32")
    assert st == (bbsa.BBSA_OK_FULL_FALLBACK if full else bbsa.BBSA_OK)
    f = oracle.backward_padded if pad else oracle.backward
    want = f(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block, dout, query_key_mask=qk)
    check(got, want, f"backward f32 L{L} pad={pad} qk={qk}", dtype="f32")


def test_backward_on_two_streams_at_once():
    # Two backward calls that both need the workspace (split global rows),
    # enqueued on two streams without ordering between them: each stream has
    # its own workspace, so both equal their calls made one at a time.
    announce("backward two streams")
    runs = []
    for seed in (41, 42):
        inp = workloads.make_case(1, 2, 4096, 64, seed, valid=(4000,))
        cplan, _ = plans(2, 64, 3, seed)
        q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
        mask = to_dev(inp["mask"], torch.float32)
        ra = torch.from_numpy(cplan).cuda()
        g = torch.Generator(device="cuda").manual_seed(seed)
        dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
        out, lse, _ = bbsa.bbsa_forward_ex(q, k, v, mask, ra, 64, 3, return_lse=True)
        alone = bbsa.bbsa_backward(q, k, v, out, dout, lse, mask, ra, 64, 3)
        torch.cuda.synchronize()
        runs.append(((q, k, v, out, dout, lse, mask, ra), [t.float().cpu().numpy() for t in alone[:3]]))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = []
    for s, (args, _) in zip(streams, runs):
        with torch.cuda.stream(s):
            results.append(bbsa.bbsa_backward(*args, 64, 3))
    torch.cuda.synchronize()
    for (_, alone), got in zip(runs, results):
        assert got[3] == bbsa.BBSA_OK
        for name, t, a in zip(("dq", "dk", "dv"), got[:3], alone):
            assert np.array_equal(t.float().cpu().numpy(), a), f"{name} differs from the call made alone"


@pytest.mark.parametrize("L,block,pad,dtype", [(2048, 64, False, "bf16"), (1000, 64, True, "bf16"),
                                               (2048, 128, False, "bf16"), (1000, 64, True, "f32")])
def test_backward_without_mask(L, block, pad, dtype):
    # A NULL mask: every real key is unmasked; with a ragged length only the
    # positions past L carry the padding bias.
    announce(f"backward no mask L{L} block{block} pad={pad} {dtype}")
    B, H, r, seed = 1, 2, 3, 13
    inp = workloads.make_case(B, H, L, 64, 200 + seed, dtype=dtype)
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    dout = rng.standard_normal((B, H, L, 64)).astype(np.float32)
    if dtype == "bf16":
        dout = bf16_exact(dout)
    nb = -(-L // block)
    cplan, oplan = plans(H, nb, r, seed)
    got, st = run_backward(inp, dout, block, r, cplan, pad=pad, dtype=dtype, no_mask=True)
    assert st == bbsa.BBSA_OK
    f = oracle.backward_padded if pad else oracle.backward
    want = f(inp["q"], inp["k"], inp["v"], None, oplan, block, dout)
    check(got, want, f"backward no mask L{L} pad={pad}", dtype=dtype)


def draw_backward_case(i):
    rng = np.random.Generator(np.random.PCG64(9100 + i))
    block = int(rng.choice([64, 128]))
    r = int(rng.integers(1, 6))
    nb = int(rng.integers(1, max(2, 2048 // block) + 1))
    L = nb * block
    pad = bool(i % 2 == 1 and L > block)
    if pad:
        L -= int(rng.integers(1, block))
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 4))
    dtype = "f32" if i % 3 == 2 else "bf16"
    valid = [int(rng.integers(0, L + 1)) for _ in range(B)] if rng.random() < 0.7 else None
    qk = bool(valid is not None and rng.random() < 0.4)
    q_scale = float(rng.choice([1.0 / 8.0, 0.5, 1.0]))
    return B, H, L, block, r, pad, dtype, valid, qk, q_scale


@pytest.mark.parametrize("i", range(12))
def test_backward_seeded_sweep(i):
    # Seeded draws of shape, block, r, ragged length, dtype, padding, query x
    # key mode and score scale (every case reproducible from its index).
    B, H, L, block, r, pad, dtype, valid, qk, q_scale = draw_backward_case(i)
    announce(f"backward sweep {i}: B{B} H{H} L{L} block{block} r{r} pad={pad} {dtype} valid={valid} "
             f"qk={qk} q_scale={q_scale}")
    inp = workloads.make_case(B, H, L, 64, 9100 + i, dtype=dtype, valid=valid, q_scale=q_scale)
    rng = np.random.Generator(np.random.PCG64(9200 + i))
    dout = rng.standard_normal((B, H, L, 64)).astype(np.float32)
    if dtype == "bf16":
        dout = bf16_exact(dout)
    nb = -(-L // block)
    full = L <= (5 + 2 * r) * block
    cplan, oplan = plans_for(H, nb, r, 9100 + i, full)
    got, st = run_backward(inp, dout, block, r, None if full else cplan, pad=pad, qk=qk, dtype=dtype)
    assert st == (bbsa.BBSA_OK_FULL_FALLBACK if full else bbsa.BBSA_OK)
    f = oracle.backward_padded if pad else oracle.backward
    want = f(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block, dout, query_key_mask=qk)
    check(got, want, f"backward sweep {i}", dtype=dtype)
