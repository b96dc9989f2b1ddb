"""Key blocks whose keys are all padded: the bf16 kernels leave them out of a
query tile's list when the tile attends a key of mask 1 (their probabilities
are exactly zero then).  Checked two ways: against the float64 oracle on
masks with padded blocks anywhere in the sequence, and against the same call
with BBSA_FLAG_KEEP_PADDED_BLOCKS (every block computed), which must give the
same output and log-sum-exp bit for bit.

The masks follow the pages' padding (mask 0 on padded tokens, "models 仓库中
的 BigBird…", section "随机块掩码是如何生成的"), with padded blocks placed in
the middle of the sequence as well as at its end, so that window, global and
random blocks of a row are each sometimes padded."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import announce, assert_close, plans, to_dev

pytestmark = pytest.mark.gpu


def _run(q, k, v, mask, plan, block, r, keep, qk=False):
    out = torch.full_like(q, float("nan"))
    out, lse, st = bbsa.bbsa_forward_ex(q, k, v, mask, plan, block, r, out=out, return_lse=True,
                                        query_key_mask=qk, keep_padded_blocks=keep, warn_fallback=False)
    torch.cuda.synchronize()
    assert st >= 0
    return out, lse


def _first_blocks(H, L, block, r, plan):
    """Key blocks at list position 0 of some work item (block 0 for middle
    rows, each key chunk's first block for the global rows), from the
    library's work map."""
    st, _, rec = bbsa.bbsa_work_map(1, H, L, 64, block, r, bbsa.BBSA_BF16, plan)
    assert st >= 0
    return {int(row[16 + row[8]]) for row in rec if row[9] > row[8]}


def _mask_with_holes(B, L, block, rng, frac_blocks, avoid):
    """Whole padded blocks at random places, none of them at a list position
    0 (where a padded first block would make the kept and the dropped run
    round differently; the edge-mask test covers that case)."""
    nb = L // block
    m = np.ones((B, L), np.float32)
    allowed = np.array([kb for kb in range(nb) if kb not in avoid])
    for b in range(B):
        n = max(1, int(frac_blocks * nb))
        for kb in rng.choice(allowed, size=min(n, len(allowed)), replace=False):
            m[b, kb * block:(kb + 1) * block] = 0.0
    return m


CASES = [
    # (B, H, L, block, r, seed, fraction of padded blocks, query x key masking)
    (2, 3, 2048, 64, 3, 1, 0.3, False),
    (2, 3, 2048, 64, 3, 2, 0.3, True),
    (1, 2, 4096, 128, 2, 3, 0.25, False),
    (1, 2, 4096, 128, 2, 4, 0.25, True),
    (2, 2, 1152, 64, 3, 5, 0.5, False),
    (1, 2, 2048, 64, 7, 6, 0.4, False),    # long random lists
]


@pytest.mark.parametrize("B,H,L,block,r,seed,frac,qk", CASES)
def test_padded_blocks_match_oracle_and_keep(B, H, L, block, r, seed, frac, qk):
    announce(f"padded blocks B{B} H{H} L{L} b{block} r{r} seed{seed} frac{frac} qk{qk}")
    rng = np.random.default_rng(seed)
    inp = workloads.make_case(B, H, L, 64, seed, "bf16")
    nb = L // block
    c_plan, o_plan = plans(H, nb, r, seed)
    inp["mask"] = _mask_with_holes(B, L, block, rng, frac, _first_blocks(H, L, block, r, c_plan))
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32)
    ra = torch.from_numpy(c_plan).cuda()
    out, lse = _run(q, k, v, mask, ra, block, r, keep=False, qk=qk)
    out_k, lse_k = _run(q, k, v, mask, ra, block, r, keep=True, qk=qk)
    assert torch.equal(out, out_k), "skipping padded blocks changed the output"
    assert torch.equal(lse, lse_k), "skipping padded blocks changed the log-sum-exp"
    want, want_lse = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], o_plan, block,
                                    query_key_mask=qk, return_lse=True)
    assert_close(out.float().cpu().numpy().astype(np.float64), want, "bf16",
                 f"padded blocks B{B} H{H} L{L} b{block} r{r} qk{qk}")
    lse_err = float(np.abs(lse.cpu().numpy() - want_lse).max())
    assert lse_err <= 1e-2, f"lse max abs {lse_err}"


EDGE_MASKS = {
    # Only block 0 holds valid keys: middle rows keep block 0 alone.
    "only_block0": lambda m, block: m.__setitem__((slice(None), slice(block, None)), 0.0),
    # Leading padding: position 0 of every middle row (key block 0) is padded.
    "leading": lambda m, block: m.__setitem__((slice(None), slice(0, 3 * block)), 0.0),
    # Padded blocks next to blocks whose keys are all 0.5 (never dropped, and
    # no key of mask 1 among them).
    "fractional": lambda m, block: (m.__setitem__((slice(None), slice(0, 8 * block)), 0.5),
                                    m.__setitem__((slice(None), slice(8 * block, None)), 0.0)),
    # A single valid key in an otherwise padded sequence.
    "one_key": lambda m, block: (m.__setitem__((slice(None), slice(None)), 0.0),
                                 m.__setitem__((slice(None), 5 * block + 7), 1.0)),
    # Every key padded: nothing is dropped, the rows are uniform softmaxes.
    "all_padded": lambda m, block: m.__setitem__((slice(None), slice(None)), 0.0),
}


@pytest.mark.parametrize("name", sorted(EDGE_MASKS))
@pytest.mark.parametrize("block", [64, 128])
def test_padded_block_edge_masks(name, block):
    B, H, r, seed = 2, 2, 3, 21
    L = 24 * block
    announce(f"padded-block edge mask {name} block {block}")
    inp = workloads.make_case(B, H, L, 64, seed, "bf16")
    m = np.ones((B, L), np.float32)
    EDGE_MASKS[name](m, block)
    inp["mask"] = m
    nb = L // block
    c_plan, o_plan = plans(H, nb, r, seed)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(m, torch.float32)
    ra = torch.from_numpy(c_plan).cuda()
    out, lse = _run(q, k, v, mask, ra, block, r, keep=False)
    out_k, lse_k = _run(q, k, v, mask, ra, block, r, keep=True)
    got = out.float().cpu().numpy().astype(np.float64)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], m, o_plan, block)
    assert_close(got, want, "bf16", f"edge mask {name} b{block}")
    # With block 0 padded the first block a tile walks carries padded keys
    # only, and the reference max moves once a valid block follows: the two
    # runs then round differently (both are checked against the oracle).
    if name not in ("leading", "one_key"):
        assert torch.equal(out, out_k), "skipping padded blocks changed the output"
        assert torch.equal(lse, lse_k), "skipping padded blocks changed the log-sum-exp"
    else:
        assert_close(out_k.float().cpu().numpy().astype(np.float64), want, "bf16",
                     f"edge mask {name} b{block} keep")


@pytest.mark.parametrize("wid", [2, 3, 5])
def test_full_size_skip_equals_keep(wid):
    """At the benchmark shapes every output row and every log-sum-exp of the
    default call equals the call that computes every block."""
    w = workloads.WORKLOADS[wid]
    announce(f"skip vs keep at full size {w.name}")
    x = workloads.make_inputs(wid)
    q, k, v = (to_dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(x["mask"], torch.float32)
    c_plan, _ = plans(w.H, w.nb, w.r, w.plan_seed)
    ra = torch.from_numpy(c_plan).cuda()
    out, lse = _run(q, k, v, mask, ra, w.block, w.r, keep=False)
    out_k, lse_k = _run(q, k, v, mask, ra, w.block, w.r, keep=True)
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out, out_k)
    assert torch.equal(lse, lse_k)


# Backward: a step whose 32 keys all have mask 0 adds exactly nothing to the
# rows whose log-sum-exp shows a real key (and whose own mask is 1 under
# query x key masking), so the kernels skip it; computing every step
# (BBSA_FLAG_KEEP_PADDED_BLOCKS) gives the same gradients bit for bit.

def _backward(q, k, v, dout, mask, plan, block, r, qk=False, pad=False):
    """One forward (saving the LSE), then the backward twice on its output:
    skipping the padded steps and computing every step."""
    out, lse, st = bbsa.bbsa_forward_ex(q, k, v, mask, plan, block, r, return_lse=True, query_key_mask=qk,
                                        pad_to_block=pad, warn_fallback=False)
    res = []
    for keep in (False, True):
        grads = [torch.full_like(q, float("nan")) for _ in range(3)]
        dq, dk, dv, st2 = bbsa.bbsa_backward(q, k, v, out, dout, lse, mask, plan, block, r, dq=grads[0],
                                             dk=grads[1], dv=grads[2], query_key_mask=qk, pad_to_block=pad,
                                             keep_padded_blocks=keep)
        torch.cuda.synchronize()
        assert st >= 0 and st2 == st
        res.append((dq, dk, dv))
    return res


BWD_CASES = [
    # (B, H, L, block, r, seed, fraction of padded blocks, query x key masking, leading padding)
    (2, 2, 2048, 64, 3, 31, 0.3, False, False),
    (2, 2, 2048, 64, 3, 32, 0.3, True, False),
    (1, 2, 4096, 128, 2, 33, 0.25, False, True),
    (2, 2, 704, 64, 3, 34, 0.4, False, False),      # full-attention fallback
    (1, 2, 2048, 64, 12, 35, 0.3, False, False),    # 17-block lists: the probe's three passes
]


@pytest.mark.parametrize("B,H,L,block,r,seed,frac,qk,lead", BWD_CASES)
def test_backward_padded_steps(B, H, L, block, r, seed, frac, qk, lead):
    announce(f"backward padded steps B{B} H{H} L{L} b{block} r{r} qk{qk} lead{lead}")
    rng = np.random.default_rng(seed)
    inp = workloads.make_case(B, H, L, 64, seed, "bf16")
    nb = L // block
    full = L <= (5 + 2 * r) * block
    c_plan, o_plan = plans(H, nb, r, seed) if not full else (None, np.zeros((H, nb - 2, r), np.int32))
    m = np.ones((B, L), np.float32)
    for b in range(B):
        for kb in rng.choice(np.arange(nb), size=max(1, int(frac * nb)), replace=False):
            m[b, kb * block:(kb + 1) * block] = 0.0
    if lead:
        m[:, :block] = 0.0
    inp["mask"] = m
    dout_np = workloads.round_to_bf16(rng.standard_normal((B, H, L, 64)).astype(np.float32))
    q, k, v, dout = (to_dev(x, torch.bfloat16) for x in (inp["q"], inp["k"], inp["v"], dout_np))
    mask = to_dev(m, torch.float32)
    ra = None if c_plan is None else torch.from_numpy(c_plan).cuda()
    got, ref = _backward(q, k, v, dout, mask, ra, block, r, qk=qk)
    for name, g, w in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(g.float()).all(), f"{name}: unwritten entries"
        assert torch.equal(g, w), f"{name}: skipping padded steps changed the gradient"
    want = oracle.backward(inp["q"], inp["k"], inp["v"], m, o_plan, block, dout_np, query_key_mask=qk)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        g = g.float().cpu().numpy().astype(np.float64)
        s = max(1.0, float(np.abs(w).max()))
        err = np.abs(g - w)
        announce(f"backward padded steps {name}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} scale={s:.3g}")
        assert err.max() <= 2e-2 * s and err.mean() <= 2e-3 * s, f"{name}: max abs {err.max()}"


def test_backward_full_size_skip_equals_keep():
    """The BigBird-base workload's gradients with and without the skipped
    steps, bit for bit."""
    w = workloads.WORKLOADS[2]
    announce(f"backward skip vs keep at full size {w.name}")
    x = workloads.make_inputs(2)
    rng = np.random.Generator(np.random.PCG64(401))
    dout = to_dev(workloads.round_to_bf16(rng.standard_normal(x["q"].shape).astype(np.float32)), torch.bfloat16)
    q, k, v = (to_dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(x["mask"], torch.float32)
    c_plan, _ = plans(w.H, w.nb, w.r, w.plan_seed)
    ra = torch.from_numpy(c_plan).cuda()
    got, ref = _backward(q, k, v, dout, mask, ra, w.block, w.r)
    for name, g, r_ in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(g.float()).all(), f"{name}: unwritten entries"
        assert torch.equal(g, r_), f"{name} differs"


def test_keep_flag_covers_scores_beyond_the_padding_bias():
    """Scores so large that a padded key still outweighs the valid ones
    under the -10000 bias (here 16384 - 10000 against about 0): the
    default call leaves such a key out (its documented limit), while
    BBSA_FLAG_KEEP_PADDED_BLOCKS computes it and matches the oracle."""
    B, H, L, block, r, seed = 1, 1, 1536, 64, 3, 41
    announce("padded key beyond the bias, keep flag")
    inp = workloads.make_case(B, H, L, 64, seed, "bf16")
    nb = L // block
    pad_blk = nb - 4
    inp["q"][:] = 16.0                           # every query row: q = 16 (exact in bf16)
    inp["k"] = workloads.round_to_bf16(inp["k"] * np.float32(0.01))   # other scores: about N(0, 1.6)
    inp["k"][0, 0, pad_blk * block:(pad_blk + 1) * block, :] = 16.0   # padded keys: score 64 * 256 = 16384
    m = np.ones((B, L), np.float32)
    m[:, pad_blk * block:(pad_blk + 1) * block] = 0.0
    inp["mask"] = m
    c_plan, o_plan = plans(H, nb, r, seed)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(m, torch.float32)
    ra = torch.from_numpy(c_plan).cuda()
    out_k, _ = _run(q, k, v, mask, ra, block, r, keep=True)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], m, o_plan, block)
    assert_close(out_k.float().cpu().numpy().astype(np.float64), want, "bf16", "keep flag, scores beyond the bias")


@pytest.mark.parametrize("draw", range(10))
def test_padded_blocks_seeded_sweep(draw):
    """Seeded draws of shape, block size, r, query x key mode and a mask
    with whole padded blocks, partially padded blocks and fractional values:
    forward and backward against the oracle; the backward bit for bit
    against computing every step, the forward bit for bit where no list
    starts with a padded block (else to bf16 rounding)."""
    rng = np.random.Generator(np.random.PCG64(9300 + draw))
    block = int(rng.choice([64, 128]))
    r = int(rng.integers(1, 6))
    nb = int(rng.integers(6 + 2 * r, 6 + 2 * r + 14))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    L = nb * block
    qk = bool(draw % 3 == 2)
    seed = 9400 + draw
    announce(f"padded sweep {draw}: B{B} H{H} L{L} b{block} r{r} qk{qk}")
    inp = workloads.make_case(B, H, L, 64, seed, "bf16")
    m = np.ones((B, L), np.float32)
    for b in range(B):
        for kb in rng.choice(np.arange(nb), size=int(rng.integers(1, nb // 2)), replace=False):
            kind = rng.integers(0, 4)
            lo, hi = kb * block, (kb + 1) * block
            if kind <= 1:
                m[b, lo:hi] = 0.0                                   # whole padded block
            elif kind == 2:
                m[b, lo + int(rng.integers(1, block)):hi] = 0.0     # partially padded block
            else:
                m[b, lo:hi] = np.float32(rng.choice([0.0, 0.25, 1.0]))
    inp["mask"] = m
    c_plan, o_plan = plans(H, nb, r, seed)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(m, torch.float32)
    ra = torch.from_numpy(c_plan).cuda()
    out, lse = _run(q, k, v, mask, ra, block, r, keep=False, qk=qk)
    out_k, lse_k = _run(q, k, v, mask, ra, block, r, keep=True, qk=qk)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], m, o_plan, block, query_key_mask=qk)
    assert_close(out.float().cpu().numpy().astype(np.float64), want, "bf16", f"padded sweep {draw} forward")
    first = _first_blocks(H, L, block, r, c_plan)
    blocks = m.reshape(B, nb, block)
    if not any((blocks[:, f] == 0).all() for f in first):
        assert torch.equal(out, out_k) and torch.equal(lse, lse_k), "forward: skip and keep differ"
    else:
        assert float((out.float() - out_k.float()).abs().max()) <= 1.6e-2
    dout_np = workloads.round_to_bf16(rng.standard_normal((B, H, L, 64)).astype(np.float32))
    dout = to_dev(dout_np, torch.bfloat16)
    got, ref = _backward(q, k, v, dout, mask, ra, block, r, qk=qk)
    for name, g, w in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(g.float()).all(), f"{name}: unwritten entries"
        assert torch.equal(g, w), f"{name}: skipping padded steps changed the gradient"
    want_g = oracle.backward(inp["q"], inp["k"], inp["v"], m, o_plan, block, dout_np, query_key_mask=qk)
    for name, g, w in zip(("dq", "dk", "dv"), got, want_g):
        g = g.float().cpu().numpy().astype(np.float64)
        s = max(1.0, float(np.abs(w).max()))
        err = np.abs(g - w)
        assert err.max() <= 2e-2 * s and err.mean() <= 2e-3 * s, f"{name}: max abs {err.max()} (scale {s})"
