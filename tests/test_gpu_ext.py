"""Parity of bbsa_forward_ex with the oracle on MI355X: the row log-sum-exp,
the query x key masking mode ("models 仓库中的 BigBird…", section
"随机块掩码是如何生成的": the band mask is the product of the query-side and
key-side masks) and lengths that are not a multiple of the block
("BigBirdPegasus…", section "序列长度的块对齐要求": the encoder pads to the
block and trims its output).

Tolerances: outputs as for bbsa_forward.  Row log-sum-exp: on the bf16 path
the row sums add bf16-rounded probabilities (relative error up to 2^-9 of
the sum, i.e. about 2e-3 in lse) -> max abs 5e-3; on the fp32 path
1e-4 + 2^-23 |lse| (the final fp32 rounding of a value near -10000 on fully
padded rows is up to 6e-4).
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import announce, assert_close, oracle_slices, plans, to_dev, varied_blocks

pytestmark = pytest.mark.gpu

BF16_LSE_MAX_ABS = 5e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bbsa.lib()


def check_lse(got, want, dtype, what):
    assert np.isfinite(got).all(), f"{what}: non-finite lse"
    err = np.abs(got - want)
    announce(f"{what} lse max_abs={err.max():.3e}")
    if dtype == "f32":
        bound = 1e-4 + 2.0 ** -23 * np.abs(want)
        assert (err <= bound).all(), f"{what}: lse error {err.max()}"
    else:
        assert err.max() <= BF16_LSE_MAX_ABS, f"{what}: lse error {err.max()}"


def run_ex(inp, block, r, dtype, plan, pad=False, qk=False, use_mask=True):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (to_dev(inp[n], tdt) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32) if use_mask else None
    ra = torch.from_numpy(plan).cuda() if plan is not None else None
    B, H, L, _ = q.shape
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, L), float("nan"), dtype=torch.float32, device="cuda")
    out, lse, st = bbsa.bbsa_forward_ex(q, k, v, mask, ra, block, r, out=out, lse=lse, pad_to_block=pad,
                                        query_key_mask=qk, warn_fallback=False)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), st


def ref(inp, plan, block, pad=False, qk=False, use_mask=True):
    m = inp["mask"] if use_mask else None
    f = oracle.forward_padded if pad else oracle.forward
    return f(inp["q"], inp["k"], inp["v"], m, plan, block, query_key_mask=qk, return_lse=True)


CASES = [
    # B, H, L, block, r, dtype, valid, pad, qk
    (2, 2, 1024, 64, 3, "bf16", (1024, 700), False, False),    # lse, key-side mask
    (2, 2, 1024, 64, 3, "f32", (1024, 700), False, False),
    (1, 2, 8192, 64, 3, "bf16", (8000,), False, False),        # lse through the merge kernel
    (1, 2, 2048, 128, 2, "f32", (2000,), False, False),        # fp32 partials + merge
    (2, 2, 1536, 64, 3, "bf16", (1536, 900), False, True),     # query x key
    (2, 2, 1536, 64, 3, "f32", (1400, 900), False, True),
    (1, 2, 8192, 64, 3, "bf16", (6000,), False, True),         # query x key through the merge kernel
    (2, 3, 1000, 64, 3, "bf16", (1000, 937), True, False),     # ragged length, last block partial
    (2, 3, 1000, 64, 3, "f32", (1000, 937), True, False),
    (1, 2, 5000, 128, 2, "bf16", (4900,), True, False),        # ragged, block 128
    (1, 2, 9000, 64, 3, "bf16", (9000,), True, False),         # ragged, merge kernel
    (2, 2, 1000, 64, 3, "bf16", (1000, 800), True, True),      # ragged + query x key
    (1, 2, 1100, 64, 3, "f32", (1050,), True, True),
    (1, 2, 700, 64, 3, "bf16", (650,), True, False),           # ragged + short: full attention
    (1, 2, 333, 64, 1, "f32", (300,), True, False),
    (1, 1, 1024, 64, 3, "f32", (0,), False, False),            # fully padded: lse near -10000
    (1, 1, 1024, 64, 3, "bf16", (0,), False, True),            # fully padded, query x key
    (1, 1, 1000, 64, 3, "bf16", (0,), True, False),            # ragged + fully padded: past L reads as 0
]


@pytest.mark.parametrize("B,H,L,block,r,dtype,valid,pad,qk", CASES)
def test_forward_ex_matches_oracle(B, H, L, block, r, dtype, valid, pad, qk):
    announce(f"ex B{B} H{H} L{L} block{block} r{r} {dtype} valid={valid} pad={pad} qk={qk}")
    inp = workloads.make_case(B, H, L, 64, 80 + L % 97, dtype=dtype, valid=valid)
    nb = -(-L // block)
    full = L <= (5 + 2 * r) * block
    # The oracle takes its fallback from the plan's r, so it gets the plan
    # even when the library (which ignores it then) gets none.
    cplan, oplan = plans(H, nb, r, 80)
    got, lse, st = run_ex(inp, block, r, dtype, None if full else cplan, pad=pad, qk=qk)
    assert st == (bbsa.BBSA_OK_FULL_FALLBACK if full else bbsa.BBSA_OK)
    want, want_lse = ref(inp, oplan, block, pad=pad, qk=qk)
    assert_close(got, want, dtype, f"ex L{L} {dtype} pad={pad} qk={qk}")
    check_lse(lse, want_lse, dtype, f"ex L{L} {dtype} pad={pad} qk={qk}")


def test_ragged_length_writes_nothing_past_the_tensors():
    # Output and lse sit inside larger buffers filled with a sentinel: rows
    # past L (the padded positions) must never be written.
    announce("ragged guard regions")
    B, H, L, block, r = 1, 2, 1000, 64, 3
    inp = workloads.make_case(B, H, L, 64, 91, valid=(950,))
    cplan, oplan = plans(H, 16, r, 91)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32)
    n = q.numel()
    big = torch.full((n + 2 * 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[4096:4096 + n].view(q.shape)
    lbig = torch.full((B * H * L + 2 * 1024,), 7.0, dtype=torch.float32, device="cuda")
    lse = lbig[1024:1024 + B * H * L].view(B, H, L)
    bbsa.bbsa_forward_ex(q, k, v, mask, torch.from_numpy(cplan).cuda(), block, r, out=out, lse=lse,
                         pad_to_block=True)
    torch.cuda.synchronize()
    assert (big[:4096] == 7.0).all() and (big[4096 + n:] == 7.0).all()
    assert (lbig[:1024] == 7.0).all() and (lbig[1024 + B * H * L:] == 7.0).all()
    want, want_lse = ref(inp, oplan, block, pad=True)
    assert_close(out.float().cpu().numpy().astype(np.float64), want, "bf16", "ragged guarded")
    check_lse(lse.cpu().numpy().astype(np.float64), want_lse, "bf16", "ragged guarded")


def test_flags_zero_is_bbsa_forward_bitwise():
    announce("forward_ex flags 0 == forward")
    inp = workloads.make_case(2, 3, 2048, 64, 92, valid=(2048, 1500))
    cplan, _ = plans(3, 32, 3, 92)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32)
    ra = torch.from_numpy(cplan).cuda()
    a, _ = bbsa.bbsa_forward(q, k, v, mask, ra, 64, 3)
    b, _ = bbsa.bbsa_forward_ex(q, k, v, mask, ra, 64, 3)
    c, _, _ = bbsa.bbsa_forward_ex(q, k, v, mask, ra, 64, 3, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("wid,qk,pad_L", [(3, True, None), (2, False, 4000), (4, False, None)])
def test_full_size_ex(wid, qk, pad_L):
    # Full-size workloads through bbsa_forward_ex: the Pegasus-large encoder
    # shape in query x key mode (every row), the BigBird-base shape cut to a
    # ragged 4000 tokens (every row), and the 16384-token shape's lse (the
    # merge kernel's rows; every row of two pairs, sampled blocks elsewhere).
    w = workloads.WORKLOADS[wid]
    announce(f"full-size ex workload {wid} qk={qk} L={pad_L or w.L}")
    inp = workloads.make_inputs(wid)
    L = pad_L or w.L
    if pad_L:
        inp = {n: np.ascontiguousarray(inp[n][:, :, :L]) for n in ("q", "k", "v")} | {
            "mask": np.ascontiguousarray(inp["mask"][:, :L])}
    nb = -(-L // w.block)
    cplan, oplan = plans(w.H, nb, w.r, w.plan_seed)
    got, lse, st = run_ex(inp, w.block, w.r, w.dtype, cplan, pad=pad_L is not None, qk=qk)
    assert st == bbsa.BBSA_OK
    assert np.isfinite(got).all() and np.isfinite(lse).all()
    if pad_L:
        want, want_lse = ref(inp, oplan, w.block, pad=True)
        assert_close(got, want, w.dtype, f"{w.name} cut to {L} tokens (padded to the block) all rows")
        check_lse(lse, want_lse, w.dtype, f"{w.name} cut to {L}")
        return
    full_pairs = None if wid == 3 else (0, 9)
    jobs = []
    for b in range(w.B):
        for h in range(w.H):
            bh = b * w.H + h
            qbs = None if full_pairs is None or bh in full_pairs else varied_blocks(w.nb, bh, seed=5)
            jobs.append((b, h, qbs))

    def one(job):
        b, h, qbs = job
        o, l = oracle.forward(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1], inp["v"][b:b + 1, h:h + 1],
                              inp["mask"][b:b + 1], oplan[h:h + 1], w.block, query_blocks=qbs,
                              query_key_mask=qk, return_lse=True)
        return o[0, 0], l[0, 0]

    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(8) as ex:
        wants = list(ex.map(one, jobs))
    g_all, w_all, gl, wl = [], [], [], []
    for (b, h, qbs), (wo, wlse) in zip(jobs, wants):
        blocks = range(w.nb) if qbs is None else qbs
        rows = np.concatenate([np.arange(i * w.block, (i + 1) * w.block) for i in blocks])
        g_all.append(got[b, h, rows])
        w_all.append(wo)
        gl.append(lse[b, h, rows])
        wl.append(wlse)
    assert_close(np.concatenate(g_all), np.concatenate(w_all), w.dtype, f"{w.name} ex qk={qk}")
    check_lse(np.concatenate(gl), np.concatenate(wl), w.dtype, f"{w.name} ex qk={qk}")
