"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Small cases are compared over every output element.  The five workloads run
at their full sizes in the launch configuration the benchmark times: the
first three are compared on every row, the two longest on every row of two
(batch, head) pairs and on sampled query blocks of every other pair; the
rows inside each sequence's valid length are also reported on their own.
Output buffers start as NaN, so a row the kernels never write fails.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import (announce, assert_close, gather_rows, oracle_slices, plans, run_gpu,
                         sample_blocks, to_dev, valid_query_rows, varied_blocks)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bbsa.lib()


SMALL = [
    # B, H, L, block, r, dtype, valid lengths (None = unpadded), seed
    (2, 3, 1024, 64, 3, "bf16", (700, 1024), 1),
    (1, 2, 768, 64, 3, "bf16", None, 2),          # smallest sparse length at r=3 (nb = 12)
    (1, 2, 2048, 128, 2, "bf16", (1900,), 3),      # block 128, partial block
    (2, 2, 4096, 64, 3, "bf16", (3072, 4000), 4),  # full rows: four chunks merged in one workgroup
    (1, 3, 1536, 64, 1, "bf16", None, 5),
    (1, 2, 2560, 64, 5, "bf16", (2000,), 6),
    (1, 1, 5120, 128, 3, "bf16", (4321,), 7),      # block 128, 40 blocks: 8 chunks, two groups + merge kernel
    (1, 2, 1024, 64, 3, "f32", None, 8),
    (2, 1, 2048, 128, 2, "f32", (1500, 2048), 9),
    (1, 2, 4096, 64, 2, "f32", (3333,), 10),
]


@pytest.mark.parametrize("B,H,L,block,r,dtype,valid,seed", SMALL)
def test_small_full_compare(B, H, L, block, r, dtype, valid, seed):
    announce(f"small B{B} H{H} L{L} block{block} r{r} {dtype} valid={valid} seed={seed}")
    inp = workloads.make_case(B, H, L, 64, seed, dtype=dtype, valid=valid)
    cplan, oplan = plans(H, L // block, r, seed)
    got, st = run_gpu(inp, block, r, dtype, cplan)
    assert st == bbsa.BBSA_OK
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block)
    assert_close(got, want, dtype, f"small L{L}")



def test_f32_large_call_without_middle_split():
    # 1472 work items (5888 wavefronts): enough that the fp32 path leaves
    # middle rows whole (smaller fp32 calls split them into two key parts).
    announce("f32 without middle split B4 H8 L2048")
    inp = workloads.make_case(4, 8, 2048, 64, 16, dtype="f32", valid=(2048, 1900, 1500, 2048))
    cplan, oplan = plans(8, 32, 3, 16)
    got, st = run_gpu(inp, 64, 3, "f32", cplan)
    assert st == bbsa.BBSA_OK
    blocks = sample_blocks(32)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, 64, query_blocks=blocks)
    assert_close(gather_rows(got, blocks, 64), want, "f32", "f32 no split")

# The full-row chunk length grows with the launch's work (1024, 2048 or
# 4096 keys); four chunks share a workgroup and merge in LDS, more leave
# partials for the merge kernel.  One case per length and merge path, padded
# so that whole chunks of the global rows lie in the padding.
CHUNK_CASES = [
    # B, H, L, r, expected (chunk blocks, chunks per full row), valid lengths
    (8, 16, 8192, 3, (32, 4), (8192, 7000, 6500, 8192, 4000, 8000, 7777, 6144)),
    (2, 16, 16384, 3, (32, 8), (16384, 9000)),
    (4, 16, 16384, 3, (64, 4), (16384, 12000, 3000, 15999)),
    (4, 16, 32768, 3, (64, 8), (32768, 20000, 30001, 9000)),
]


@pytest.mark.parametrize("B,H,L,r,chunking,valid", CHUNK_CASES)
def test_full_row_chunk_lengths(B, H, L, r, chunking, valid):
    block, nb, seed = 64, L // 64, 21
    announce(f"chunk lengths B{B} H{H} L{L} r{r} chunking {chunking}")
    cplan, oplan = plans(H, nb, r, seed)
    st, _, rec = bbsa.bbsa_work_map(B, H, L, 64, block, r, bbsa.BBSA_BF16, cplan)
    glob = rec[rec[:, 6] >= 0]
    assert st == bbsa.BBSA_OK and (glob[:, 11] == chunking[1]).all()
    assert ((glob[:, 9] - glob[:, 8]) == chunking[0]).all()
    inp = workloads.make_case(B, H, L, 64, seed, valid=valid)
    got, st = run_gpu(inp, block, r, "bf16", cplan)
    assert st == bbsa.BBSA_OK
    assert np.isfinite(got).all(), "non-finite output: some row was not written"
    # Both global rows and two middle rows of one pair per XCD lane and of
    # the last pair.
    jobs = []
    for bh in sorted(set(list(range(min(8, B * H))) + [B * H - 1])):
        b, h = divmod(bh, H)
        jobs.append((b, h, [0, 1 + bh % (nb - 2), nb // 2, nb - 1]))
    wants = oracle_slices(inp, oplan, block, jobs)
    g = np.concatenate([gather_rows(got[b, h], qbs, block) for b, h, qbs in jobs])
    assert_close(g, np.concatenate(wants), "bf16", f"chunks B{B} H{H} L{L}")


FALLBACK = [
    (1, 2, 704, 64, 3, "bf16", (650,)),    # (5 + 2*3) * 64 = 704: full attention
    (2, 1, 1152, 128, 2, "bf16", None),    # (5 + 2*2) * 128
    (1, 1, 2880, 64, 20, "bf16", (2800,)), # 45 blocks: full rows are chunked and merged
    (1, 2, 448, 64, 1, "f32", None),
    # Rows shorter than four blocks: some of the four chunks of a row are empty.
    (1, 2, 64, 64, 1, "bf16", None),
    (2, 1, 128, 64, 1, "bf16", (100, 128)),
    (1, 1, 192, 64, 2, "bf16", None),
    (1, 2, 256, 128, 1, "bf16", (200,)),
    (1, 1, 128, 64, 1, "f32", None),
]


@pytest.mark.parametrize("B,H,L,block,r,dtype,valid", FALLBACK)
def test_short_sequence_falls_back_to_full_attention(B, H, L, block, r, dtype, valid):
    announce(f"fallback B{B} H{H} L{L} block{block} r{r} {dtype}")
    inp = workloads.make_case(B, H, L, 64, 11, dtype=dtype, valid=valid)
    got, st = run_gpu(inp, block, r, dtype, None)
    assert st == bbsa.BBSA_OK_FULL_FALLBACK
    want = oracle.full_attention(inp["q"], inp["k"], inp["v"], inp["mask"])
    assert_close(got, want, dtype, f"fallback L{L}")


def test_fallback_boundary_status():
    # 704 falls back, 768 does not (block 64, r 3).
    for L, want in ((704, bbsa.BBSA_OK_FULL_FALLBACK), (768, bbsa.BBSA_OK)):
        announce(f"boundary L{L}")
        inp = workloads.make_case(1, 1, L, 64, 12)
        plan = bbsa.bbsa_plan_rand_attn(1, L // 64, 3, 0) if L > 704 else None
        _, st = run_gpu(inp, 64, 3, "bf16", plan)
        assert st == want


def test_null_mask_equals_all_ones_mask():
    announce("null mask")
    inp = workloads.make_case(2, 2, 2048, 64, 13)
    cplan, _ = plans(2, 32, 3, 3)
    a, _ = run_gpu(inp, 64, 3, "bf16", cplan, use_mask=True)
    b, _ = run_gpu(inp, 64, 3, "bf16", cplan, use_mask=False)
    assert np.array_equal(a, b)


def test_batch_independence_bitwise():
    announce("batch independence")
    inp = workloads.make_case(3, 2, 2048, 64, 14, valid=(2048, 1111, 1800))
    cplan, _ = plans(2, 32, 3, 5)
    whole, _ = run_gpu(inp, 64, 3, "bf16", cplan)
    for b in range(3):
        one = {kk: inp[kk][b:b + 1] for kk in ("q", "k", "v", "mask")}
        alone, _ = run_gpu(one, 64, 3, "bf16", cplan)
        assert np.array_equal(alone[0], whole[b]), b


def test_deterministic_bitwise():
    announce("determinism")
    inp = workloads.make_case(2, 4, 4096, 64, 15, valid=(4096, 3500))
    cplan, _ = plans(4, 64, 3, 6)
    a, _ = run_gpu(inp, 64, 3, "bf16", cplan)
    b, _ = run_gpu(inp, 64, 3, "bf16", cplan)
    assert np.array_equal(a, b)


def test_fully_padded_sequence_matches_oracle():
    # Every key padded: the constant -10000 cancels; rows are plain softmax.
    announce("fully padded")
    inp = workloads.make_case(1, 2, 1024, 64, 16, valid=(0,))
    cplan, oplan = plans(2, 16, 3, 7)
    got, _ = run_gpu(inp, 64, 3, "bf16", cplan)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, 64)
    assert_close(got, want, "bf16", "fully padded")


@pytest.mark.parametrize("B,H,L,block,valid", [
    (1, 2, 1024, 64, (0,)),          # every key padded: a constant -10000 on every score
    (2, 2, 2048, 128, (0, 2048)),    # one fully padded sequence next to an unpadded one
])
def test_f32_fully_padded_sequence_matches_oracle(B, H, L, block, valid):
    announce(f"f32 fully padded B{B} H{H} L{L} block{block} valid={valid}")
    inp = workloads.make_case(B, H, L, 64, 19, dtype="f32", valid=valid)
    r = 3 if block == 64 else 2
    cplan, oplan = plans(H, L // block, r, 19)
    got, _ = run_gpu(inp, block, r, "f32", cplan)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block)
    assert_close(got, want, "f32", f"f32 fully padded L{L}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_padded_query_rows_match_oracle(dtype):
    # Valid lengths that end inside a block: the query rows past the valid
    # length are computed with the same formula (key-side masking only) and
    # compared like every other row; the valid rows are reported on their own.
    announce(f"padded query rows {dtype}")
    B, H, L = 3, 2, 2048
    valid = (1000, 1537, 64)
    inp = workloads.make_case(B, H, L, 64, 20, dtype=dtype, valid=valid)
    cplan, oplan = plans(H, L // 64, 3, 20)
    got, _ = run_gpu(inp, 64, 3, dtype, cplan)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, 64)
    assert_close(got, want, dtype, f"padded query rows {dtype} all rows")
    for b, n in enumerate(valid):
        assert_close(got[b, :, n:], want[b, :, n:], dtype, f"padded query rows {dtype} b{b} padded rows")
        assert_close(got[b, :, :n], want[b, :, :n], dtype, f"padded query rows {dtype} b{b} valid rows")


def test_out_of_range_plan_stays_in_bounds():
    # Indices are clamped: no fault, finite output (result unspecified).
    announce("clamped plan")
    inp = workloads.make_case(1, 2, 1024, 64, 17)
    bad = np.full((2, 14, 3), 10**6, dtype=np.int32)
    bad[1] = -5
    got, st = run_gpu(inp, 64, 3, "bf16", bad)
    assert st == bbsa.BBSA_OK and np.isfinite(got).all()


def test_output_guard_regions_untouched():
    announce("guard regions")
    inp = workloads.make_case(1, 2, 1024, 64, 18, valid=(900,))
    cplan, oplan = plans(2, 16, 3, 8)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32)
    n = q.numel()
    big = torch.full((n + 2 * 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[4096:4096 + n].view(q.shape)
    bbsa.bbsa_forward(q, k, v, mask, torch.from_numpy(cplan).cuda(), 64, 3, out=out)
    torch.cuda.synchronize()
    assert (big[:4096] == 7.0).all() and (big[4096 + n:] == 7.0).all()
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, 64)
    assert_close(out.float().cpu().numpy().astype(np.float64), want, "bf16", "guarded")


# Full-size workloads, in the launch configuration the benchmark times.
# C1-C3: every row of every (batch, head).  C4, C5: every row of two
# (batch, head) pairs that the kernel maps to different XCD lanes (pair x
# runs on lane x mod 8), plus both global rows, their neighbours and six
# middle blocks drawn per pair on every other pair.
FULL_PAIRS = {4: (0, 9), 5: (0, 15)}


@pytest.mark.parametrize("wid,seed", [(1, None), (2, None), (3, None), (3, 1), (4, None), (5, None)])
def test_workload_parity(wid, seed):
    w = workloads.WORKLOADS[wid]
    plan_seed = w.plan_seed if seed is None else seed
    announce(f"workload {wid} {w.name} plan seed {plan_seed}")
    inp = workloads.make_inputs(wid)
    cplan, oplan = plans(w.H, w.nb, w.r, plan_seed)
    got, st = run_gpu(inp, w.block, w.r, w.dtype, cplan, use_mask=w.masked)
    assert st == bbsa.BBSA_OK
    # Every output row was written (the buffer started as NaN).
    assert np.isfinite(got).all(), "non-finite output: some row was not written"
    full = FULL_PAIRS.get(wid)
    jobs = []
    for b in range(w.B):
        for h in range(w.H):
            bh = b * w.H + h
            qbs = None if full is None or bh in full else varied_blocks(w.nb, bh)
            jobs.append((b, h, qbs))
    wants = oracle_slices(inp, oplan, w.block, jobs)
    g_all, w_all, g_valid, w_valid = [], [], [], []
    for (b, h, qbs), want in zip(jobs, wants):
        blocks = range(w.nb) if qbs is None else qbs
        rows = np.concatenate([np.arange(i * w.block, (i + 1) * w.block) for i in blocks])
        g = got[b, h, rows]
        g_all.append(g)
        w_all.append(want)
        keep = valid_query_rows(inp["mask"], b, rows)
        g_valid.append(g[keep])
        w_valid.append(want[keep])
    g_all, w_all = np.concatenate(g_all), np.concatenate(w_all)
    assert_close(g_all, w_all, w.dtype, f"{w.name} seed{plan_seed} all rows")
    g_valid, w_valid = np.concatenate(g_valid), np.concatenate(w_valid)
    assert_close(g_valid, w_valid, w.dtype, f"{w.name} seed{plan_seed} valid rows")
