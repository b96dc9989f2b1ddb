"""The attention kernel's work decomposition, checked on the CPU.

``bbsa_work_map`` runs on the host the item mapping and key-list construction
the kernels run (the same source, bbsa_schedule.h).  For every launch shape
below these tests check that the grid covers every (batch, head, query tile)
exactly as the pattern requires: the key blocks a query tile walks, summed
over its chunks or key parts, are exactly the blocks of its row of the
oracle's block mask, each once ("models 仓库中的 BigBird…", section
"BigBird：从二次方注意力到线性稀疏注意力"; full rows on the fallback,
"BigBirdPegasus…", section "序列过短时的自动回退"); that every wavefront runs
at most one item; that the full-row chunks sharing a workgroup are the
chunks of one row tile (they merge through LDS); and that with eight or more
(batch, head) pairs every item of a pair is on the XCD lane wg % 8 = pair % 8.
"""
from collections import Counter, defaultdict

import numpy as np
import pytest

import oracle

bbsa = pytest.importorskip("block_sparse_long_bbsa_amd.bbsa")


@pytest.fixture(scope="module")
def lib():
    try:
        return bbsa.lib()
    except RuntimeError as e:
        pytest.skip(str(e))


SHAPES = [
    # B, H, L, block, r, dtype
    (1, 2, 1024, 64, 3, bbsa.BBSA_F32),      # fp32 workload: small call, chunked finer
    (4, 12, 4096, 64, 3, bbsa.BBSA_BF16),    # BigBird-base workload
    (8, 16, 4096, 64, 3, bbsa.BBSA_BF16),    # Pegasus-large encoder workload
    (2, 12, 16384, 64, 3, bbsa.BBSA_BF16),   # long context: rows of more than four chunks
    (1, 16, 32768, 128, 2, bbsa.BBSA_BF16),  # block 128: two query tiles per block
    (3, 3, 1024, 64, 2, bbsa.BBSA_BF16),     # 9 pairs: XCD lanes with one and two pairs
    (1, 11, 896, 64, 2, bbsa.BBSA_BF16),     # 11 pairs, odd middle-unit count per pair
    (5, 3, 1280, 128, 2, bbsa.BBSA_BF16),    # 15 pairs, block 128
    (1, 1, 5120, 128, 3, bbsa.BBSA_BF16),    # one pair: no XCD remap
    (1, 2, 768, 64, 3, bbsa.BBSA_BF16),      # shortest sparse length at r = 3
    (4, 8, 2048, 64, 3, bbsa.BBSA_F32),      # fp32 call large enough for whole middle rows
    (1, 2, 704, 64, 3, bbsa.BBSA_BF16),      # fallback: full attention
    (1, 1, 2880, 64, 20, bbsa.BBSA_BF16),    # fallback, rows of 45 blocks
    (1, 2, 128, 64, 1, bbsa.BBSA_BF16),      # fallback, rows shorter than four chunks
    (1, 2, 448, 64, 1, bbsa.BBSA_F32),       # fallback, fp32
    (1, 2, 8192, 128, 20, bbsa.BBSA_BF16),   # many random blocks
]


def _check(B, H, L, block, r, dtype, flags=0):
    nb = -(-L // block)
    full = L <= (5 + 2 * r) * block
    plan = None if full else oracle.plan_rand_attn(H, nb, r, 3)
    st, grid, rec = bbsa.bbsa_work_map(B, H, L, 64, block, r, dtype, plan, flags=flags)
    assert st == (bbsa.BBSA_OK_FULL_FALLBACK if full else bbsa.BBSA_OK)
    qtiles = block // 64
    waves = 4 if dtype == bbsa.BBSA_BF16 else 1

    # Every (workgroup, wavefront, unit) at most once, inside the grid.
    assert (rec[:, 0] >= 0).all() and (rec[:, 0] < grid).all()
    assert (rec[:, 1] >= 0).all() and (rec[:, 1] < waves).all()
    keys = Counter(map(tuple, rec[:, :3].tolist()))
    assert max(keys.values()) == 1

    # Key blocks walked per (pair, query block, query tile), over all its items.
    walked = defaultdict(Counter)
    for rr in rec:
        bh, qb, qt = int(rr[3]), int(rr[4]), int(rr[5])
        assert 0 <= bh < B * H and 0 <= qb < nb and 0 <= qt < qtiles
        blocks = rr[16 + rr[8]:16 + rr[9]]
        assert (blocks >= 0).all() and (blocks < nb).all()
        walked[(bh, qb, qt)].update(blocks.tolist())
    assert len(walked) == B * H * nb * qtiles, "some query tile is never computed"
    for h in range(H):
        M = np.ones((nb, nb), dtype=bool) if full else oracle.block_mask(nb, plan[h])
        for b in range(B):
            for qb in range(nb):
                want = Counter(np.flatnonzero(M[qb]).tolist())
                for qt in range(qtiles):
                    assert walked[(b * H + h, qb, qt)] == want, (b, h, qb, qt)

    # Full-row chunks that share a bf16 workgroup are the four chunks of one
    # row tile, and such a workgroup holds nothing else.
    if dtype == bbsa.BBSA_BF16:
        by_wg = defaultdict(list)
        for rr in rec:
            by_wg[int(rr[0])].append(rr)
        for wg, rows in by_wg.items():
            fulls = [rr for rr in rows if rr[6] >= 0]
            if fulls:
                assert len(fulls) == len(rows) == 4, wg
                assert len({(int(x[3]), int(x[6]), int(x[5])) for x in fulls}) == 1, wg
                assert sorted(int(x[7]) % 4 for x in fulls) == [0, 1, 2, 3], wg
                assert sorted(int(x[1]) for x in fulls) == [0, 1, 2, 3], wg

    # XCD lanes: with eight or more pairs, pair p runs only on lane p % 8.
    if B * H >= 8:
        assert ((rec[:, 0] % 8) == (rec[:, 3] % 8)).all()


@pytest.mark.parametrize("B,H,L,block,r,dtype", SHAPES)
def test_work_map_covers_the_pattern_once(lib, B, H, L, block, r, dtype):
    _check(B, H, L, block, r, dtype)


@pytest.mark.parametrize("B,H,L,block,r,dtype", [
    (4, 12, 4000, 64, 3, bbsa.BBSA_BF16),    # ragged: 63 blocks, the last one partial
    (1, 3, 5000, 128, 2, bbsa.BBSA_BF16),
    (2, 2, 1000, 64, 3, bbsa.BBSA_F32),
    (1, 2, 700, 64, 3, bbsa.BBSA_BF16),      # ragged and short: fallback
    (1, 1, 16385, 64, 3, bbsa.BBSA_BF16),    # one token past a block boundary
])
def test_work_map_ragged_lengths(lib, B, H, L, block, r, dtype):
    # Lengths that are not a multiple of the block (padded to the block):
    # the pattern of ceil(L / block) blocks is covered exactly once.
    _check(B, H, L, block, r, dtype, flags=bbsa.BBSA_FLAG_PAD_TO_BLOCK)
    # Without the flag such a length is refused.
    assert bbsa.bbsa_work_map(B, H, L, 64, block, r, dtype, None)[0] == bbsa.BBSA_ERR_SHAPE


def test_work_map_reports_errors_like_forward(lib):
    assert bbsa.bbsa_work_map(1, 1, 1000, 64, 64, 3, bbsa.BBSA_BF16)[0] == bbsa.BBSA_ERR_SHAPE
    assert bbsa.bbsa_work_map(1, 1, 1024, 128, 64, 3, bbsa.BBSA_BF16)[0] == bbsa.BBSA_ERR_UNSUPPORTED
    assert bbsa.bbsa_work_map(1, 1, 1024, 64, 64, 3, bbsa.BBSA_BF16, None)[0] == bbsa.BBSA_ERR_ARG


@pytest.mark.parametrize("seed", range(12))
def test_work_map_random_shapes(lib, seed):
    rng = np.random.Generator(np.random.PCG64(500 + seed))
    block = int(rng.choice([64, 128]))
    r = int(rng.integers(1, 8))
    nb = int(rng.integers(2, 48))
    B, H = int(rng.integers(1, 5)), int(rng.integers(1, 7))
    dtype = int(rng.choice([bbsa.BBSA_BF16, bbsa.BBSA_F32]))
    L = nb * block
    if L > (5 + 2 * r) * block and nb < 5 + r:
        return
    _check(B, H, L, block, r, dtype)


@pytest.mark.parametrize("B,H,L,block,r", [
    (1, 1, 1024, 64, 3), (4, 12, 4096, 64, 3), (8, 16, 4096, 64, 3), (2, 12, 16384, 64, 3),
    (2, 16, 16384, 64, 3), (4, 16, 16384, 64, 3), (1, 16, 32768, 128, 2), (8, 16, 8192, 64, 3),
    (1, 1, 1 << 20, 64, 3), (3, 5, 65536, 128, 7), (64, 16, 4096, 64, 3),
])
def test_bf16_full_row_chunk_length(lib, B, H, L, block, r):
    # bf16 full rows are cut into chunks of 1024, 2048 or 4096 keys, as many
    # as a multiple of four (four chunks share a workgroup; a row of at most
    # four chunks is cut into four shorter ones).  A chunk longer than 1024
    # keys fits in one wavefront slot's share of the launch's 32-key steps
    # (2048 slots); a row of more than four chunks uses the longest length
    # that fits.
    nb = L // block
    plan = bbsa.bbsa_plan_rand_attn(H, nb, r, 3)
    st, grid, rec = bbsa.bbsa_work_map(B, H, L, 64, block, r, bbsa.BBSA_BF16, plan)
    assert st == bbsa.BBSA_OK
    steps = sum(int(x[9] - x[8]) * int(x[10]) for x in rec)
    share = steps / 2048
    glob = rec[rec[:, 6] >= 0]
    chunks = int(glob[0, 11])
    assert (glob[:, 11] == chunks).all() and chunks % 4 == 0
    keys = max(int(x[9] - x[8]) for x in glob) * block
    if keys > 1024:
        assert keys // 32 <= share
    if chunks > 4:
        assert keys in (1024, 2048, 4096)
        assert chunks == 4 * -(-nb // (4 * (keys // block)))
        if keys < 4096:
            assert 2 * keys // 32 > share
    else:
        assert keys == -(-nb // 4) * block
