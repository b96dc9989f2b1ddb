"""Pins of the oracle's block-constant closed form (CPU only), which checks
the HIP path at lengths whose dense oracle does not fit in memory.

* ``attended_blocks`` against the rows of ``block_mask`` (itself pinned by
  scalar brute force and the closed-form attended-key counts) for planner
  plans, with and without random blocks;
* ``forward_block_constant`` against ``forward`` on the same inputs
  expanded to every token (padding at the tail, inside a block, fractional
  mask values, no mask, another query vector, block 64 and 128);
* a case it must reduce to by hand: equal block scores and no mask give
  every attended block the same weight, so the output is the plain mean of
  the attended blocks' value vectors.

Also the invariants of ``workloads.block_constant_case``'s plan.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_bbsa_amd import workloads


@pytest.mark.parametrize("nb,r,seed", [(8, 3, 1), (16, 3, 2), (24, 5, 3), (40, 2, 4)])
def test_attended_blocks_are_the_block_mask_rows(nb, r, seed):
    plan = oracle.plan_rand_attn(1, nb, r, seed)[0]
    M = oracle.block_mask(nb, plan)
    M0 = oracle.block_mask(nb, None)
    for i in range(nb):
        assert np.array_equal(oracle.attended_blocks(nb, i, plan), np.flatnonzero(M[i]))
        assert np.array_equal(oracle.attended_blocks(nb, i, None), np.flatnonzero(M0[i]))


def _expand(case, block, query=None):
    kb, vb = case["k_blocks"], case["v_blocks"]
    nb, d = kb.shape
    L = nb * block
    qv = np.zeros(d, dtype=np.float32)
    if query is None:
        qv[0] = 1.0
    else:
        qv[:] = query
    q = np.broadcast_to(qv, (1, 1, L, d)).copy()
    k = np.repeat(kb, block, axis=0)[None, None]
    v = np.repeat(vb, block, axis=0)[None, None]
    return q, k, v


@pytest.mark.parametrize("L,block,r,valid,mask_kind,use_query", [
    (1536, 64, 3, 1400, "tail", False),        # padding inside block 21, blocks 22-23 padded
    (2048, 64, 3, 2048, "none", False),
    (2048, 128, 2, 1000, "tail", False),
    (1280, 64, 1, 1280, "fractional", False),
    (1536, 64, 3, 1300, "tail", True),          # a general query vector
])
def test_block_constant_matches_forward(L, block, r, valid, mask_kind, use_query):
    case = workloads.block_constant_case(L, 64, block, r, seed=7 + L + block, valid=valid)
    nb = L // block
    plan = case["plan"]
    assert oracle.check_rand_attn(plan, nb, r) == []
    mask = case["mask"]
    if mask_kind == "none":
        mask = None
    elif mask_kind == "fractional":
        rng = np.random.Generator(np.random.PCG64(5))
        mask = rng.uniform(0.0, 1.0, size=(1, L)).astype(np.float32)
        mask[:, : L // 2] = 1.0
    query = None
    if use_query:
        query = np.random.Generator(np.random.PCG64(6)).standard_normal(64).astype(np.float32) * 0.3
    q, k, v = _expand(case, block, query)
    assert not oracle.uses_full_fallback(L, block, r)
    want = oracle.forward(q, k, v, mask, plan, block)[0, 0]
    qbs = list(range(nb))
    got = oracle.forward_block_constant(case["k_blocks"], case["v_blocks"], None if mask is None else mask[0],
                                        plan[0], block, qbs, query=query)
    for n, i in enumerate(qbs):
        rows = want[i * block:(i + 1) * block]
        assert np.abs(rows - got[n][None, :]).max() < 1e-12


def test_equal_scores_give_the_mean_of_the_attended_values():
    L, block, r = 1536, 64, 3
    case = workloads.block_constant_case(L, 64, block, r, seed=11, valid=L)
    nb = L // block
    kb = case["k_blocks"].copy()
    kb[:, 0] = 0.5                     # every key scores 0.5 against e_0
    plan = case["plan"][0]
    got = oracle.forward_block_constant(kb, case["v_blocks"], None, plan, block, range(nb))
    for i in range(nb):
        if i in (0, nb - 1):
            seen = list(range(nb))
        else:
            seen = sorted({0, nb - 1, i - 1, i, i + 1, *(int(x) for x in plan[i - 1])})
        want = case["v_blocks"][seen].astype(np.float64).mean(axis=0)
        assert np.abs(got[i] - want).max() < 1e-12


def test_block_constant_case_plan_is_valid_at_scale():
    # 2048 blocks: the redraws leave r distinct middle blocks outside every
    # row's window; inputs are bf16-exact and the mask has the valid length.
    L, block, r = 2048 * 64, 64, 3
    case = workloads.block_constant_case(L, 64, block, r, seed=3, valid=L - 1000)
    assert case["plan"].shape == (1, 2046, 3) and case["plan"].dtype == np.int32
    assert oracle.check_rand_attn(case["plan"], 2048, r) == []
    assert np.array_equal(workloads.round_to_bf16(case["k_blocks"]), case["k_blocks"])
    assert case["mask"].sum() == L - 1000 and case["mask"][0, L - 1001] == 1 and case["mask"][0, L - 1000] == 0
