"""Pins of the attention oracle (CPU only).

The oracle (masked dense attention under the BigBird block mask) is pinned
against things other than itself:

1. scalar brute force on tiny inputs, with the pattern evaluated per token
   pair from the block indices of the two tokens;
2. torch's scaled_dot_product_attention in float64 with an explicit mask;
3. invariants of the softmax (row sums, exact zeros outside the pattern);
4. closed-form attended-key counts per query block ("BigBirdPegasus…",
   section "三类注意力组合全局 局部 随机": 2 global + 3 window + r random);
5. special cases that reduce to textbook full attention (global rows, the
   short-sequence fallback, full coverage);
6. closed forms: constant V, Q = 0 (plain or padded means), key shifts,
   a constant bias on every key;
7. batch independence.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.planner import plan_rand_attn


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _brute(q, k, v, mask, ra, block, full):
    """Per-element brute force in Python floats."""
    B, H, L, d = q.shape
    nb = L // block
    out = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                i = t // block
                scores = []
                for u in range(L):
                    j = u // block
                    if full:
                        seen = True
                    else:
                        seen = (i == 0 or i == nb - 1 or j == 0 or j == nb - 1
                                or abs(i - j) <= 1
                                or (1 <= i <= nb - 2 and j in [int(x) for x in ra[h][i - 1]]))
                    if not seen:
                        continue
                    s = 0.0
                    for e in range(d):
                        s += float(q[b, h, t, e]) * float(k[b, h, u, e])
                    s += -10000.0 * (1.0 - float(mask[b, u]))
                    scores.append((u, s))
                mx = max(s for _, s in scores)
                den = 0.0
                acc = [0.0] * d
                for u, s in scores:
                    w = math.exp(s - mx)
                    den += w
                    for e in range(d):
                        acc[e] += w * float(v[b, h, u, e])
                out[b, h, t] = [a / den for a in acc]
    return out


BRUTE_CASES = [
    # B, H, block, nb, d, r
    (1, 1, 1, 6, 1, 1),
    (2, 2, 2, 8, 3, 1),
    (1, 2, 4, 9, 8, 2),
    (2, 1, 2, 14, 3, 2),
    (1, 1, 4, 7, 3, 2),     # nb = 5 + r: smallest sparse case
    (2, 2, 1, 12, 8, 1),
]


@pytest.mark.parametrize("B,H,block,nb,d,r", BRUTE_CASES)
@pytest.mark.parametrize("padded", [False, True])
def test_matches_scalar_brute_force(B, H, block, nb, d, r, padded):
    rng = np.random.default_rng(B * 1000 + H * 100 + nb * 10 + d + r)
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    mask = np.ones((B, L))
    if padded:
        mask[0, L - block - 1:] = 0.0          # partial block + last block padded
        if B > 1:
            mask[1, :] = 0.0                   # a fully padded sequence
    ra = plan_rand_attn(H, nb, r, seed=nb + r)
    got = A.forward(q, k, v, mask, ra, block, allow_fallback=False)
    want = _brute(q, k, v, mask, ra, block, full=False)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,H,block,nb,d,r", [(1, 2, 2, 6, 3, 1), (2, 1, 4, 9, 3, 2)])
def test_fallback_matches_brute_force_full(B, H, block, nb, d, r):
    # L <= (5 + 2r) * block: full attention is computed.
    rng = np.random.default_rng(7)
    L = nb * block
    assert A.uses_full_fallback(L, block, r)
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    mask = np.ones((B, L)); mask[-1, -3:] = 0
    ra = plan_rand_attn(H, nb, r, seed=1) if nb >= 5 + r else np.zeros((H, nb - 2, r), np.int32)
    got = A.forward(q, k, v, mask, ra, block)
    want = _brute(q, k, v, mask, ra, block, full=True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_fallback_threshold_reading():
    # 704 = (5 + 2*3) * 64 at the default block 64, r 3.
    assert A.uses_full_fallback(704, 64, 3)
    assert not A.uses_full_fallback(768, 64, 3)
    assert not A.uses_full_fallback(1024, 64, 3)
    assert A.uses_full_fallback(9 * 128, 128, 2) and not A.uses_full_fallback(10 * 128, 128, 2)


@pytest.mark.parametrize("block,nb,r", [(4, 12, 3), (8, 9, 2), (2, 20, 1)])
def test_matches_torch_sdpa(block, nb, r):
    rng = np.random.default_rng(11)
    B, H, d = 2, 3, 16
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng, 0.7) for _ in range(3))
    mask = (rng.random((B, L)) > 0.2).astype(np.float64)
    ra = plan_rand_attn(H, nb, r, seed=3)
    got = A.forward(q, k, v, mask, ra, block, allow_fallback=False)
    want = np.empty_like(got)
    for h in range(H):
        seen = A.token_mask(A.block_mask(nb, ra[h]), block)
        for b in range(B):
            bias = torch.tensor(-10000.0 * (1.0 - mask[b]), dtype=torch.float64)[None, :].repeat(L, 1)
            bias[~torch.from_numpy(seen)] = -math.inf
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h])[None], torch.from_numpy(k[b, h])[None],
                torch.from_numpy(v[b, h])[None], attn_mask=bias[None], scale=1.0)
            want[b, h] = o[0].numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_probability_invariants():
    rng = np.random.default_rng(5)
    B, H, block, nb, d, r = 2, 2, 4, 12, 8, 2
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng, 2.0) for _ in range(3))
    mask = np.ones((B, L)); mask[1, 30:] = 0
    ra = plan_rand_attn(H, nb, r, seed=9)
    out, P = A.forward(q, k, v, mask, ra, block, return_probs=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (P >= 0).all()
    for h in range(H):
        outside = ~A.token_mask(A.block_mask(nb, ra[h]), block)
        assert (P[:, h][:, outside] == 0).all()
    np.testing.assert_allclose(np.einsum("bhij,bhjd->bhid", P, v), out, atol=1e-12)


@pytest.mark.parametrize("nb,r", [(16, 3), (64, 3), (256, 2), (8, 3), (9, 1)])
def test_attended_key_counts_closed_form(nb, r):
    block = 64
    ra = plan_rand_attn(3, nb, r, seed=0)
    L = nb * block
    for h in range(3):
        cnt = A.attended_key_counts(nb, block, ra[h])
        assert cnt[0] == L and cnt[-1] == L
        assert cnt[1] == (4 + r) * block and cnt[-2] == (4 + r) * block
        assert (cnt[2:-2] == (5 + r) * block).all()


def test_global_rows_equal_full_attention():
    rng = np.random.default_rng(3)
    B, H, block, nb, d, r = 2, 2, 8, 16, 16, 3
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    mask = np.ones((B, L)); mask[0, 100:] = 0
    ra = plan_rand_attn(H, nb, r, seed=2)
    out = A.forward(q, k, v, mask, ra, block)
    full = A.full_attention(q, k, v, mask)
    np.testing.assert_allclose(out[:, :, :block], full[:, :, :block], atol=1e-12)
    np.testing.assert_allclose(out[:, :, -block:], full[:, :, -block:], atol=1e-12)
    # a middle row is not full attention
    assert np.abs(out[:, :, 5 * block] - full[:, :, 5 * block]).max() > 1e-3


def test_full_attention_matches_sdpa():
    rng = np.random.default_rng(4)
    q, k, v = (_rand((1, 2, 40, 8), rng) for _ in range(3))
    mask = np.ones((1, 40)); mask[0, 33:] = 0
    got = A.full_attention(q, k, v, mask)
    bias = torch.tensor(-10000.0 * (1 - mask[0]))[None, :].repeat(40, 1)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0]), torch.from_numpy(k[0]), torch.from_numpy(v[0]),
        attn_mask=bias, scale=1.0).numpy()
    np.testing.assert_allclose(got[0], want, atol=1e-12)


@pytest.mark.parametrize("nb", [3, 4])
def test_no_random_blocks_small_nb_is_full(nb):
    rng = np.random.default_rng(nb)
    block = 4
    q, k, v = (_rand((1, 2, nb * block, 5), rng) for _ in range(3))
    mask = np.ones((1, nb * block))
    got = A.forward(q, k, v, mask, None, block, allow_fallback=False)
    np.testing.assert_allclose(got, A.full_attention(q, k, v, mask), atol=1e-12)


def test_minimum_nb_middle_rows_are_full():
    # nb = 5 + r: middle rows 2..nb-3 see every block.
    rng = np.random.default_rng(8)
    r, block = 2, 4
    nb = 5 + r
    q, k, v = (_rand((1, 2, nb * block, 6), rng) for _ in range(3))
    mask = np.ones((1, nb * block))
    ra = plan_rand_attn(2, nb, r, seed=4)
    got = A.forward(q, k, v, mask, ra, block, allow_fallback=False)
    full = A.full_attention(q, k, v, mask)
    np.testing.assert_allclose(got[:, :, 2 * block:(nb - 2) * block],
                               full[:, :, 2 * block:(nb - 2) * block], atol=1e-12)
    assert np.abs(got[:, :, block:2 * block] - full[:, :, block:2 * block]).max() > 1e-6


def test_constant_v_gives_constant_output():
    rng = np.random.default_rng(12)
    B, H, block, nb, d, r = 1, 2, 4, 12, 6, 2
    L = nb * block
    q, k = _rand((B, H, L, d), rng, 3.0), _rand((B, H, L, d), rng, 3.0)
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (B, H, L, d)).copy()
    mask = np.ones((B, L)); mask[0, 40:] = 0
    out = A.forward(q, k, v, mask, plan_rand_attn(H, nb, r, 1), block)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), atol=1e-12)


def test_zero_q_gives_mean_over_attended_blocks():
    rng = np.random.default_rng(13)
    B, H, block, nb, d, r = 1, 2, 4, 12, 5, 3
    L = nb * block
    q = np.zeros((B, H, L, d))
    k, v = _rand((B, H, L, d), rng), _rand((B, H, L, d), rng)
    ra = plan_rand_attn(H, nb, r, 6)
    out = A.forward(q, k, v, None, ra, block)
    for h in range(H):
        for i in range(nb):
            if i in (0, nb - 1):
                blocks = set(range(nb))
            else:
                blocks = {0, nb - 1, i - 1, i, i + 1} | set(int(x) for x in ra[h, i - 1])
            keys = [u for j in sorted(blocks) for u in range(j * block, (j + 1) * block)]
            want = v[0, h, keys].mean(axis=0)
            np.testing.assert_allclose(out[0, h, i * block:(i + 1) * block],
                                       np.broadcast_to(want, (block, d)), atol=1e-12)


def test_zero_q_padded_gives_mean_over_valid_keys():
    # -10000 additive: exp(-10000) is exactly 0 in float64 next to a valid key.
    rng = np.random.default_rng(14)
    B, H, block, nb, d, r = 1, 1, 4, 12, 3, 2
    L = nb * block
    valid = 30
    q = np.zeros((B, H, L, d))
    k, v = _rand((B, H, L, d), rng), _rand((B, H, L, d), rng)
    mask = np.zeros((B, L)); mask[0, :valid] = 1
    out = A.forward(q, k, v, mask, plan_rand_attn(H, nb, r, 2), block)
    # global query rows see every key: the mean over the valid ones
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, :valid].mean(0), atol=1e-12)
    np.testing.assert_allclose(out[0, 0, -1], v[0, 0, :valid].mean(0), atol=1e-12)


def test_fractional_mask_is_additive_bias():
    # mask 1 - 1e-4 on one key adds exactly -1 to that key's score.
    rng = np.random.default_rng(15)
    B, H, block, nb, d, r = 1, 1, 2, 10, 4, 1
    L = nb * block
    q = np.zeros((B, H, L, d))
    k, v = _rand((B, H, L, d), rng), _rand((B, H, L, d), rng)
    mask = np.ones((B, L)); mask[0, 3] = 1 - 1e-4
    out = A.forward(q, k, v, mask, plan_rand_attn(H, nb, r, 2), block)
    w = np.ones(L); w[3] = math.exp(-10000.0 * 1e-4)
    want = (w[:, None] * v[0, 0]).sum(0) / w.sum()
    np.testing.assert_allclose(out[0, 0, 0], want, atol=1e-12)


def test_fully_padded_sequence_equals_unpadded():
    # A constant -10000 on every key cancels in the softmax.
    rng = np.random.default_rng(16)
    B, H, block, nb, d, r = 1, 2, 4, 12, 6, 2
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    ra = plan_rand_attn(H, nb, r, 5)
    a = A.forward(q, k, v, np.zeros((B, L)), ra, block)
    b = A.forward(q, k, v, np.ones((B, L)), ra, block)
    np.testing.assert_allclose(a, b, atol=1e-10)


def test_key_shift_invariance():
    rng = np.random.default_rng(17)
    B, H, block, nb, d, r = 2, 2, 4, 12, 6, 2
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    w = rng.standard_normal(d)
    mask = np.ones((B, L)); mask[1, 37:] = 0
    ra = plan_rand_attn(H, nb, r, 5)
    a = A.forward(q, k, v, mask, ra, block)
    b = A.forward(q, k + w, v, mask, ra, block)
    np.testing.assert_allclose(a, b, atol=1e-10)


def test_batch_independence():
    rng = np.random.default_rng(18)
    B, H, block, nb, d, r = 3, 2, 4, 12, 6, 2
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    mask = np.ones((B, L)); mask[1, 20:] = 0
    ra = plan_rand_attn(H, nb, r, 5)
    whole = A.forward(q, k, v, mask, ra, block)
    for b in range(B):
        alone = A.forward(q[b:b + 1], k[b:b + 1], v[b:b + 1], mask[b:b + 1], ra, block)
        assert np.array_equal(alone[0], whole[b])


def test_query_block_subset_matches_full_run():
    rng = np.random.default_rng(19)
    B, H, block, nb, d, r = 1, 2, 4, 16, 6, 3
    L = nb * block
    q, k, v = (_rand((B, H, L, d), rng) for _ in range(3))
    ra = plan_rand_attn(H, nb, r, 5)
    whole = A.forward(q, k, v, None, ra, block)
    sub = A.forward(q, k, v, None, ra, block, query_blocks=[15, 0, 7])
    assert np.array_equal(sub[:, :, :block], whole[:, :, 15 * block:])
    assert np.array_equal(sub[:, :, block:2 * block], whole[:, :, :block])
    assert np.array_equal(sub[:, :, 2 * block:], whole[:, :, 7 * block:8 * block])


def test_misaligned_length_raises():
    z = np.zeros((1, 1, 65, 4))
    with pytest.raises(ValueError):
        A.forward(z, z, z, None, None, 64)
