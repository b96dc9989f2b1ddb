"""Pins of the oracle's extensions (CPU only): the query x key masking mode,
the row log-sum-exp, and lengths that are not a multiple of the block.

Each is pinned against something other than the oracle itself:

* query x key mode ("models 仓库中的 BigBird…", section "随机块掩码是如何生成的":
  the band mask is the einsum of the from-mask and the to-mask): a scalar
  brute force with the bias -10000 * (1 - m[t] * m[u]) evaluated per token
  pair, and torch's scaled_dot_product_attention in float64 with the full
  [L, L] additive mask; closed forms: a row whose query is valid equals the
  key-side row exactly, a row whose query is padded equals the unmasked row
  (a constant shift);
* log-sum-exp: torch.logsumexp of the explicit dense masked score matrix;
  exp(S - lse) reproduces the probabilities;
* padding to the block ("BigBirdPegasus…", section "序列长度的块对齐要求":
  the encoder pads to a multiple of the block and trims the output): a
  block-aligned length gives exactly ``forward``; a ragged length gives, on
  every row that attends at least one valid key, the brute force that
  ignores the padding positions altogether (their weight exp(-10000 + s) is
  exactly 0 in float64); the padding positions' content does not matter.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.planner import plan_rand_attn


def _sees(i, j, nb, ra_h, full):
    if full:
        return True
    return (i == 0 or i == nb - 1 or j == 0 or j == nb - 1 or abs(i - j) <= 1
            or (1 <= i <= nb - 2 and j in [int(x) for x in ra_h[i - 1]]))


def _brute(q, k, v, mask, ra, block, full, query_key, keys=None):
    """Per-element brute force.  The bias of (t, u) is -10000(1 - m_t m_u)
    with ``query_key``, else -10000(1 - m_u); with ``keys`` only key
    positions below it exist at all.  Returns (out, lse)."""
    B, H, L, d = q.shape
    nb = -(-L // block)
    out = np.zeros((B, H, L, d))
    lse = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                scores = []
                for u in range(L if keys is None else keys):
                    if not _sees(t // block, u // block, nb, None if ra is None else ra[h], full):
                        continue
                    s = sum(float(q[b, h, t, e]) * float(k[b, h, u, e]) for e in range(d))
                    mt = float(mask[b, t]) if query_key else 1.0
                    s += -10000.0 * (1.0 - mt * float(mask[b, u]))
                    scores.append((u, s))
                mx = max(s for _, s in scores)
                den = sum(math.exp(s - mx) for _, s in scores)
                for e in range(d):
                    out[b, h, t, e] = sum(math.exp(s - mx) * float(v[b, h, u, e]) for u, s in scores) / den
                lse[b, h, t] = mx + math.log(den)
    return out, lse


@pytest.mark.parametrize("B,H,block,nb,d,r,seed", [(1, 1, 2, 8, 3, 1, 0), (2, 2, 2, 9, 2, 2, 1),
                                                   (1, 2, 4, 8, 3, 1, 2)])
def test_query_key_mode_brute_force(B, H, block, nb, d, r, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    L = nb * block
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    mask = (rng.random((B, L)) < 0.7).astype(np.float64)
    mask[:, 0] = 1.0
    mask[0, 3] = 0.35                       # one fractional value
    ra = plan_rand_attn(H, nb, r, seed)
    want, want_lse = _brute(q, k, v, mask, ra, block, False, True)
    got, lse = A.forward(q, k, v, mask, ra, block, allow_fallback=False, query_key_mask=True,
                         return_lse=True)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, want_lse, atol=1e-9, rtol=0)


def test_query_key_mode_matches_sdpa_with_outer_product_mask():
    rng = np.random.Generator(np.random.PCG64(7))
    B, H, L, block, r = 2, 2, 1024, 64, 3
    nb = L // block
    q, k, v = (rng.standard_normal((B, H, L, 16)) for _ in range(3))
    mask = np.ones((B, L))
    mask[0, 900:] = 0.0
    mask[1, :100] = 0.0
    ra = plan_rand_attn(H, nb, r, 7)
    got = A.forward(q, k, v, mask, ra, block, query_key_mask=True)
    for h in range(H):
        M = np.kron(A.block_mask(nb, ra[h]).astype(np.int8), np.ones((block, block), np.int8)).astype(bool)
        for b in range(B):
            add = -10000.0 * (1.0 - np.outer(mask[b], mask[b]))
            add[~M] = -np.inf
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h])[None], torch.from_numpy(k[b, h])[None], torch.from_numpy(v[b, h])[None],
                attn_mask=torch.from_numpy(add)[None], scale=1.0)[0].numpy()
            np.testing.assert_allclose(got[b, h], ref, atol=1e-10, rtol=0)


def test_query_key_mode_closed_forms():
    rng = np.random.Generator(np.random.PCG64(8))
    B, H, L, block, r = 2, 2, 1536, 64, 3
    q, k, v = (rng.standard_normal((B, H, L, 8)) for _ in range(3))
    mask = np.ones((B, L))
    mask[0, 1200:] = 0.0
    mask[1, 50:700] = 0.0
    ra = plan_rand_attn(H, L // block, r, 8)
    qk = A.forward(q, k, v, mask, ra, block, query_key_mask=True)
    key = A.forward(q, k, v, mask, ra, block)
    none = A.forward(q, k, v, None, ra, block)
    valid = mask > 0.5
    for b in range(B):
        # Valid query rows: the same bias as the key-side mode, bit for bit.
        assert np.array_equal(qk[b][:, valid[b]], key[b][:, valid[b]])
        # Padded query rows: -10000 on every key, a constant shift (up to the
        # float64 rounding of s - 10000, whose spacing is 1.8e-12).
        np.testing.assert_allclose(qk[b][:, ~valid[b]], none[b][:, ~valid[b]], atol=1e-10, rtol=0)
    # All-ones mask: the two modes agree exactly.
    ones = np.ones((B, L))
    assert np.array_equal(A.forward(q, k, v, ones, ra, block, query_key_mask=True),
                          A.forward(q, k, v, ones, ra, block))


@pytest.mark.parametrize("qk", [False, True])
def test_lse_matches_torch_logsumexp(qk):
    rng = np.random.Generator(np.random.PCG64(9))
    B, H, L, block, r = 2, 2, 1024, 64, 2
    nb = L // block
    q, k, v = (rng.standard_normal((B, H, L, 8)) for _ in range(3))
    mask = np.ones((B, L))
    mask[1, 700:] = 0.0
    ra = plan_rand_attn(H, nb, r, 9)
    out, P, lse = A.forward(q, k, v, mask, ra, block, return_probs=True, return_lse=True, query_key_mask=qk)
    for h in range(H):
        M = np.kron(A.block_mask(nb, ra[h]).astype(np.int8), np.ones((block, block), np.int8)).astype(bool)
        for b in range(B):
            S = q[b, h] @ k[b, h].T
            S = S + (-10000.0 * (1.0 - (np.outer(mask[b], mask[b]) if qk else mask[b][None, :])))
            S[~M] = -np.inf
            ref = torch.logsumexp(torch.from_numpy(S), dim=-1).numpy()
            np.testing.assert_allclose(lse[b, h], ref, atol=1e-9, rtol=0)
            np.testing.assert_allclose(np.exp(S - lse[b, h][:, None]), P[b, h], atol=1e-12, rtol=0)


def test_padded_aligned_length_is_forward():
    rng = np.random.Generator(np.random.PCG64(10))
    q, k, v = (rng.standard_normal((2, 2, 1024, 8)) for _ in range(3))
    mask = np.ones((2, 1024))
    mask[1, 800:] = 0
    ra = plan_rand_attn(2, 16, 3, 10)
    assert np.array_equal(A.forward_padded(q, k, v, mask, ra, 64), A.forward(q, k, v, mask, ra, 64))


@pytest.mark.parametrize("B,H,block,L,d,r,seed,qk", [(1, 1, 2, 15, 3, 1, 0, False), (2, 2, 4, 31, 2, 1, 1, False),
                                                      (1, 2, 2, 19, 3, 2, 2, True)])
def test_padded_ragged_length_brute_force(B, H, block, L, d, r, seed, qk):
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = -(-L // block)
    q, k, v = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    mask = np.ones((B, L))
    mask[-1, L - 3:] = 0.0
    ra = plan_rand_attn(H, nb, r, seed)
    full = A.uses_full_fallback(nb * block, block, r)
    got = A.forward_padded(q, k, v, mask, ra, block, query_key_mask=qk)
    assert got.shape == (B, H, L, d)
    # Brute force over the L real keys only: on every row that sees a key
    # with a bias above the padding's, the padding positions never count.
    # (In query x key mode a padded query row puts every key, the padding
    # included, at the same level; those rows are left out here.)
    want, _ = _brute(q, k, v, mask, ra, block, full, qk, keys=L)
    rows = mask > 0.5 if qk else np.ones((B, L), dtype=bool)
    for b in range(B):
        np.testing.assert_allclose(got[b][:, rows[b]], want[b][:, rows[b]], atol=1e-12, rtol=0)


def test_padded_content_of_padding_does_not_matter():
    # Padding positions are zero vectors in the oracle; any other content
    # gives the same result on every row with at least one valid key, since
    # a padded key's weight exp(s - 10000 - max) is exactly 0 in float64.
    rng = np.random.Generator(np.random.PCG64(11))
    B, H, L, block = 2, 2, 1000, 64
    Lp = 1024
    q, k, v = (rng.standard_normal((B, H, L, 8)) for _ in range(3))
    mask = np.ones((B, L))
    mask[1, 900:] = 0.0
    ra = plan_rand_attn(H, Lp // block, 3, 11)
    got = A.forward_padded(q, k, v, mask, ra, block)
    junk = [np.concatenate([x, rng.standard_normal((B, H, Lp - L, 8)) * 3], axis=2) for x in (q, k, v)]
    mp = np.concatenate([mask, np.zeros((B, Lp - L))], axis=1)
    alt = A.forward(*junk, mp, ra, block)[:, :, :L]
    np.testing.assert_allclose(got, alt, atol=1e-12, rtol=0)
