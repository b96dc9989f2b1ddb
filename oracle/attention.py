"""Oracle for the BigBird block-sparse attention forward (numpy, float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The block-sparse computation reaches, up to rounding order, the result of
plain masked dense attention under a block mask, so the oracle is that
definition written out: materialise which key blocks each query block sees,
compute every score densely, exclude the blocks outside the pattern exactly,
add the padding bias, take the row softmax and multiply by V.

Sources (by page title and section):

* "models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
  section "BigBird：从二次方注意力到线性稀疏注意力": the pattern has three
  parts -- the first and the last block attend to (and are attended by) the
  whole sequence, each middle block sees a 3-block window around itself, and
  each middle block sees ``num_rand_blocks`` random blocks; masked positions
  get an additive -10000 before the softmax.
* same page, section "随机块掩码是如何生成的": the random blocks come from the
  per-head adjacency ``rand_attn`` and never overlap the window; the
  ``[B, L]`` input mask is viewed per block (``[B, L//block, block]``).
* "BigBirdPegasus 长序列条件生成模型详解从稀疏注意力原理到 Transformers 实战",
  section "三类注意力组合全局 局部 随机": 2 global blocks, 3 window blocks,
  ``num_random_blocks`` random blocks per query block, handled as five parts
  q[0], q[1], q[2:-2], q[-2], q[-1]; section "序列长度的块对齐要求": the length
  must be a multiple of the block size (ValueError otherwise); section
  "序列过短时的自动回退": when the length does not exceed
  ``(5 + 2*num_random_blocks) * block_size`` the layer falls back to full
  attention.

Readings where the pages are silent:

* no internal softmax scale -- the caller folds 1/sqrt(d) into Q;
* padding is key-side only: bias ``-10000 * (1 - mask[key])`` on every
  score of that key; padded query rows are computed with the same formula;
* blocks outside the pattern get probability exactly 0 (excluded), while
  padded keys inside the pattern get the additive -10000, as written;
* rows 1 and nb-2 see a set of blocks: the window already holds the global
  block, which is counted once (4 + r distinct blocks);
* the fallback threshold reads ``L <= (5 + 2r) * block`` (the "+" is lost in
  the page's text; 704 = (5 + 2*3) * 64 confirms it).

Parity status: pinned (tests/test_oracle_attention.py) against scalar brute
force on tiny inputs, against torch's scaled_dot_product_attention in
float64, against closed forms (constant V, Q = 0, key shift, attended-key
counts) and against invariants (row sums, exact zeros, batch independence).
"""
from __future__ import annotations

import numpy as np

PAD_BIAS = -10000.0


def uses_full_fallback(L: int, block: int, r: int) -> bool:
    """True when the sequence is too short for the sparse pattern and full
    attention is computed instead ("BigBirdPegasus…", section
    "序列过短时的自动回退")."""
    return L <= (5 + 2 * r) * block


def block_mask(nb: int, rand_attn_h) -> np.ndarray:
    """Boolean ``[nb, nb]`` block mask of one head: entry (i, j) is True when
    query block i sees key block j.  ``rand_attn_h`` is ``[nb-2, r]`` (row
    i-1 for middle block i) or None for no random blocks."""
    M = np.zeros((nb, nb), dtype=bool)
    M[0, :] = True          # first block is global: sees everything
    M[nb - 1, :] = True     # last block is global
    M[:, 0] = True          # everyone sees the first block
    M[:, nb - 1] = True     # everyone sees the last block
    for i in range(nb):
        for j in range(max(0, i - 1), min(nb, i + 2)):
            M[i, j] = True  # 3-block sliding window
    if rand_attn_h is not None:
        ra = np.asarray(rand_attn_h)
        for i in range(1, nb - 1):
            for j in ra[i - 1]:
                M[i, int(j)] = True
    return M


def token_mask(M: np.ndarray, block: int) -> np.ndarray:
    """Expand a block mask to the token level, ``[L, L]``."""
    return np.kron(M.astype(np.int8), np.ones((block, block), dtype=np.int8)).astype(bool)


def key_bias(mask, B: int, L: int) -> np.ndarray:
    """Additive key bias ``-10000 * (1 - mask)`` as float64 ``[B, L]``;
    ``mask`` None means every key is valid."""
    if mask is None:
        return np.zeros((B, L), dtype=np.float64)
    m = np.asarray(mask, dtype=np.float64).reshape(B, L)
    return PAD_BIAS * (1.0 - m)


def attended_key_counts(nb: int, block: int, rand_attn_h) -> np.ndarray:
    """Number of keys each query block attends to, from the block mask."""
    return block_mask(nb, rand_attn_h).sum(axis=1) * block


def _softmax_rows(S: np.ndarray) -> np.ndarray:
    mx = S.max(axis=-1, keepdims=True)
    E = np.exp(S - mx)
    return E / E.sum(axis=-1, keepdims=True)


def forward(q, k, v, mask, rand_attn, block: int, query_blocks=None,
            allow_fallback: bool = True, return_probs: bool = False):
    """Masked dense attention under the BigBird block mask, in float64.

    q, k, v: ``[B, H, L, d]`` (any real dtype; upcast exactly to float64).
    mask: ``[B, L]`` values in [0, 1] (1 = valid key) or None.
    rand_attn: ``[H, nb-2, r]`` integer plan, or None (no random blocks).
    query_blocks: iterable of query block indices to compute (default: all);
    the result then holds only those blocks' rows, in the order given.
    allow_fallback: apply the short-sequence fallback to full attention.

    Returns ``out`` (float64 ``[B, H, rows, d]``), or ``(out, P)`` with the
    probabilities ``[B, H, rows, L]`` when ``return_probs`` is set.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    if L % block != 0:
        raise ValueError(f"sequence length {L} is not a multiple of block size {block}")
    nb = L // block
    r = 0 if rand_attn is None else int(np.asarray(rand_attn).shape[2])
    full = allow_fallback and uses_full_fallback(L, block, r)
    bias = key_bias(mask, B, L)
    qbs = list(range(nb)) if query_blocks is None else [int(i) for i in query_blocks]
    rows = len(qbs) * block
    out = np.empty((B, H, rows, d), dtype=np.float64)
    probs = np.empty((B, H, rows, L), dtype=np.float64) if return_probs else None
    for h in range(H):
        if full:
            M = np.ones((nb, nb), dtype=bool)
        else:
            M = block_mask(nb, None if rand_attn is None else np.asarray(rand_attn)[h])
        for b in range(B):
            for n, i in enumerate(qbs):
                Qi = q[b, h, i * block:(i + 1) * block]          # [block, d]
                S = Qi @ k[b, h].T + bias[b][None, :]           # [block, L]
                seen = np.repeat(M[i], block)                   # key tokens this block sees
                S[:, ~seen] = -np.inf                           # outside the pattern: excluded
                P = _softmax_rows(S)
                out[b, h, n * block:(n + 1) * block] = P @ v[b, h]
                if probs is not None:
                    probs[b, h, n * block:(n + 1) * block] = P
    return (out, probs) if return_probs else out


def full_attention(q, k, v, mask):
    """Plain dense attention ``softmax(Q K^T + bias) V`` with the key bias,
    float64 -- the "original_full" reference ("BigBirdPegasus…", section
    "两种注意力实现original_full 与 block_sparse选择原则与默认配置")."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    bias = key_bias(mask, B, L)
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            S = q[b, h] @ k[b, h].T + bias[b][None, :]
            out[b, h] = _softmax_rows(S) @ v[b, h]
    return out
