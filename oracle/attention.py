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

Also: the query x key masking mode (the pages' band mask is the outer
product of the query-side and key-side masks), each row's log-sum-exp,
lengths that are not a multiple of the block (the encoder pads to the block
and trims the output), and the output for inputs constant over each key
block one query block at a time (for lengths whose dense scores do not fit
in memory).

Parity status: pinned (tests/test_oracle_attention.py,
tests/test_oracle_extensions.py, tests/test_oracle_block_constant.py) against scalar brute force on tiny inputs,
against torch's scaled_dot_product_attention and logsumexp in float64,
against closed forms (constant V, Q = 0, key shift, attended-key counts,
query x key rows with mask 1 or 0) and against invariants (row sums, exact
zeros, batch independence, padding that changes nothing).
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


def pair_bias(mask_b, rows, L: int, query_key: bool = False) -> np.ndarray:
    """Additive padding bias ``[len(rows), L]`` of one sequence for the query
    rows ``rows``.

    Key side (the default): ``-10000 * (1 - m[u])`` for every query row.
    Query x key (``query_key``): ``-10000 * (1 - m[t] * m[u])``, the outer
    product of the query-side and key-side masks that the pages' band mask
    is built from ("models 仓库中的 BigBird…", section "随机块掩码是如何生成的":
    BigBirdMasks forms the 3-D band mask from the from-mask and the to-mask by
    an einsum).  ``mask_b`` None means every position is valid."""
    rows = np.asarray(rows)
    if mask_b is None:
        return np.zeros((len(rows), L), dtype=np.float64)
    m = np.asarray(mask_b, dtype=np.float64).reshape(L)
    if not query_key:
        return np.broadcast_to(PAD_BIAS * (1.0 - m)[None, :], (len(rows), L)).copy()
    return PAD_BIAS * (1.0 - m[rows][:, None] * m[None, :])


def forward(q, k, v, mask, rand_attn, block: int, query_blocks=None,
            allow_fallback: bool = True, return_probs: bool = False,
            query_key_mask: bool = False, return_lse: bool = False):
    """Masked dense attention under the BigBird block mask, in float64.

    q, k, v: ``[B, H, L, d]`` (any real dtype; upcast exactly to float64).
    mask: ``[B, L]`` values in [0, 1] (1 = valid) or None.
    rand_attn: ``[H, nb-2, r]`` integer plan, or None (no random blocks).
    query_blocks: iterable of query block indices to compute (default: all);
    the result then holds only those blocks' rows, in the order given.
    allow_fallback: apply the short-sequence fallback to full attention.
    query_key_mask: bias -10000 * (1 - m[query] * m[key]) instead of the
    key-side -10000 * (1 - m[key]) (see ``pair_bias``).

    Returns ``out`` (float64 ``[B, H, rows, d]``); with ``return_probs`` also
    the probabilities ``[B, H, rows, L]`` and with ``return_lse`` the natural
    log-sum-exp of each row's scores over the keys it attends, bias included
    (``[B, H, rows]``), in that order after ``out``.
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
    qbs = list(range(nb)) if query_blocks is None else [int(i) for i in query_blocks]
    rows = len(qbs) * block
    out = np.empty((B, H, rows, d), dtype=np.float64)
    probs = np.empty((B, H, rows, L), dtype=np.float64) if return_probs else None
    lse = np.empty((B, H, rows), dtype=np.float64) if return_lse else None
    for h in range(H):
        if full:
            M = np.ones((nb, nb), dtype=bool)
        else:
            M = block_mask(nb, None if rand_attn is None else np.asarray(rand_attn)[h])
        for b in range(B):
            mb = None if mask is None else np.asarray(mask)[b]
            for n, i in enumerate(qbs):
                qrows = np.arange(i * block, (i + 1) * block)
                Qi = q[b, h, i * block:(i + 1) * block]          # [block, d]
                S = Qi @ k[b, h].T + pair_bias(mb, qrows, L, query_key_mask)   # [block, L]
                seen = np.repeat(M[i], block)                   # key tokens this block sees
                S[:, ~seen] = -np.inf                           # outside the pattern: excluded
                P = _softmax_rows(S)
                out[b, h, n * block:(n + 1) * block] = P @ v[b, h]
                if probs is not None:
                    probs[b, h, n * block:(n + 1) * block] = P
                if lse is not None:
                    mx = S.max(axis=-1)
                    lse[b, h, n * block:(n + 1) * block] = mx + np.log(np.exp(S - mx[:, None]).sum(axis=-1))
    res = (out,)
    if return_probs:
        res += (probs,)
    if return_lse:
        res += (lse,)
    return res if len(res) > 1 else out


def forward_padded(q, k, v, mask, rand_attn, block: int, **kw):
    """Forward for a length that need not be a multiple of the block.

    "BigBirdPegasus…", section "序列长度的块对齐要求": the encoder pads its input
    to a multiple of the block size and cuts the padding off the output.
    Here the padding positions are zero vectors with mask 0 (so as keys they
    get the -10000 bias like any padded key); the padded sequence goes
    through ``forward`` and every result is cut back to the first L rows (and
    the first L keys for the probabilities).  ``rand_attn`` is the plan of the
    padded length, ``[H, ceil(L/block) - 2, r]``.  Keyword arguments go to
    ``forward``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    Lp = -(-L // block) * block
    pad = ((0, 0), (0, 0), (0, Lp - L), (0, 0))
    m = np.ones((B, L)) if mask is None else np.asarray(mask, dtype=np.float64).reshape(B, L)
    mp = np.concatenate([m, np.zeros((B, Lp - L))], axis=1)
    res = forward(np.pad(q, pad), np.pad(k, pad), np.pad(v, pad), mp, rand_attn, block, **kw)
    if not isinstance(res, tuple):
        return res[:, :, :L]
    out = [res[0][:, :, :L]]
    i = 1
    if kw.get("return_probs"):
        out.append(res[i][:, :, :L, :L])
        i += 1
    if kw.get("return_lse"):
        out.append(res[i][:, :, :L])
    return tuple(out)


def backward(q, k, v, mask, rand_attn, block: int, dout, allow_fallback: bool = True,
             query_key_mask: bool = False):
    """Gradients of the forward with respect to q, k and v, in float64.

    "models 仓库中的 BigBird…", section "梯度检查点的实现方式": training goes
    through this operator's backward (the encoder can recompute the forward
    instead of storing it); "BigBirdPegasus…", section "使用限制与注意事项":
    the sparse probability matrix itself carries no gradient, so the
    gradients are those of out = P V with P the masked row softmax.  Written
    from the definition: with S the scores plus bias (excluded entries -inf),
    P = softmax(S), O = P V and dO the gradient of the output,

        dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dO * O)),
        dQ = dS K,     dK = dS^T Q

    (no internal scale; the padding bias and the block mask do not depend on
    q or k).  Arguments as ``forward``; dout like q.  Returns (dq, dk, dv),
    float64 ``[B, H, L, d]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, H, L, d = q.shape
    if L % block != 0:
        raise ValueError(f"sequence length {L} is not a multiple of block size {block}")
    nb = L // block
    r = 0 if rand_attn is None else int(np.asarray(rand_attn).shape[2])
    full = allow_fallback and uses_full_fallback(L, block, r)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(H):
        if full:
            M = np.ones((nb, nb), dtype=bool)
        else:
            M = block_mask(nb, None if rand_attn is None else np.asarray(rand_attn)[h])
        seen = np.kron(M.astype(np.int8), np.ones((block, block), np.int8)).astype(bool)
        for b in range(B):
            mb = None if mask is None else np.asarray(mask)[b]
            S = q[b, h] @ k[b, h].T + pair_bias(mb, np.arange(L), L, query_key_mask)
            S[~seen] = -np.inf
            P = _softmax_rows(S)
            O = P @ v[b, h]
            dv[b, h] = P.T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            dS = P * (dP - (do[b, h] * O).sum(axis=-1, keepdims=True))
            dq[b, h] = dS @ k[b, h]
            dk[b, h] = dS.T @ q[b, h]
    return dq, dk, dv


def backward_padded(q, k, v, mask, rand_attn, block: int, dout, **kw):
    """``backward`` for a length that need not be a multiple of the block:
    the zero padding of ``forward_padded`` (mask 0 on the padding), a zero
    output gradient on the padded rows (they are cut off the output), then
    the gradients of the first L rows."""
    q = np.asarray(q, dtype=np.float64)
    B, H, L, d = q.shape
    Lp = -(-L // block) * block
    pad = ((0, 0), (0, 0), (0, Lp - L), (0, 0))
    m = np.ones((B, L)) if mask is None else np.asarray(mask, dtype=np.float64).reshape(B, L)
    mp = np.concatenate([m, np.zeros((B, Lp - L))], axis=1)
    g = backward(np.pad(q, pad), np.pad(np.asarray(k, np.float64), pad), np.pad(np.asarray(v, np.float64), pad),
                 mp, rand_attn, block, np.pad(np.asarray(dout, np.float64), pad), **kw)
    return tuple(x[:, :, :L] for x in g)


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


def attended_blocks(nb: int, i: int, rand_attn_h) -> np.ndarray:
    """The key blocks query block ``i`` sees, ascending and distinct: the
    row of ``block_mask`` taken on its own, for sequences whose ``[nb, nb]``
    mask does not fit in memory.  The global blocks 0 and nb-1 see every
    block; a middle block sees blocks 0 and nb-1, its window i-1..i+1 and
    its random blocks (row i-1 of ``rand_attn_h``)."""
    if i == 0 or i == nb - 1:
        return np.arange(nb)
    seen = {0, nb - 1, i - 1, i, i + 1}
    if rand_attn_h is not None:
        seen.update(int(j) for j in np.asarray(rand_attn_h)[i - 1])
    return np.array(sorted(seen))


def forward_block_constant(k_blocks, v_blocks, mask_b, rand_attn_h, block: int, query_blocks, query=None):
    """``forward`` of one (batch, head) whose query rows all equal ``query``
    (default: the unit vector e_0) and whose key and value rows are constant
    over each key block: row u of K is ``k_blocks[u // block]``, row u of V
    is ``v_blocks[u // block]``.  For lengths whose dense scores do not fit
    in memory; no fallback (the sequence must be longer than the fallback
    threshold).

    The definition as in ``forward``, with its sums regrouped: key u of block
    b scores query . k_b plus the key bias -10000 (1 - m_u), the row softmax
    runs over the keys of the attended blocks, and since every key of block
    b carries v_b the output is sum_b (sum of the probabilities of block b's
    keys) v_b.  All rows of a query block are equal; returns float64
    ``[len(query_blocks), d]``, one row per query block."""
    kb = np.asarray(k_blocks, dtype=np.float64)
    vb = np.asarray(v_blocks, dtype=np.float64)
    nb, d = kb.shape
    L = nb * block
    qv = np.zeros(d) if query is None else np.asarray(query, dtype=np.float64)
    if query is None:
        qv[0] = 1.0
    m = np.ones(L) if mask_b is None else np.asarray(mask_b, dtype=np.float64).reshape(L)
    block_scores = kb @ qv                                      # [nb]
    out = np.empty((len(query_blocks), d), dtype=np.float64)
    for n, i in enumerate(query_blocks):
        A = attended_blocks(nb, int(i), rand_attn_h)
        tok = (A[:, None] * block + np.arange(block)[None, :]).ravel()
        S = np.repeat(block_scores[A], block) + PAD_BIAS * (1.0 - m[tok])
        P = np.exp(S - S.max())
        P /= P.sum()
        out[n] = P.reshape(len(A), block).sum(axis=1) @ vb[A]
    return out
