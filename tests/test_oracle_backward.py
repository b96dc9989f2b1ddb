"""Pins of the oracle's backward (CPU only).

``oracle.backward`` writes the gradients of out = softmax(S) V out of their
definition ("models 仓库中的 BigBird…", section "梯度检查点的实现方式": the
operator is trained through; "BigBirdPegasus…", section "使用限制与注意事项":
the sparse probabilities carry no gradient of their own).  Pinned against:

1. torch autograd through scaled_dot_product_attention in float64 with the
   explicit [L, L] additive mask (padding bias, -inf outside the pattern),
   key-side and query x key masking, block 1..64, padded sequences;
2. central finite differences of sum(out * dout) on tiny inputs;
3. closed forms: the key gradients of each (batch, head) sum to zero over
   the keys (the output does not change when one vector is added to every
   key), and a V whose rows are all equal gives dQ = dK = 0;
4. the padded-length variant against autograd through the zero-padded
   computation with the output gradient on the real rows only.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.planner import plan_rand_attn


def _torch_grads(q, k, v, mask, ra, block, dout, qk=False, L_real=None):
    """Autograd through SDPA with the dense additive mask (float64)."""
    B, H, L, d = q.shape
    nb = L // block
    r = 0 if ra is None else ra.shape[2]
    full = A.uses_full_fallback(L, block, r)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    outs = []
    for b in range(B):
        for h in range(H):
            M = np.ones((nb, nb), bool) if full else A.block_mask(nb, ra[h])
            T = np.kron(M.astype(np.int8), np.ones((block, block), np.int8)).astype(bool)
            m = np.ones(L) if mask is None else np.asarray(mask[b], dtype=np.float64)
            add = -10000.0 * (1.0 - (np.outer(m, m) if qk else m[None, :]))
            add = np.where(T, add, -np.inf)
            o = torch.nn.functional.scaled_dot_product_attention(
                tq[b, h][None], tk[b, h][None], tv[b, h][None], attn_mask=torch.from_numpy(add)[None], scale=1.0)[0]
            outs.append(o)
    out = torch.stack(outs).reshape(B, H, L, d)
    w = torch.from_numpy(np.asarray(dout, dtype=np.float64))
    if L_real is not None:
        w = w.clone()
        w[:, :, L_real:] = 0.0
    (out * w).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("B,H,L,block,r,d,qk,seed", [
    (1, 2, 64, 4, 2, 8, False, 0),
    (2, 2, 1024, 64, 3, 16, False, 1),
    (2, 1, 1536, 64, 3, 8, True, 2),
    (1, 2, 2048, 128, 2, 8, False, 3),
    (1, 1, 448, 64, 1, 8, False, 4),      # short: full attention
])
def test_backward_matches_torch_autograd(B, H, L, block, r, d, qk, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    mask = np.ones((B, L))
    mask[-1, int(0.8 * L):] = 0.0
    nb = L // block
    ra = plan_rand_attn(H, nb, r, seed) if nb >= 5 + r else None
    got = A.backward(q, k, v, mask, ra, block, do, query_key_mask=qk)
    want = _torch_grads(q, k, v, mask, ra, block, do, qk=qk)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, atol=1e-10, rtol=0)


def test_backward_central_differences():
    rng = np.random.Generator(np.random.PCG64(5))
    B, H, L, block, r, d = 1, 1, 16, 2, 1, 3
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    mask = np.ones((B, L))
    mask[0, 13:] = 0.0
    ra = plan_rand_attn(H, L // block, r, 5)
    dq, dk, dv = A.backward(q, k, v, mask, ra, block, do, allow_fallback=False)

    def f(q_, k_, v_):
        return float((A.forward(q_, k_, v_, mask, ra, block, allow_fallback=False) * do).sum())

    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(6):
            t, e = int(rng.integers(0, L)), int(rng.integers(0, d))
            xs = [q.copy(), k.copy(), v.copy()]
            xs[which][0, 0, t, e] += eps
            fp = f(*xs)
            xs[which][0, 0, t, e] -= 2 * eps
            fm = f(*xs)
            assert abs((fp - fm) / (2 * eps) - grad[0, 0, t, e]) < 1e-6, (which, t, e)


def test_backward_closed_forms():
    rng = np.random.Generator(np.random.PCG64(6))
    B, H, L, block, r, d = 2, 2, 1024, 64, 3, 8
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    mask = np.ones((B, L))
    mask[1, 600:] = 0.0
    ra = plan_rand_attn(H, L // block, r, 6)
    dq, dk, dv = A.backward(q, k, v, mask, ra, block, do)
    # A vector added to every key leaves the output unchanged.
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-9)
    # Equal value rows: the output is that row whatever the weights.
    vc = np.broadcast_to(rng.standard_normal((B, H, 1, d)), v.shape).copy()
    dq0, dk0, dv0 = A.backward(q, k, vc, mask, ra, block, do)
    assert np.abs(dq0).max() < 1e-10 and np.abs(dk0).max() < 1e-10


@pytest.mark.parametrize("L,block,r,qk", [(1000, 64, 3, False), (1100, 64, 3, True), (333, 64, 1, False)])
def test_backward_padded_matches_autograd(L, block, r, qk):
    rng = np.random.Generator(np.random.PCG64(7))
    B, H, d = 1, 2, 8
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for _ in range(4))
    mask = np.ones((B, L))
    mask[0, L - 40:] = 0.0
    nb = -(-L // block)
    Lp = nb * block
    ra = plan_rand_attn(H, nb, r, 7)
    got = A.backward_padded(q, k, v, mask, ra, block, do, query_key_mask=qk)
    pad = ((0, 0), (0, 0), (0, Lp - L), (0, 0))
    mp = np.concatenate([mask, np.zeros((B, Lp - L))], axis=1)
    want = _torch_grads(np.pad(q, pad), np.pad(k, pad), np.pad(v, pad), mp, ra, block, np.pad(do, pad), qk=qk,
                        L_real=L)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w[:, :, :L], atol=1e-10, rtol=0)
    # Aligned lengths: the padded variant is the plain one.
    Lq = nb * block
    qa, ka, va, da = (rng.standard_normal((B, H, Lq, d)) for _ in range(4))
    ma = np.ones((B, Lq))
    for g, w in zip(A.backward_padded(qa, ka, va, ma, ra, block, da), A.backward(qa, ka, va, ma, ra, block, da)):
        assert np.array_equal(g, w)
