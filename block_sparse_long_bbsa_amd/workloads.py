"""Seeded synthetic inputs for the BigBird block-sparse attention forward.

This module holds no attention arithmetic and no planner: it only draws the
inputs (Q, K, V, padding mask) that both the HIP path and the CPU oracle
consume, so that both sides see exactly the same numbers.  The random-block
plan is *not* drawn here; each side builds it from the plan seed with its
own SplitMix64 planner.  The one exception is ``block_constant_case``, for
lengths where the oracle planner's per-row candidate lists do not fit in
memory: it draws an arbitrary plan that satisfies the plan invariants (not
the method's planner) and passes it to both sides as an input.

The five workloads stand in for the encoder shapes the pages describe
(BigBird-base: 12 heads of 64 on hidden 768, block 64, 3 random blocks;
BigBirdPegasus-large encoder: 16 heads of 64 on d_model 1024, block 64,
3 random blocks).  No dataset is used.

Recipe (all draws from ``numpy.random.Generator(PCG64(1000 + id))``, in this
order): q, k, v as float32 ``standard_normal`` in C order ``[B, H, L, d]``;
then the valid lengths; then the outlier positions.  Q is scaled by 1/8
(= 1/sqrt(64)) for the bf16 workloads, all three by 1/sqrt(8) for the fp32
one.  bf16 workloads are rounded from float32 to bfloat16 with
round-to-nearest-even; the returned float32 arrays hold exactly those bf16
values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic forward workload."""
    id: int
    name: str
    B: int
    H: int
    L: int
    d: int
    block: int
    r: int
    dtype: str                  # "f32" or "bf16"
    plan_seed: int
    description: str = ""
    extra_plan_seeds: tuple = field(default_factory=tuple)
    masked: bool = True         # the call gets the padding mask (False: no mask, every key valid)

    @property
    def nb(self) -> int:
        return self.L // self.block


WORKLOADS = {
    1: Workload(1, "fp32_B1_H2_L1024_b64_r3", 1, 2, 1024, 64, 64, 3, "f32", 1,
                "fp32, q/k/v ~ N(0,1)/sqrt(8), mask all ones"),
    2: Workload(2, "bf16_B4_H12_L4096_b64_r3", 4, 12, 4096, 64, 64, 3, "bf16", 0,
                "BigBird-base shape; valid length 64*round(U{3072..4096}/64), mask 0 on the tail"),
    3: Workload(3, "bf16_B8_H16_L4096_b64_r3", 8, 16, 4096, 64, 64, 3, "bf16", 0,
                "Pegasus-large encoder shape; valid length U{1024..4096} (partial blocks)",
                extra_plan_seeds=(1,)),
    4: Workload(4, "bf16_B2_H12_L16384_b64_r3", 2, 12, 16384, 64, 64, 3, "bf16", 0,
                "long context, no padding (the call gets no mask)", masked=False),
    5: Workload(5, "bf16_B1_H16_L32768_b128_r2", 1, 16, 32768, 64, 128, 2, "bf16", 0,
                "block 128; 1% of keys per (b,h) get +4 on every element; last 10% padded"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16 -> float32 (exact values)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def make_inputs(wid: int):
    """Draw the inputs of workload ``wid``.

    Returns a dict with ``q, k, v`` (float32 ``[B,H,L,d]``, bf16-exact for
    bf16 workloads), ``mask`` (float32 ``[B, L]`` of 0/1), ``valid``
    (int array of valid lengths) and ``workload``.
    """
    w = WORKLOADS[wid]
    rng = np.random.Generator(np.random.PCG64(1000 + wid))
    shape = (w.B, w.H, w.L, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if wid == 1:
        valid = np.full(w.B, w.L, dtype=np.int64)
    elif wid == 2:
        valid = (64 * np.round(rng.integers(3072, 4097, size=w.B) / 64)).astype(np.int64)
    elif wid == 3:
        valid = rng.integers(1024, 4097, size=w.B).astype(np.int64)
    elif wid == 4:
        valid = np.full(w.B, w.L, dtype=np.int64)
    elif wid == 5:
        valid = np.full(w.B, int(np.floor(0.9 * w.L)), dtype=np.int64)
        n_out = int(round(0.01 * w.L))
        for b in range(w.B):
            for h in range(w.H):
                pos = rng.choice(w.L, size=n_out, replace=False)
                k[b, h, pos, :] += np.float32(4.0)
    else:
        raise KeyError(wid)
    if w.dtype == "f32":
        s = np.float32(1.0 / np.sqrt(8.0))
        q *= s
        k *= s
        v *= s
    else:
        q *= np.float32(0.125)
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    mask = (np.arange(w.L)[None, :] < valid[:, None]).astype(np.float32)
    return {"q": q, "k": k, "v": v, "mask": mask, "valid": valid, "workload": w}


def make_case(B, H, L, d, seed, dtype="bf16", valid=None, q_scale=None):
    """Small seeded case for tests: N(0,1) inputs, Q scaled by 1/sqrt(d)
    (or ``q_scale``), optional per-batch valid lengths, bf16-exact when
    ``dtype == "bf16"``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, L, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    q *= np.float32(1.0 / np.sqrt(d) if q_scale is None else q_scale)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    if valid is None:
        mask = np.ones((B, L), dtype=np.float32)
    else:
        valid = np.asarray(valid)
        mask = (np.arange(L)[None, :] < valid[:, None]).astype(np.float32)
    return {"q": q, "k": k, "v": v, "mask": mask}


def block_constant_case(L, d, block, r, seed, valid):
    """Inputs constant over each key block, for checks at lengths whose dense
    oracle does not fit in memory (one batch, one head).

    Every query row is the unit vector e_0, so a key's score is component 0
    of its key vector.  Key and value vectors are drawn per block (float32
    ``standard_normal``, keys times 2, rounded to bfloat16) and repeated over
    the block's rows.  The mask is 1 on the first ``valid`` positions.  The
    plan ``[1, nb - 2, r]`` holds, for every middle row, r distinct middle
    blocks outside the row's window, drawn uniformly with redraws of entries
    that break this; it is an input like the others, not the method's
    planner.  Returns block-level ``k_blocks``, ``v_blocks`` (``[nb, d]``),
    ``mask`` (``[1, L]``) and ``plan``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = L // block
    kb = round_to_bf16(2.0 * rng.standard_normal((nb, d), dtype=np.float32))
    vb = round_to_bf16(rng.standard_normal((nb, d), dtype=np.float32))
    rows = np.arange(1, nb - 1)[:, None]
    plan = rng.integers(1, nb - 1, size=(nb - 2, r))

    def bad(pl):
        out = np.abs(pl - rows) <= 1
        for t in range(1, r):
            out[:, t] |= (pl[:, :t] == pl[:, t:t + 1]).any(axis=1)
        return out

    b = bad(plan)
    while b.any():
        plan[b] = rng.integers(1, nb - 1, size=int(b.sum()))
        b = bad(plan)
    mask = (np.arange(L)[None, :] < valid).astype(np.float32)
    return {"k_blocks": kb, "v_blocks": vb, "mask": mask, "plan": plan.astype(np.int32)[None]}
