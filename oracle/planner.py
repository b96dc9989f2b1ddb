"""Oracle planner for the random-block adjacency ``rand_attn`` (pure Python).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix
------------------
"models 仓库中的 BigBird：线性复杂度稀疏注意力与长序列训练的完整实践",
section "随机块掩码是如何生成的": every middle query block row (all block
indices except the first and the last) gets ``num_rand_blocks`` random key
blocks, drawn by a permutation over the middle block indices with the row's
own 3-block window removed, so random blocks never overlap the window; the
plan is fixed per attention head when the layer is built, with the layer
index as the seed.

What the pages leave open, and the reading taken here
-----------------------------------------------------
The pages draw with numpy's permutation, whose stream cannot be reproduced
bit for bit outside numpy.  This planner replaces it with a fully specified
stream so that the host C++ planner of the library and this oracle agree bit
for bit:

* generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014), one stream seeded with the
  layer seed, consumed head by head, row by row, pick by pick;
* bounded draw ``U(m)``: rejection of the lowest ``2**64 mod m`` outputs, then
  ``x mod m`` (exactly uniform);
* row ``i`` (1 <= i <= nb-2): candidates ``C`` = ascending block indices in
  ``1..nb-2`` at distance > 1 from ``i``; the first ``r`` positions of a
  partial Fisher-Yates (Durstenfeld) shuffle of ``C`` are the row's picks, in
  draw order;
* the page's ``last_idx`` limit (random blocks only within the first 1024
  tokens) is an option: it removes from ``C`` the blocks that do not lie
  wholly inside the first ``last_idx`` tokens, with the same stream and
  shuffle; a plan built for a longer sequence is used for a shorter one by
  keeping its first nb-2 rows (``truncate_plan``), as the page describes.

Parity status: pinned.  SplitMix64 against its published test vector, the
bounded draw against closed forms and a chi-square test, the plan against
its invariants (tests/test_oracle_planner.py) and against the independent
C++ planner (tests/test_plan_c.py).
"""
from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


class SplitMix64:
    """SplitMix64 generator, written from its published definition.

    state += golden gamma; output = mix(state), where mix xors-shifts by 30,
    multiplies, xors-shifts by 27, multiplies, xors-shifts by 31 (all mod 2**64).
    """

    def __init__(self, seed: int):
        self.state = int(seed) & _MASK64

    def next_u64(self) -> int:
        self.state = (self.state + _GAMMA) & _MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        return z ^ (z >> 31)

    def below(self, m: int) -> int:
        """Exactly uniform integer in [0, m) by rejection (m >= 1)."""
        if m < 1:
            raise ValueError("bounded draw needs m >= 1")
        threshold = (1 << 64) % m          # == (2**64 - m) mod m
        while True:
            x = self.next_u64()
            if x >= threshold:
                return x % m


def cap_block(nb: int, block: int = None, last_idx: int = None) -> int:
    """Largest block index a random pick may take.

    Without a cap it is nb-2 (the last middle block).  With ``last_idx`` > 0
    the picks lie wholly inside the first ``last_idx`` tokens ("models 仓库中的
    BigBird…", section "随机块掩码是如何生成的": the layer limits the random
    blocks to the first 1024 tokens), i.e. block c needs (c+1)*block <=
    last_idx, so the cap is min(nb-2, last_idx // block - 1)."""
    if last_idx is None or last_idx <= 0:
        return nb - 2
    if block is None or block < 1:
        raise ValueError("a last_idx cap needs the block size")
    return min(nb - 2, last_idx // block - 1)


def candidate_blocks(nb: int, i: int, block: int = None, last_idx: int = None) -> list[int]:
    """Random-block candidates of middle row ``i``: the middle block indices
    (first and last block removed) outside the row's window {i-1, i, i+1}
    (page "models 仓库中的 BigBird…", section "随机块掩码是如何生成的"),
    ascending; with a ``last_idx`` cap only blocks up to ``cap_block``."""
    top = cap_block(nb, block, last_idx)
    return [c for c in range(1, top + 1) if abs(c - i) > 1]


def plan_rand_attn(H: int, nb: int, r: int, seed: int, block: int = None,
                   last_idx: int = None) -> np.ndarray:
    """Build ``rand_attn`` as int32 ``[H, nb-2, r]``; row ``i-1`` holds the
    random key blocks of middle query block ``i``.  ``last_idx`` (tokens,
    with ``block``) caps the picks as in ``cap_block``; without it, or when
    the cap reaches nb-2, the plan is the uncapped one.

    Raises ValueError when an argument is out of range or when a row has
    fewer than ``r`` candidates (nb < 5 + r, or a cap too low for r).
    """
    if H < 1 or nb < 1 or r < 1:
        raise ValueError("H, nb and r must be >= 1")
    if nb < 5 + r:
        raise ValueError("nb must be >= 5 + r for every middle row to have r candidates")
    cands = [candidate_blocks(nb, i, block, last_idx) for i in range(1, nb - 1)]
    if min(len(c) for c in cands) < r:
        raise ValueError(f"the last_idx cap leaves a middle row fewer than r = {r} candidates")
    rng = SplitMix64(seed)
    out = np.zeros((H, nb - 2, r), dtype=np.int32)
    for h in range(H):
        for i in range(1, nb - 1):
            cand = list(cands[i - 1])
            n = len(cand)
            for t in range(r):
                j = t + rng.below(n - t)
                cand[t], cand[j] = cand[j], cand[t]
                out[h, i - 1, t] = cand[t]
    return out


def truncate_plan(rand_attn: np.ndarray, nb: int) -> np.ndarray:
    """The plan of a shorter sequence taken from a longer one's: its first
    nb-2 rows ("models 仓库中的 BigBird…", section "随机块掩码是如何生成的": the
    layer builds the plan once for its maximum length and uses the first
    from_seq_length // block - 2 rows of it).  The result is valid for nb
    blocks only when every kept pick is a middle block of the shorter
    sequence, which a last_idx cap within the shorter length guarantees;
    check it with ``check_rand_attn``."""
    ra = np.asarray(rand_attn)
    if ra.ndim != 3 or ra.shape[1] < nb - 2 or nb < 3:
        raise ValueError("the source plan must have at least nb-2 rows")
    return np.ascontiguousarray(ra[:, :nb - 2, :]).astype(np.int32)


def check_rand_attn(rand_attn: np.ndarray, nb: int, r: int, block: int = None,
                    last_idx: int = None) -> list[str]:
    """Return the list of invariant violations of a plan (empty when valid):
    shape [H, nb-2, r]; every entry a middle block (at most ``cap_block``
    under a last_idx cap); the r entries of a row distinct; none inside the
    row's window."""
    errs: list[str] = []
    ra = np.asarray(rand_attn)
    if ra.ndim != 3 or ra.shape[1] != nb - 2 or ra.shape[2] != r:
        return [f"shape {ra.shape} is not [H, {nb - 2}, {r}]"]
    top = cap_block(nb, block, last_idx)
    for h in range(ra.shape[0]):
        for i in range(1, nb - 1):
            row = [int(x) for x in ra[h, i - 1]]
            if len(set(row)) != r:
                errs.append(f"h={h} i={i}: repeated block in {row}")
            for c in row:
                if not (1 <= c <= nb - 2):
                    errs.append(f"h={h} i={i}: block {c} is not a middle block")
                elif c > top:
                    errs.append(f"h={h} i={i}: block {c} lies past the last_idx cap (block {top})")
                elif abs(c - i) <= 1:
                    errs.append(f"h={h} i={i}: block {c} lies in the window")
    return errs
