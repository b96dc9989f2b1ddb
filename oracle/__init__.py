"""Plain CPU oracle for BigBird block-sparse attention (forward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the test-suite, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library (``block_sparse_long_bbsa_amd``) and
imports nothing from it.

The oracle is slow and obviously correct by construction:

* ``oracle.planner``   -- the random-block adjacency (``rand_attn``) built
  with a SplitMix64 stream and a partial Fisher-Yates shuffle.
* ``oracle.attention`` -- masked dense attention under the materialised
  BigBird block mask, in float64.

Every function cites the passage of the source pages it follows, by page
title and section.  Parity status of each function is listed in its module
header; every function here is pinned by a ``-m "not gpu"`` test against
something other than itself (brute force, a library routine, closed forms,
invariants or a published test vector).
"""
from .planner import (SplitMix64, plan_rand_attn, check_rand_attn, candidate_blocks, cap_block,
                      truncate_plan)
from .attention import (
    block_mask, token_mask, key_bias, uses_full_fallback, forward, full_attention,
    attended_key_counts, pair_bias, forward_padded, backward, backward_padded, attended_blocks,
    forward_block_constant,
)

__all__ = [
    "SplitMix64", "plan_rand_attn", "check_rand_attn", "candidate_blocks", "cap_block",
    "truncate_plan",
    "block_mask", "token_mask", "key_bias", "uses_full_fallback", "forward",
    "full_attention", "attended_key_counts", "pair_bias", "forward_padded",
    "backward", "backward_padded", "attended_blocks", "forward_block_constant",
]
