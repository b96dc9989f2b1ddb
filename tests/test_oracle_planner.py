"""Pins of the oracle planner (CPU only).

The planner is pinned to things other than itself: the published SplitMix64
test vector, closed forms of the bounded draw, chi-square uniformity, and
the invariants the pages state for the random blocks ("models 仓库中的
BigBird…", section "随机块掩码是如何生成的"): r distinct blocks per middle
row, all middle blocks, none in the row's 3-block window.
"""
import numpy as np
import pytest

from oracle.planner import SplitMix64, plan_rand_attn, check_rand_attn, candidate_blocks


def test_splitmix64_published_vector():
    # Published test vector of SplitMix64 for seed 1234567 (Rosetta Code task
    # "Pseudo-random numbers/Splitmix64", matching Vigna's reference
    # splitmix64.c, which follows Steele, Lea and Flood, OOPSLA 2014).
    g = SplitMix64(1234567)
    got = [g.next_u64() for _ in range(5)]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_splitmix64_state_advances_by_gamma():
    g = SplitMix64(0)
    for n in range(1, 6):
        g.next_u64()
        assert g.state == (n * 0x9E3779B97F4A7C15) % (1 << 64)


@pytest.mark.parametrize("k", [0, 1, 5, 17, 63])
def test_bounded_draw_power_of_two_is_low_bits(k):
    # 2**64 mod 2**k == 0: no rejection, the draw is the low k bits.
    a, b = SplitMix64(99), SplitMix64(99)
    for _ in range(50):
        assert a.below(1 << k) == b.next_u64() & ((1 << k) - 1)


def test_bounded_draw_rejects_exactly_the_low_values():
    # For m = 3, 2**64 mod 3 == 1: only x == 0 is rejected.  For m = 2**63 + 1,
    # 2**64 mod m == 2**63 - 1: outputs below it are rejected and skipped.
    m = (1 << 63) + 1
    thr = (1 << 64) % m
    assert thr == (1 << 63) - 1
    a, b = SplitMix64(7), SplitMix64(7)
    for _ in range(40):
        got = a.below(m)
        while True:
            x = b.next_u64()
            if x >= thr:
                break
        assert got == x % m
    assert (1 << 64) % 3 == 1


@pytest.mark.parametrize("m", [3, 7, 10])
def test_bounded_draw_uniform_chi_square(m):
    g = SplitMix64(2024 + m)
    n = 20000
    counts = np.bincount([g.below(m) for _ in range(n)], minlength=m)
    exp = n / m
    chi2 = ((counts - exp) ** 2 / exp).sum()
    # 99.9% quantile of chi-square with m-1 <= 9 degrees of freedom is < 28
    assert chi2 < 28.0, counts


def test_candidates_exclude_window_and_globals():
    nb = 12
    assert candidate_blocks(nb, 1) == list(range(3, 11))
    assert candidate_blocks(nb, 5) == [1, 2, 3, 7, 8, 9, 10]
    assert candidate_blocks(nb, 10) == list(range(1, 9))


@pytest.mark.parametrize("H,nb,r", [(1, 12, 1), (12, 16, 3), (16, 64, 3), (3, 8, 3),
                                    (2, 40, 5), (16, 256, 2), (1, 6, 1)])
def test_plan_invariants(H, nb, r):
    for seed in (0, 1, 12345):
        ra = plan_rand_attn(H, nb, r, seed)
        assert ra.shape == (H, nb - 2, r) and ra.dtype == np.int32
        assert check_rand_attn(ra, nb, r) == []
        # independent statement of the invariants
        for h in range(H):
            for i in range(1, nb - 1):
                row = ra[h, i - 1]
                assert len(set(row.tolist())) == r
                assert all(1 <= c <= nb - 2 and abs(int(c) - i) > 1 for c in row)


def test_plan_deterministic_and_seed_dependent():
    a = plan_rand_attn(4, 32, 3, 5)
    b = plan_rand_attn(4, 32, 3, 5)
    c = plan_rand_attn(4, 32, 3, 6)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    # heads draw from one stream: head 1 differs from head 0
    assert not np.array_equal(a[0], a[1])


def test_plan_exhausts_candidates_at_minimum_nb():
    # nb = 5 + r: a middle row 2..nb-3 has exactly r candidates, so it takes all.
    r = 3
    nb = 5 + r
    ra = plan_rand_attn(2, nb, r, 3)
    for h in range(2):
        for i in range(2, nb - 2):
            assert sorted(ra[h, i - 1].tolist()) == candidate_blocks(nb, i)


def test_plan_pick_frequencies_uniform():
    # Each candidate of a row is picked with probability r/n.
    nb, r, i = 14, 3, 6
    cand = candidate_blocks(nb, i)
    n = len(cand)
    counts = dict.fromkeys(cand, 0)
    trials = 3000
    for seed in range(trials):
        for c in plan_rand_attn(1, nb, r, seed)[0, i - 1]:
            counts[int(c)] += 1
    exp = trials * r / n
    chi2 = sum((c - exp) ** 2 / exp for c in counts.values())
    assert chi2 < 30.0, counts   # n-1 = 8 degrees of freedom; 99.9% quantile ~26.1


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):
        plan_rand_attn(1, 7, 3, 0)      # nb < 5 + r
    with pytest.raises(ValueError):
        plan_rand_attn(1, 16, 0, 0)     # r = 0 unsupported
    with pytest.raises(ValueError):
        plan_rand_attn(0, 16, 3, 0)


def test_check_rand_attn_catches_planted_mistakes():
    ra = plan_rand_attn(2, 16, 3, 1)
    bad = ra.copy(); bad[0, 4, 1] = bad[0, 4, 0]
    assert any("repeated" in e for e in check_rand_attn(bad, 16, 3))
    bad = ra.copy(); bad[1, 6, 2] = 7          # row i=7 owns window {6,7,8}
    assert any("window" in e for e in check_rand_attn(bad, 16, 3))
    bad = ra.copy(); bad[0, 9, 0] = 0
    assert any("middle" in e for e in check_rand_attn(bad, 16, 3))
    bad = ra.copy(); bad[0, 9, 0] = 15
    assert any("middle" in e for e in check_rand_attn(bad, 16, 3))
    assert check_rand_attn(ra[:, :-1], 16, 3)


def test_golden_plan_fixture():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "plan_H3_nb16_r3_seed1.txt")
    rows = [list(map(int, ln.split())) for ln in open(path) if ln.strip() and not ln.startswith("#")]
    want = np.array(rows, dtype=np.int32).reshape(3, 14, 3)
    assert np.array_equal(plan_rand_attn(3, 16, 3, 1), want)


# ---- the last_idx cap ("models 仓库中的 BigBird…", section "随机块掩码是如何生成的":
# random blocks only within the first 1024 tokens; the plan of the maximum
# length serves shorter sequences through its first rows).

from oracle.planner import cap_block, truncate_plan  # noqa: E402


def test_cap_block_closed_form():
    assert cap_block(64, 64, 1024) == 15          # blocks 0..15 hold tokens 0..1023
    assert cap_block(64, 64, 1087) == 15          # block 16 would end at token 1088
    assert cap_block(64, 64, 1088) == 16
    assert cap_block(256, 128, 1024) == 7
    assert cap_block(64, 64, 0) == 62 and cap_block(64, 64, None) == 62
    assert cap_block(20, 64, 1 << 20) == 18        # never past the last middle block


def test_capped_candidates_explicit():
    # nb = 20, block 64, last_idx 384: blocks 1..5 allowed.
    assert candidate_blocks(20, 1, 64, 384) == [3, 4, 5]
    assert candidate_blocks(20, 2, 64, 384) == [4, 5]
    assert candidate_blocks(20, 4, 64, 384) == [1, 2]
    assert candidate_blocks(20, 6, 64, 384) == [1, 2, 3, 4]
    assert candidate_blocks(20, 12, 64, 384) == [1, 2, 3, 4, 5]
    assert candidate_blocks(20, 12) == [c for c in range(1, 19) if abs(c - 12) > 1]


def test_capped_plan_exhausts_rows_with_exactly_r_candidates():
    # r = 2 under the cap above: rows 2, 3 and 4 have exactly two candidates,
    # so they must pick exactly those, in some order.
    plan = plan_rand_attn(4, 20, 2, 9, block=64, last_idx=384)
    for h in range(4):
        assert set(plan[h, 1]) == {4, 5}
        assert set(plan[h, 2]) == {1, 5}
        assert set(plan[h, 3]) == {1, 2}
    assert check_rand_attn(plan, 20, 2, block=64, last_idx=384) == []
    assert plan.max() <= 5


def test_capped_plan_invariants_and_inactive_cap():
    for seed in range(5):
        capped = plan_rand_attn(3, 64, 3, seed, block=64, last_idx=1024)
        assert check_rand_attn(capped, 64, 3, block=64, last_idx=1024) == []
        assert capped.max() <= 15 and capped.min() >= 1
        # A cap at or past the last middle block changes nothing.
        for li in (63 * 64, 1 << 20, 0, None):
            assert np.array_equal(plan_rand_attn(3, 64, 3, seed, block=64, last_idx=li),
                                  plan_rand_attn(3, 64, 3, seed))
    # The same plan violates a lower cap, and an uncapped plan violates this one.
    capped = plan_rand_attn(3, 64, 3, 1, block=64, last_idx=1024)
    assert check_rand_attn(capped, 64, 3, block=64, last_idx=512) != []
    assert check_rand_attn(plan_rand_attn(3, 64, 3, 1), 64, 3, block=64, last_idx=1024) != []


def test_capped_pick_frequencies_are_uniform():
    # Row 40 of nb = 64 under last_idx 1024: 15 candidates (blocks 1..15),
    # each picked with probability 3/15 over many seeds (chi-square, loose).
    counts = np.zeros(16)
    n = 600
    for seed in range(n):
        for c in plan_rand_attn(1, 64, 3, seed, block=64, last_idx=1024)[0, 39]:
            counts[c] += 1
    exp = n * 3 / 15
    chi2 = ((counts[1:] - exp) ** 2 / exp).sum()
    assert counts[0] == 0 and chi2 < 45.0      # 14 degrees of freedom; p ~ 5e-5


def test_capped_plan_too_low_cap_raises():
    with pytest.raises(ValueError):
        plan_rand_attn(1, 64, 3, 0, block=64, last_idx=256)
    with pytest.raises(ValueError):
        plan_rand_attn(1, 64, 3, 0, last_idx=1024)      # a cap needs the block size


def test_truncated_plan_serves_shorter_sequences():
    big = plan_rand_attn(2, 64, 3, 3, block=64, last_idx=1024)
    for nb in (17, 20, 40):
        small = truncate_plan(big, nb)
        assert small.shape == (2, nb - 2, 3)
        assert np.array_equal(small, big[:, :nb - 2])
        assert check_rand_attn(small, nb, 3) == []
    # Uncapped picks reach past a shorter sequence's middle blocks.
    assert check_rand_attn(truncate_plan(plan_rand_attn(2, 64, 3, 3), 20), 20, 3) != []
