"""Pins of the oracle's energy score and largest-marginal-gain allocation.

The exactness claim of the Block-GTQ abstract (greedy exactly minimises the
separable integer proxy under equal costs and diminishing gains) is checked by
exhaustive search on tiny instances, with a negative control that breaks the
diminishing-gains premise and must make greedy fail."""
import itertools
import math

import numpy as np
import pytest

from gtq_inputs import HALF, INTERLEAVED, apply_rope
from oracle import gtq_oracle as O

D = O.rate_distortion()


def _brute_min(scores, dist, b_min, b_max, budget):
    best = math.inf
    for bits in itertools.product(range(b_min, b_max + 1), repeat=len(scores)):
        if sum(bits) == budget:
            best = min(best, sum(s * dist[b] for s, b in zip(scores, bits)))
    return best


def test_greedy_equals_brute_force():
    rng = np.random.default_rng(2024)
    cases = 0
    for n in range(2, 7):
        for b_min, b_max in [(1, 4), (1, 3), (2, 4), (1, 2)]:
            for _ in range(3):
                s = np.exp(1.5 * rng.standard_normal(n))
                for budget in range(n * b_min, n * b_max + 1):
                    rates = O.greedy_allocate(s, D, b_min, b_max, budget)
                    assert int(rates.sum()) == budget
                    assert rates.min() >= b_min and rates.max() <= b_max
                    got = O.proxy(s, D, rates)
                    ref = _brute_min(list(s), D, b_min, b_max, budget)
                    assert got == pytest.approx(ref, rel=1e-12, abs=1e-15)
                    cases += 1
    assert cases > 300


def test_negative_control_nonconvex_penalties():
    """With gains that grow (D = 1.0, 0.9, 0.1, 0.0 for b = 1..4 is not diminishing),
    greedy must miss the exhaustive minimum on some instance: proves the test above
    can fail."""
    bad = np.array([1.0, 1.0, 0.9, 0.1, 0.0])
    rng = np.random.default_rng(9)
    failures = 0
    for _ in range(50):
        n = int(rng.integers(2, 5))
        s = np.exp(rng.standard_normal(n))
        for budget in range(n, 4 * n + 1):
            got = O.proxy(s, bad, O.greedy_allocate(s, bad, 1, 4, budget))
            ref = _brute_min(list(s), bad, 1, 4, budget)
            if got > ref * (1 + 1e-9) + 1e-15:
                failures += 1
    assert failures > 0


def test_equal_scores_give_uniform_allocation():
    for avg in (1, 2, 3, 4):
        r = O.greedy_allocate(np.ones(64), D, 1, 4, 64 * avg)
        assert np.all(r == avg)          # uniform TQ-MSE is the equal-score special case


def test_dominant_block_reaches_max_first():
    s = np.ones(64)
    s[17] = 1e6
    r = O.greedy_allocate(s, D, 1, 4, 64 + 3)
    assert r[17] == 4 and r.sum() == 67 and np.all(np.delete(r, 17) == 1)


def test_tie_break_smallest_index():
    r = O.greedy_allocate(np.ones(4), D, 1, 4, 5)
    assert r.tolist() == [2, 1, 1, 1]


def test_bad_parameters():
    with pytest.raises(ValueError):
        O.greedy_allocate(np.ones(4), D, 1, 4, 3)
    with pytest.raises(ValueError):
        O.greedy_allocate(np.ones(4), D, 1, 4, 17)
    with pytest.raises(ValueError):
        O.greedy_allocate(np.ones(4), D, 3, 2, 10)


def test_energy_score_hand_example():
    """Two calibration rows; block 0 = coordinates (0, 64), block 5 = (5, 69)."""
    q = np.zeros((2, 128), np.float32)
    k = np.zeros((1, 128), np.float32)
    q[0, 0], q[0, 64], q[1, 0] = 1.0, 2.0, 3.0      # block 0: (1+4 + 9) / 2 = 7
    q[1, 5], q[1, 69] = 2.0, 2.0                    # block 5: (0 + 8) / 2 = 4
    k[0, 0], k[0, 64], k[0, 5] = 1.0, 1.0, 3.0      # block 0: 2, block 5: 9
    s = O.energy_scores(q, k, HALF)
    assert s[0] == pytest.approx(14.0)
    assert s[5] == pytest.approx(36.0)
    assert np.count_nonzero(s) == 2


@pytest.mark.parametrize("layout", [HALF, INTERLEAVED])
def test_scores_are_rope_invariant_only_with_the_right_pairing(layout):
    """Block energies do not change under RoPE when blocks pair the coordinates that
    RoPE rotates together; scoring with the other pairing changes them."""
    rng = np.random.default_rng(3)
    q = (rng.standard_normal((256, 128)) * np.exp(rng.standard_normal(128))).astype(np.float32)
    k = (rng.standard_normal((256, 128)) * np.exp(rng.standard_normal(128))).astype(np.float32)
    pos = rng.integers(0, 100000, size=256)
    qr = apply_rope(q, pos, layout=layout)
    kr = apply_rope(k, pos, layout=layout)
    s_pre = O.energy_scores(q, k, layout)
    s_post = O.energy_scores(qr, kr, layout)
    assert np.allclose(s_pre, s_post, rtol=1e-5)
    other = INTERLEAVED if layout == HALF else HALF
    assert not np.allclose(O.energy_scores(q, k, other), O.energy_scores(qr, kr, other), rtol=1e-3)


def test_groups_layout():
    rates = np.ones(64, dtype=int)
    rates[[3, 10]] = 3
    rates[0] = 2
    g = O.groups_from_rates(rates, HALF)
    assert [r for r, _ in g] == [1, 2, 3]
    assert g[1][1].tolist() == [0, 64]
    assert g[2][1].tolist() == [3, 67, 10, 74]
    assert sum(len(c) for _, c in g) == 128
    gi = O.groups_from_rates(rates, INTERLEAVED)
    assert gi[2][1].tolist() == [6, 7, 20, 21]
