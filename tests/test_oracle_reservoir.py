"""Pins of the oracle's reservoir stage: keys, selection and the law they draw (CPU).

The A-Res key ln(u)/w with the top-B rule ([Nexus] section 2.3, Eq. (6) at
n = 1) must draw the successive-sampling law of weighted sampling without
replacement (Efraimidis and Spirakis, cited in [Nexus] appendix 11).  The law is
computed independently by enumeration (oracle/enumerate.py) and the oracle's
frequencies over many Philox step counters must match within 5 sigma.
"""

import numpy as np
import pytest

from oracle import nexus, philox
from oracle.enumerate import inclusion_probabilities_float


def _frequencies(w, budget, n_draws, seed=7, unit=3, layer=1):
    w = np.asarray(w, dtype=np.float64)
    n = len(w)
    steps = np.arange(n_draws, dtype=np.uint64)[:, None]
    u = philox.uniforms(np.arange(n, dtype=np.uint64)[None, :], unit, layer, steps, seed)
    counts = np.zeros(n)
    for s in range(n_draws):
        keep = nexus.select_top(nexus.reservoir_keys(w, u[s]), budget)
        assert len(keep) == budget
        counts[keep] += 1
    return counts / n_draws


def _assert_within_5_sigma(freq, pi, n_draws):
    pi = np.asarray(pi)
    sigma = np.sqrt(pi * (1 - pi) / n_draws)
    bad = np.abs(freq - pi) > 5 * sigma + 1e-12
    assert not bad.any(), (freq, pi, sigma)


def test_keys_special_values():
    w = np.array([0.5, 0.0, -1.0, 0.25, 0.1])
    u = np.array([0.5, 0.5, 0.5, 1.0, 0.25])
    keys = nexus.reservoir_keys(w, u)
    assert keys[1] == -np.inf and keys[2] == -np.inf
    assert keys[3] == 0.0
    np.testing.assert_allclose(keys[0], np.log(0.5) / 0.5)
    forced = nexus.reservoir_keys(w, u, n_sink=1, n_recent=2)
    assert forced[0] == np.inf and forced[3] == np.inf and forced[4] == np.inf
    with pytest.raises(ValueError):
        nexus.reservoir_keys(np.array([0.1, np.nan]), np.array([0.5, 0.5]))
    with pytest.raises(ValueError):
        nexus.reservoir_keys(np.array([0.1, np.inf]), np.array([0.5, 0.5]))


def test_select_ties_prefer_newer_and_output_ascending():
    keys = np.array([1.0, 1.0, 0.0, 1.0, -np.inf, np.inf])
    np.testing.assert_array_equal(nexus.select_top(keys, 2), [3, 5])
    np.testing.assert_array_equal(nexus.select_top(keys, 3), [1, 3, 5])
    np.testing.assert_array_equal(nexus.select_top(keys, 6), np.arange(6))
    np.testing.assert_array_equal(nexus.select_top(keys, 10), np.arange(6))
    # -inf positions fill the budget only when nothing else is left.
    np.testing.assert_array_equal(nexus.select_top(keys, 5), [0, 1, 2, 3, 5])


def test_select_matches_brute_force_ranking():
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        keys = rng.choice([-np.inf, -2.0, -1.0, 0.0, np.inf], size=n) if rng.random() < 0.3 \
            else rng.standard_normal(n)
        b = int(rng.integers(1, n + 2))
        ranked = sorted(range(n), key=lambda j: (keys[j], j), reverse=True)
        assert list(nexus.select_top(keys, b)) == sorted(ranked[:b])


def test_scale_invariance_by_powers_of_two():
    rng = np.random.default_rng(1)
    w = rng.random(200) + 1e-3
    u = philox.uniforms(np.arange(200, dtype=np.uint64), 0, 0, 0, 123)
    k1 = nexus.select_top(nexus.reservoir_keys(w, u), 37)
    k2 = nexus.select_top(nexus.reservoir_keys(4.0 * w, u), 37)
    np.testing.assert_array_equal(k1, k2)


@pytest.mark.slow
def test_single_slot_is_proportional_to_weight():
    w = [0.05, 0.1, 0.15, 0.3, 0.4]
    n_draws = 40000
    freq = _frequencies(w, 1, n_draws)
    _assert_within_5_sigma(freq, np.array(w) / sum(w), n_draws)


@pytest.mark.slow
def test_equal_weights_are_uniform_reservoir():
    n_draws = 40000
    freq = _frequencies([0.125] * 8, 3, n_draws, seed=11)
    _assert_within_5_sigma(freq, np.full(8, 3 / 8), n_draws)


@pytest.mark.slow
def test_inclusion_matches_exact_enumeration():
    rng = np.random.default_rng(2)
    n_draws = 40000
    for n, b in ((3, 2), (6, 2), (7, 4)):
        w = rng.random(n) + 0.05
        pi = inclusion_probabilities_float(w, b)
        freq = _frequencies(w, b, n_draws, seed=100 + n)
        _assert_within_5_sigma(freq, pi, n_draws)
        assert np.all(np.diff(np.array(pi)[np.argsort(w)]) > 0)   # monotone in w


@pytest.mark.slow
def test_horvitz_thompson_estimator_is_unbiased():
    """[Nexus] appendix 8.5, Proposition 2 part 1: E[sum_j I_j z_j / p_j] = sum_j z_j."""
    rng = np.random.default_rng(3)
    w = rng.random(6) + 0.1
    z = rng.random(6)
    b = 3
    pi = np.array(inclusion_probabilities_float(w, b))
    n = len(w)
    n_draws = 30000
    steps = np.arange(n_draws, dtype=np.uint64)[:, None]
    u = philox.uniforms(np.arange(n, dtype=np.uint64)[None, :], 5, 0, steps, 99)
    est = np.empty(n_draws)
    for s in range(n_draws):
        keep = nexus.select_top(nexus.reservoir_keys(w, u[s]), b)
        est[s] = np.sum(z[keep] / pi[keep])
    se = est.std() / np.sqrt(n_draws)
    assert abs(est.mean() - z.sum()) < 5 * se


def test_forced_slots_always_survive():
    n = 64
    w = np.linspace(1e-4, 1.0, n)
    for step in range(20):
        u = philox.uniforms(np.arange(n, dtype=np.uint64), 0, 0, step, 5)
        keep = nexus.select_top(nexus.reservoir_keys(w, u, n_sink=3, n_recent=4), 10)
        assert set(range(3)) <= set(keep) and set(range(60, 64)) <= set(keep)
        assert len(keep) == 10
