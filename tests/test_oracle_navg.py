"""Pins of the oracle's n-averaged reservoir priority and its deterministic limit.

[Nexus] section 2.3, Eq. (6): pi_j = (1/n) sum_i u_ji^(1/w_j), keep the top B by
pi; appendix 8.2: E[u^(1/w)] = w/(w+1) (unbiasedness, Lemma 2), the average of
n draws concentrates (Lemma 3: variance / n), pi is monotone in w, and as
n -> infinity the ranking becomes top-B by w.  Every check below is a fact of
the definition or of the mathematics, not a re-typing of the oracle's formula.
"""

import numpy as np
import pytest

from oracle import nexus, philox


def _pi(w, u):
    """The priority itself from the oracle's log-domain key."""
    return np.exp(nexus.reservoir_keys(w, u))


def test_one_draw_equals_the_single_draw_key():
    j = np.arange(5000, dtype=np.uint64)
    u1 = philox.uniforms(j, 3, 7, 11, 99)
    un = philox.uniforms_n(j, 3, 7, 11, 99, 1)
    np.testing.assert_array_equal(un[:, 0], u1)
    w = np.linspace(1e-4, 1.0, 5000)
    np.testing.assert_array_equal(nexus.reservoir_keys(w, un), nexus.reservoir_keys(w, u1))
    # Draw 0 of any n is the single-draw uniform; draw 1 is another stream.
    u5 = philox.uniforms_n(j, 3, 7, 11, 99, 5)
    np.testing.assert_array_equal(u5[:, 0], u1)
    assert np.mean(u5[:, 1] == u1) < 1e-3


def test_draws_come_from_independent_blocks():
    """Draws are uniform on (0, 1] and pairwise uncorrelated (n = 6: three blocks)."""
    j = np.arange(200000, dtype=np.uint64)
    u = philox.uniforms_n(j, 1, 2, 3, 2024, 6)
    assert u.min() > 0 and u.max() <= 1
    means = u.mean(axis=0)
    assert np.all(np.abs(means - 0.5) < 5 * np.sqrt(1 / 12 / len(j)))
    c = np.corrcoef(u.T)
    off = c[~np.eye(6, dtype=bool)]
    assert np.all(np.abs(off) < 5 / np.sqrt(len(j)))


@pytest.mark.parametrize("w", [0.05, 0.5, 2.0])
@pytest.mark.parametrize("n", [1, 5])
def test_priority_is_unbiased_with_variance_over_n(w, n):
    """E[pi] = w/(w+1) (Lemma 2) and Var[pi] = Var[u^(1/w)]/n (Lemma 3)."""
    m = 200000
    j = np.arange(m, dtype=np.uint64)
    u = philox.uniforms_n(j, 5, 0, 1, 7, n) if n > 1 else philox.uniforms(j, 5, 0, 1, 7)
    pi = _pi(np.full(m, w), u)
    mean = w / (w + 1)
    var1 = w / (w + 2) - mean ** 2          # E[u^(2/w)] - E[u^(1/w)]^2
    var = var1 / n
    assert abs(pi.mean() - mean) < 5 * np.sqrt(var / m)
    # Sample variance within 5 standard errors (fourth moment of a bounded variable).
    assert abs(pi.var() - var) < 0.05 * var + 5 * np.sqrt(2 / m) * var


@pytest.mark.parametrize("n", [1, 3, 5])
def test_priority_is_monotone_in_the_weight(n):
    j = np.arange(20000, dtype=np.uint64)
    u = philox.uniforms_n(j, 2, 4, 6, 8, n)
    w_lo = np.full(len(j), 0.01)
    for w_hi in (0.0100001, 0.02, 0.5):
        assert np.all(nexus.reservoir_keys(np.full(len(j), w_hi), u) >= nexus.reservoir_keys(w_lo, u))


def test_large_n_recovers_top_b_by_weight():
    """n -> infinity: the kept set becomes the B largest weights (appendix 8.2)."""
    w = np.array([0.11, 0.32, 0.05, 0.27, 0.18, 0.39, 0.08, 0.23])
    j = np.arange(len(w), dtype=np.uint64)
    for seed in range(5):
        u = philox.uniforms_n(j, 0, 0, seed, 123, 20000)
        keep = nexus.select_top(nexus.reservoir_keys(w, u), 4)
        np.testing.assert_array_equal(keep, np.sort(np.argsort(w)[-4:]))


def test_n1_is_not_top_b_by_weight():
    """The same weights with one draw do not always give the top-B set (it samples)."""
    w = np.array([0.11, 0.32, 0.05, 0.27, 0.18, 0.39, 0.08, 0.23])
    j = np.arange(len(w), dtype=np.uint64)
    top = np.sort(np.argsort(w)[-4:])
    sets = [nexus.select_top(nexus.reservoir_keys(w, philox.uniforms(j, 0, 0, s, 123)), 4)
            for s in range(40)]
    assert any(not np.array_equal(k, top) for k in sets)


def test_deterministic_limit_is_top_b_by_weight_with_ties_to_the_newer():
    rng = np.random.default_rng(4)
    for _ in range(50):
        n = int(rng.integers(2, 40))
        w = rng.choice([0.1, 0.2, 0.3, 0.0, -1.0], size=n)
        b = int(rng.integers(1, n + 1))
        keep = nexus.select_top(nexus.topk_keys(w), b)
        # Brute force: order by weight (w <= 0 lowest, all equal), ties by larger index.
        eff = np.where(w > 0, w, -np.inf)
        order = sorted(range(n), key=lambda i: (eff[i], i), reverse=True)
        np.testing.assert_array_equal(keep, np.sort(order[:b]))


def test_head_keys_modes():
    w = np.linspace(0.001, 0.01, 300)
    k1 = nexus.head_keys(w, 300, 1, 2, 3, 4, 1)
    np.testing.assert_array_equal(k1, nexus.head_keys(w, 300, 1, 2, 3, 4, 0))
    u = nexus.unit_uniforms(300, 1, 2, 3, 4)
    np.testing.assert_array_equal(k1, np.log(u) / w)
    np.testing.assert_array_equal(nexus.head_keys(w, 300, 1, 2, 3, 4, -1), w)
    k5 = nexus.head_keys(w, 300, 1, 2, 3, 4, 5, n_sink=2, n_recent=3)
    assert np.all(np.isinf(k5[:2])) and np.all(np.isinf(k5[-3:]))
    assert np.all(np.isfinite(k5[2:-3])) and np.all(k5[2:-3] <= 0)
    with pytest.raises(ValueError):
        nexus.head_keys(w, 300, 1, 2, 3, 4, -2)
