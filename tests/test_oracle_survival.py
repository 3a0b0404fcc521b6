"""Pins of the oracle's streaming survival law ([Nexus] section 3, appendix 8.3 Lemma 1).

Each check is a fact of successive sampling or of the top-K rule worked out by
hand or by an independent formulation, not a re-typing of the oracle.
"""

from fractions import Fraction as F

import numpy as np
import pytest

from oracle import survival
from oracle.enumerate import inclusion_probabilities


def test_kept_set_law_hand_computed():
    # w = (1, 2, 3), keep 2: P({0,1}) = 1/6*2/5 + 2/6*1/4 = 3/20,
    # P({0,2}) = 1/6*3/5 + 3/6*1/3 = 4/15, P({1,2}) = 2/6*3/4 + 3/6*2/3 = 7/12.
    law = survival.kept_set_law([1, 2, 3], 2)
    assert law == {frozenset({0, 1}): F(3, 20), frozenset({0, 2}): F(4, 15),
                   frozenset({1, 2}): F(7, 12)}


@pytest.mark.parametrize("w,budget", [([1, 2, 3, 4, 5], 3), ([3, 1, 1, 7], 2),
                                      ([2, 9, 4, 1, 6, 5], 4)])
def test_kept_set_law_is_a_law_with_the_known_marginals(w, budget):
    law = survival.kept_set_law(w, budget)
    assert sum(law.values()) == 1
    assert all(len(s) == budget for s in law)
    marg = [sum(p for s, p in law.items() if j in s) for j in range(len(w))]
    assert marg == inclusion_probabilities(w, budget)


def test_kept_set_law_budget_one_is_proportional_to_weight():
    w = [F(1, 3), F(2, 7), F(5, 2), F(1, 9)]
    law = survival.kept_set_law(w, 1)
    for j in range(4):
        assert law[frozenset({j})] == w[j] / sum(w)


def test_equal_weights_survival_is_geometric():
    """Equal weights keep a uniform B-subset of the N residents every event, so
    an initial token survives e events with probability (B/N)^e."""
    n0, budget, app, events = 5, 3, 2, 4
    alive = survival.reservoir_survival_exact(lambda e, j: 1, n0, budget, app, events)
    for e in range(events):
        for j in range(n0):
            assert alive[e][j] == F(budget, n0) ** (e + 1)
        # tokens that arrived at event e' < e survived e - e' events
        for e_arr in range(e):
            for j in range(n0 + e_arr * app, n0 + (e_arr + 1) * app):
                assert alive[e][j] == F(budget, n0) ** (e - e_arr)


def test_one_event_reduces_to_the_marginals():
    w = [F(1), F(4), F(2), F(3)]
    alive = survival.reservoir_survival_exact(lambda e, j: w[j], 4, 2, 1, 1)
    assert [alive[0][j] for j in range(4)] == inclusion_probabilities(w, 2)
    assert alive[0][4] == 1                         # the appended token


def _table(seed, n_ids, events):
    rng = np.random.default_rng(seed)
    # weights on a 1/64 grid, exactly representable in fp32 and fp64
    return rng.integers(1, 64, size=(events, n_ids)) / 64.0


def _topk_by_removal(tab, n0, budget, app, events):
    """Independent formulation: evict the weakest resident one at a time
    (equal weights: the earlier cache position goes first)."""
    res = list(range(n0))
    nxt, out = n0, []
    for e in range(events):
        while len(res) > budget:
            w = [tab[e][j] for j in res]
            m = min(w)
            res.pop(w.index(m))
        res = res + list(range(nxt, nxt + app))
        nxt += app
        out.append(set(res))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_survival_matches_removal_of_the_weakest(seed):
    n0, budget, app, events = 7, 4, 3, 6
    tab = _table(seed, n0 + app * events, events)
    got = survival.topk_survival(lambda e, j: tab[e][j], n0, budget, app, events)
    assert got == _topk_by_removal(tab, n0, budget, app, events)


def test_lemma1_topk_collapses_while_the_reservoir_keeps_positive_mass():
    """Token 0 is the strongest at every event but the first, where it sits just
    under the cutoff: top-K drops it for good; the reservoir keeps it with
    positive probability at every later event."""
    n0, budget, app, events = 4, 3, 1, 4
    w = {0: [F(9, 10)] + [F(10)] * 3}

    def weight_of(e, j):
        return w[j][e] if j in w else F(1)

    top = survival.topk_survival(weight_of, n0, budget, app, events)
    assert all(0 not in s for s in top)             # gone after event 0, never back
    alive = survival.reservoir_survival_exact(weight_of, n0, budget, app, events)
    for e in range(events):
        assert all(p > 0 for p in alive[e].values())
        assert alive[e][0] > 0
    # after the first event, token 0 (weight 10 against 1) is rarely evicted
    assert alive[3][0] / alive[0][0] > F(9, 10) ** 3


def test_monte_carlo_matches_the_exact_law():
    n0, budget, app, events, reps = 4, 3, 1, 3, 20000
    tab = _table(11, n0 + app * events, events)
    exact = survival.reservoir_survival_exact(lambda e, j: F(float(tab[e][j])), n0, budget,
                                              app, events)
    paths = survival.reservoir_survival_mc(lambda e, j: tab[e][j], n0, budget, app, events,
                                           reps, seed=5)
    for e in range(events):
        res = paths[e]
        for j, p in exact[e].items():
            p = float(p)
            freq = np.mean(np.any(res == j, axis=1))
            sigma = np.sqrt(p * (1 - p) / reps)
            assert abs(freq - p) <= 5 * sigma + 1e-12, (e, j, freq, p)
