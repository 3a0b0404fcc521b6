"""Pins of the exact-enumeration law (CPU)."""

from fractions import Fraction as F

from oracle.enumerate import inclusion_probabilities


def test_hand_computed_three_items():
    # Successive sampling by hand: pi_1 = 1/6 + (2/6)(1/4) + (3/6)(1/3) = 5/12, etc.
    assert inclusion_probabilities([1, 2, 3], 2) == [F(5, 12), F(11, 15), F(17, 20)]


def test_single_draw_is_proportional():
    w = [1, 4, 2, 7, 3]
    assert inclusion_probabilities(w, 1) == [F(x, sum(w)) for x in w]


def test_equal_weights_give_budget_over_n():
    for n in range(2, 8):
        for b in range(1, n):
            assert inclusion_probabilities([5] * n, b) == [F(b, n)] * n


def test_sum_is_budget_and_monotone():
    w = [1, 2, 3, 5, 8, 13, 21]
    for b in range(1, 7):
        pi = inclusion_probabilities(w, b)
        assert sum(pi) == b
        assert all(pi[i] < pi[i + 1] for i in range(len(w) - 1))
        assert all(0 < p < 1 for p in pi)
