"""Exact inclusion probabilities of weighted sampling without replacement (test infrastructure).

[Nexus] section 2.3 and appendix 11 take the reservoir priority u^(1/w) of
Efraimidis and Spirakis: keeping the K largest priorities draws a sample with
the same law as successive sampling, where each next item is picked with
probability proportional to its weight among the items not yet picked.  This
module computes that law by brute force, independently of keys, uniforms and
sorting: it enumerates the ordered K-prefixes of successive draws.

Pure Python loops; meant for N <= 8.  With integer or Fraction weights the
result is exact (fractions.Fraction).

Pinned by the hand-computed case w = (1, 2, 3), K = 2 -> (5/12, 11/15, 17/20),
by K = 1 -> w_j / sum(w), by equal weights -> K/N, and by sum_j pi_j = K
(tests/test_oracle_enumerate.py).
"""

from fractions import Fraction
from itertools import permutations


def inclusion_probabilities(weights, budget):
    """pi_j = P(item j is among the first `budget` successive draws)."""
    w = [x if isinstance(x, Fraction) else Fraction(x) for x in weights]
    n = len(w)
    if n > 8:
        raise ValueError("enumeration is meant for N <= 8")
    if budget >= n:
        return [Fraction(1)] * n
    total = sum(w)
    pi = [Fraction(0)] * n
    for prefix in permutations(range(n), budget):
        p = Fraction(1)
        remaining = total
        for i in prefix:
            p *= w[i] / remaining
            remaining -= w[i]
        for i in prefix:
            pi[i] += p
    return pi


def inclusion_probabilities_float(weights, budget):
    """Same law for float weights (computed with exact rationals of the floats)."""
    return [float(x) for x in inclusion_probabilities(
        [Fraction(float(x)) for x in weights], budget)]
