"""Pins of the oracle's scoring stages (CPU).

Each test checks the oracle against something other than itself: the
hand-computed caches in tests/golden/tiny_caches.json, closed forms, the walk's
rank-1 decomposition ([Nexus] appendix 8.6), scipy's softmax, and invariances
that the definitions imply.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

from oracle import nexus

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_caches.json")


def _fr(xs):
    return np.array([float(Fraction(x)) for x in xs])


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_tiny_caches(golden):
    lam = float(Fraction(golden["lambda"]))
    eps = float(Fraction(golden["eps_tie"]))
    for case in golden["cases"]:
        q = np.array(case["q"], dtype=np.float64)          # [G, W, D]
        k = np.array(case["k"], dtype=np.float64)          # [N, D]
        P = nexus.window_rows(q, k)
        a = nexus.direct_score(P)
        np.testing.assert_allclose(a, _fr(case["a"]), rtol=0, atol=1e-15, err_msg=case["name"])
        for h, exp in case["by_walk_iters"].items():
            sc = nexus.head_weights(q, k, int(h), lam=lam, eps=eps)
            np.testing.assert_allclose(sc["c"], _fr(exp["c"]), rtol=0, atol=1e-15,
                                       err_msg=f'{case["name"]} H={h}')
            np.testing.assert_allclose(sc["s"], _fr(exp["s"]), rtol=0, atol=1e-15)
            n = k.shape[0]
            ramp = np.arange(n) / (n - 1)
            np.testing.assert_allclose(sc["w"], _fr(exp["s"]) + eps * ramp, rtol=0, atol=1e-15)


def test_golden_walk_order_matters(golden):
    """Feeding the rows newest-first gives the other, rejected, answer."""
    case = golden["cases"][0]
    P = nexus.window_rows(np.array(case["q"]), np.array(case["k"]))
    rev = nexus.nexus_walk(P[::-1].copy(), 2)
    np.testing.assert_allclose(rev, _fr(case["reversed_walk_order_c_H2"]), atol=1e-15)
    fwd = nexus.nexus_walk(P, 2)
    assert not np.allclose(fwd, rev)


def test_golden_gqa_mapping(golden):
    g = golden["gqa_mapping"]
    k = np.array(g["k"], dtype=np.float64)                  # [H_kv, N, D]
    v = np.zeros_like(k)
    for var in g["variants"]:
        q = np.array(var["q"], dtype=np.float64)            # [H_q, W, D]
        out = nexus.evict_step(q, k, v, budget=2, walk_iters=0, seed=0, dtype="f64")
        for h in range(g["H_kv"]):
            s = out["w"][h] - 1e-6 * np.arange(2)
            np.testing.assert_allclose(s, _fr(var["a"][h]), atol=1e-15)


def test_direct_score_sums_to_one_and_uniform_for_zero_queries():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 8, 16))
    k = rng.standard_normal((300, 16)) * 2
    a = nexus.direct_score(nexus.window_rows(q, k))
    assert abs(a.sum() - 1.0) < 1e-13
    a0 = nexus.direct_score(nexus.window_rows(np.zeros((2, 5, 16)), k))
    np.testing.assert_allclose(a0, np.full(300, 1 / 300), rtol=1e-14)


def test_window_rows_match_scipy_softmax():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 6, 32))
    k = rng.standard_normal((77, 32)) * 3
    logits = np.einsum("gwd,nd->gwn", q, k) / np.sqrt(32)
    ref = scipy_softmax(logits, axis=-1).mean(axis=0)
    np.testing.assert_allclose(nexus.window_rows(q, k), ref, rtol=1e-13, atol=1e-300)


def test_mha_group_of_one_equals_plain_softmax_rows():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((20, 8))
    P = nexus.window_rows(q, k)
    for w in range(4):
        x = k @ q[0, w] / np.sqrt(8)
        e = np.exp(x - x.max())
        np.testing.assert_allclose(P[w], e / e.sum(), rtol=1e-14)


def test_permuting_keys_permutes_scores():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 8, 16))
    k = rng.standard_normal((50, 16))
    perm = rng.permutation(50)
    s1 = nexus.head_weights(q, k, 3)
    s2 = nexus.head_weights(q, k[perm], 3)
    np.testing.assert_allclose(s2["a"], s1["a"][perm], rtol=1e-13)
    np.testing.assert_allclose(s2["c"], s1["c"][perm], rtol=1e-13)


def _walk_by_gram(rows):
    """Closed form of Eq. (4) through the Gram matrix of the walk rows.

    C = sum_t gamma_t a_t with gamma_1 = 1 and
    gamma_t = 1 + sum_{t' < t} gamma_t' <a_t, a_t'>; ||C||_1 = sum_t gamma_t
    because every row is a distribution.
    """
    G = rows @ rows.T
    gam = np.zeros(len(rows))
    for t in range(len(rows)):
        gam[t] = 1.0 + sum(gam[u] * G[t, u] for u in range(t))
    return gam @ rows / gam.sum(), gam


def test_walk_matches_gram_closed_form():
    rng = np.random.default_rng(4)
    P = rng.random((6, 40))
    P /= P.sum(axis=1, keepdims=True)
    for H in range(1, 7):
        expect, _ = _walk_by_gram(P[6 - H:])
        np.testing.assert_allclose(nexus.nexus_walk(P, H), expect, rtol=1e-13)


def test_walk_rank_one_decomposition():
    """[Nexus] appendix 8.6: C^(H) = sum_q a^(q) + sum_q M_q C^(q-1), M_q = a^(q) a^(q)^T."""
    rng = np.random.default_rng(4)
    P = rng.random((6, 40))
    P /= P.sum(axis=1, keepdims=True)
    H = 4
    rows = P[6 - H:]
    # Partial walks C^(q) from the oracle itself (unnormalised via the Gram gammas).
    partial = [np.zeros(40)]
    for q in range(1, H + 1):
        c, gam = _walk_by_gram(rows[:q])
        partial.append(c * gam.sum())
    lhs = partial[H]
    rhs = rows.sum(axis=0) + sum(np.outer(rows[q], rows[q]) @ partial[q] for q in range(H))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-13)
    c_oracle = nexus.nexus_walk(P, H)
    np.testing.assert_allclose(c_oracle, lhs / lhs.sum(), rtol=1e-13)


def test_walk_two_steps_closed_form():
    rng = np.random.default_rng(7)
    P = rng.random((3, 25))
    P /= P.sum(axis=1, keepdims=True)
    a1, a2 = P[1], P[2]
    C = a1 + (1.0 + a1 @ a2) * a2
    np.testing.assert_allclose(nexus.nexus_walk(P, 2), C / C.sum(), rtol=1e-14)


def test_walk_special_cases():
    rng = np.random.default_rng(5)
    P = rng.random((5, 30))
    P /= P.sum(axis=1, keepdims=True)
    np.testing.assert_array_equal(nexus.nexus_walk(P, 0), np.zeros(30))
    np.testing.assert_allclose(nexus.nexus_walk(P, 1), P[-1], rtol=1e-14)
    same = np.tile(P[2], (5, 1))
    np.testing.assert_allclose(nexus.nexus_walk(same, 5), P[2], rtol=1e-13)
    with pytest.raises(ValueError):
        nexus.nexus_walk(P, 6)


def test_zero_walk_reduces_to_direct_attention():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 8, 16))
    k = rng.standard_normal((64, 16))
    sc = nexus.head_weights(q, k, 0)
    np.testing.assert_array_equal(sc["s"], sc["a"])


def test_recency_ramp():
    w = nexus.recency_weights(np.zeros(5), eps=1.0)
    np.testing.assert_allclose(w, [0, 0.25, 0.5, 0.75, 1.0])
    assert nexus.recency_weights(np.array([0.3]))[0] == 0.3


def test_bf16_bits_conversion():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F80], dtype=np.uint16)
    np.testing.assert_array_equal(nexus.bf16_bits_to_f64(bits),
                                  [1.0, -1.0, 3.140625, 0.0, np.inf])
