"""Pins of the oracle's block granularity ([Nexus] section 2.1, Eq. (1) with b > 1).

Checked against: hand-derived fractions (tests/golden/tiny_blocks.json, with a
ragged last block), the sum rule stated with Eq. (1) (sum_j a_j = 1), b = 1
giving the token path bit for bit, one block covering the cache, an explicit
loop over blocks on tiny inputs, and the kept rows being whole blocks.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nexus

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_blocks.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _f(x):
    return float(Fraction(x))


def test_golden_blocks(golden):
    lam, eps = _f(golden["lambda"]), _f(golden["eps_tie"])
    for case in golden["cases"]:
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        b = case["block"]
        for h, exp in case["by_walk_iters"].items():
            sc = nexus.head_weights(q, k, int(h), lam, eps, block=b)
            np.testing.assert_allclose(sc["a"], [_f(x) for x in case["a"]], rtol=1e-13)
            np.testing.assert_allclose(sc["c"], [_f(x) for x in exp["c"]], rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(sc["s"], [_f(x) for x in exp["s"]], rtol=1e-13)
            nk = len(case["a"])
            r = np.arange(nk) / (nk - 1)
            np.testing.assert_allclose(sc["w"], np.array([_f(x) for x in exp["s"]]) + eps * r,
                                       rtol=1e-13)


def _case(seed, n, W=6, G=2, D=8):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((G, W, D)), rng.standard_normal((n, D)) * 1.5


@pytest.mark.parametrize("n,b", [(64, 8), (70, 8), (33, 32), (5, 2), (100, 7)])
def test_direct_score_over_blocks_sums_to_one(n, b):
    q, k = _case(n * b, n)
    for h in (0, 2, 4):
        sc = nexus.head_weights(q, k, h, block=b)
        assert sc["a"].shape == (-(-n // b),)
        assert abs(sc["a"].sum() - 1) < 1e-12
        if h:
            assert abs(sc["c"].sum() - 1) < 1e-12


def test_block_of_one_is_the_token_path():
    q, k = _case(1, 50)
    for h in (0, 3):
        a = nexus.head_weights(q, k, h)
        b = nexus.head_weights(q, k, h, block=1)
        for key in ("a", "c", "s", "w"):
            np.testing.assert_array_equal(a[key], b[key])


def test_one_block_covers_the_cache():
    q, k = _case(2, 40)
    sc = nexus.head_weights(q, k, 2, block=64)
    np.testing.assert_allclose(sc["a"], [1.0])
    np.testing.assert_allclose(sc["c"], [1.0])
    np.testing.assert_allclose(sc["w"], [1.5])   # s = a + c/2; one block: r = 0


def test_blocks_match_an_explicit_loop():
    """Block rows summed token by token in plain Python, then the same walk."""
    q, k = _case(3, 23, W=4, G=3, D=4)
    b, H = 5, 3
    P = nexus.window_rows(q, k)                  # token rows, [W, N]
    W, N = P.shape
    nk = (N + b - 1) // b
    S = [[0.0] * nk for _ in range(W)]
    for w in range(W):
        for j in range(N):
            S[w][j // b] += P[w, j]
        tot = sum(S[w])
        S[w] = [x / tot for x in S[w]]
    a = [sum(S[w][t] for w in range(W)) / W for t in range(nk)]
    C = [0.0] * nk
    for w in range(W - H, W):
        gamma = 1.0 + sum(S[w][t] * C[t] for t in range(nk))
        C = [C[t] + gamma * S[w][t] for t in range(nk)]
    c = [x / sum(C) for x in C]
    sc = nexus.head_weights(q, k, H, block=b)
    np.testing.assert_allclose(sc["a"], a, rtol=1e-12)
    np.testing.assert_allclose(sc["c"], c, rtol=1e-12)


def test_evict_step_keeps_whole_blocks():
    rng = np.random.default_rng(9)
    n, b, budget = 77, 8, 4                  # 10 blocks, the last of 5 tokens
    q = rng.standard_normal((4, 6, 16)).astype(np.float32)
    k = rng.standard_normal((2, n, 16)).astype(np.float32)
    v = rng.standard_normal((2, n, 16)).astype(np.float32)
    out = nexus.evict_step(q, k, v, budget, 3, 5, dtype="f32", block=b)
    for h in range(2):
        keep = out["keep"][h]
        assert len(keep) == budget and np.all(np.diff(keep) > 0) and keep.max() < 10
        rows = np.concatenate([np.arange(x * b, min(x * b + b, n)) for x in keep])
        np.testing.assert_array_equal(out["out_k"][h], k[h][rows])
        np.testing.assert_array_equal(out["out_v"][h], v[h][rows])
        assert out["w"][h].shape == (10,)
    # b = 1 is the token path.
    t = nexus.evict_step(q, k, v, 20, 3, 5, dtype="f32")
    t1 = nexus.evict_step(q, k, v, 20, 3, 5, dtype="f32", block=1)
    for h in range(2):
        np.testing.assert_array_equal(t["keep"][h], t1["keep"][h])
