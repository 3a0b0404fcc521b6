"""Pins of the oracle's per-head budgets ([Nexus] appendix 10: a layer budget
redistributed over the heads; allocation rule of the cited Ada-KV: a top-K
over the weights of all heads together, with a per-head floor).

Every check is a property of that allocation or a hand-computed case, not a
re-typing of the oracle.
"""

import numpy as np
import pytest

from oracle import nexus


def test_hand_computed_concentrated_and_spread_heads():
    # Head 0: five units at 0.2 and 95 at 1e-4; head 1: 100 units at 0.01.
    # B = 20, floor 0: the 40 largest are head 0's five, then 35 of head 1's.
    w = np.vstack([np.r_[np.full(5, 0.2), np.full(95, 1e-4)], np.full(100, 0.01)])
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 20, 0, cap=100), [5, 35])
    # Floor 4: K = 2 * 16 = 32 -> head 0 gets its five, head 1 gets 27; plus 4 each.
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 20, 4, cap=100), [9, 31])
    # Capacity 30 cuts head 1.
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 20, 4, cap=30), [9, 30])


@pytest.mark.parametrize("h,n,b,f", [(4, 50, 10, 0), (8, 33, 7, 2), (3, 20, 20, 5)])
def test_identical_heads_get_the_uniform_budget(h, n, b, f):
    rng = np.random.default_rng(1)
    row = rng.random(n)
    w = np.tile(row, (h, 1))
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, b, f), np.full(h, min(b, n)))


def test_floor_equal_to_the_budget_is_uniform():
    rng = np.random.default_rng(2)
    w = rng.random((6, 40)) ** 3
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 9, 9), np.full(6, 9))
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 9, 50), np.full(6, 9))


def test_a_dominant_head_takes_the_flexible_part():
    rng = np.random.default_rng(3)
    w = rng.random((4, 30)) * 0.1
    w[2] += 1.0                                     # every unit of head 2 beats all others
    got = nexus.ada_head_budgets(w, 6, 2, cap=30)
    k = 4 * (6 - 2)
    np.testing.assert_array_equal(got, [2, 2, min(2 + k, 30), 2])


def test_budgets_sum_to_the_layer_budget_and_respect_floor_and_caps():
    rng = np.random.default_rng(4)
    for _ in range(200):
        h = int(rng.integers(1, 9))
        n = int(rng.integers(1, 60))
        b = int(rng.integers(1, 70))
        f = int(rng.integers(0, b + 1))
        w = rng.exponential(size=(h, n)) ** rng.uniform(0.2, 4)
        got = nexus.ada_head_budgets(w, b, f, cap=n)
        bbar = min(b, n)
        # f + c_h sums to H * Bbar; only a head whose share would pass its N
        # units loses the excess.
        assert got.sum() <= h * bbar
        if np.all(got < n):
            assert got.sum() == h * bbar
        assert np.all(got >= min(f, bbar)) and np.all(got <= n)


def test_scale_invariance_and_monotonicity():
    rng = np.random.default_rng(5)
    for _ in range(100):
        h, n = 5, 25
        w = rng.exponential(size=(h, n)) ** 2
        b, f = int(rng.integers(1, 25)), int(rng.integers(0, 5))
        base = nexus.ada_head_budgets(w, b, f, cap=n)
        np.testing.assert_array_equal(nexus.ada_head_budgets(w * 7.5, b, f, cap=n), base)
        j = int(rng.integers(0, h))
        w2 = w.copy()
        w2[j] *= 1.5
        assert nexus.ada_head_budgets(w2, b, f, cap=n)[j] >= base[j]


def test_brute_force_with_ties_and_nonpositive_weights():
    """Against a list sorted by Python's sort: (weight or 0) descending, head ascending."""
    rng = np.random.default_rng(6)
    for _ in range(300):
        h = int(rng.integers(1, 6))
        n = int(rng.integers(1, 12))
        w = rng.choice([0.5, 0.25, 0.125, 0.0, -1.0], size=(h, n))
        b = int(rng.integers(1, 14))
        f = int(rng.integers(0, b + 1))
        cap = int(rng.integers(1, 20))
        items = sorted(((max(w[i, j], 0.0), i) for i in range(h) for j in range(n)),
                       key=lambda t: (-t[0], t[1]))
        bbar = min(b, n)
        ff = min(f, bbar)
        k = h * (bbar - ff)
        c = np.zeros(h, dtype=int)
        for _, i in items[:k]:
            c[i] += 1
        want = np.minimum(np.minimum(ff + c, cap), n)
        np.testing.assert_array_equal(nexus.ada_head_budgets(w, b, f, cap=cap), want)


def test_evict_step_with_head_budgets():
    rng = np.random.default_rng(7)
    h_q, h_kv, W, d, n = 8, 4, 4, 16, 64
    q = rng.standard_normal((h_q, W, d)).astype(np.float32)
    k = rng.standard_normal((h_kv, n, d)).astype(np.float32)
    v = rng.standard_normal((h_kv, n, d)).astype(np.float32)
    uni = nexus.evict_step(q, k, v, 16, 2, 9, dtype="f32")
    same = nexus.evict_step(q, k, v, 16, 2, 9, dtype="f32", head_budgets=[16] * 4)
    for h in range(h_kv):
        np.testing.assert_array_equal(uni["keep"][h], same["keep"][h])
    given = nexus.evict_step(q, k, v, 16, 2, 9, dtype="f32", head_budgets=[3, 16, 9, 1])
    for h, bh in enumerate([3, 16, 9, 1]):
        assert len(given["keep"][h]) == bh and given["out_k"][h].shape == (bh, d)
    ada = nexus.evict_step(q, k, v, 16, 2, 9, dtype="f32", ada_floor=4, head_cap=40)
    w = np.stack([ada["w"][h] for h in range(h_kv)])
    want = nexus.ada_head_budgets(w, 16, 4, cap=40)
    assert [ada["budgets"][h] for h in range(h_kv)] == list(want)
    assert sum(want) == h_kv * 16
    # The kept set of each head is the selection on its keys with its own budget.
    for h in range(h_kv):
        np.testing.assert_array_equal(ada["keep"][h], nexus.select_top(ada["keys"][h], want[h]))


def test_hand_computed_ragged_heads():
    # After earlier per-head budgets the heads hold different unit counts:
    # head 0 has 2 units, head 1 has 4.  Bbar = min(budget, 4).
    w = [np.array([0.5, 0.1]), np.array([0.4, 0.3, 0.2, 0.05])]
    # B = 2, floor 0: K = 4 -> 0.5 (h0), 0.4, 0.3, 0.2 (h1).
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 2, 0, cap=10), [1, 3])
    # Floor 1: K = 2 -> 0.5 (h0), 0.4 (h1); plus 1 each.
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 2, 1, cap=10), [2, 2])
    # B = 3: K = 6 = all units -> every head keeps everything.
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 3, 0, cap=10), [2, 4])
    # Capacity 3 cuts head 1.
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 3, 0, cap=3), [2, 3])
    # B = 4, floor 3: K = 2 -> 0.5 (h0), 0.4 (h1); head 0's 3 + 1 is cut to its 2 units.
    np.testing.assert_array_equal(nexus.ada_head_budgets(w, 4, 3, cap=10), [2, 4])


def test_brute_force_ragged_heads():
    """Ragged heads against Python's sort: (weight or 0) descending, head ascending."""
    rng = np.random.default_rng(8)
    for _ in range(300):
        h = int(rng.integers(1, 6))
        ns = rng.integers(1, 12, size=h)
        w = [rng.choice([0.5, 0.25, 0.125, 0.0, -1.0], size=int(m)) for m in ns]
        b = int(rng.integers(1, 14))
        f = int(rng.integers(0, b + 1))
        cap = int(rng.integers(1, 20))
        items = sorted(((max(w[i][j], 0.0), i) for i in range(h) for j in range(ns[i])),
                       key=lambda t: (-t[0], t[1]))
        bbar = min(b, int(ns.max()))
        ff = min(f, bbar)
        k = h * (bbar - ff)
        c = np.zeros(h, dtype=int)
        for _, i in items[:k]:
            c[i] += 1
        want = np.minimum(np.minimum(ff + c, cap), ns)
        np.testing.assert_array_equal(nexus.ada_head_budgets(w, b, f, cap=cap), want)


def test_evict_step_ragged_heads_are_independent_but_for_the_budgets():
    """Each ragged head's result is the one-head event on its own rows with the
    same Philox unit (seq_id' = seq_id * H + h) and its allocated budget."""
    rng = np.random.default_rng(9)
    h_q, h_kv, W, d = 8, 4, 4, 16
    ns = [40, 64, 17, 33]
    q = rng.standard_normal((h_q, W, d)).astype(np.float32)
    k = [rng.standard_normal((m, d)).astype(np.float32) for m in ns]
    v = [rng.standard_normal((m, d)).astype(np.float32) for m in ns]
    out = nexus.evict_step(q, k, v, 16, 2, 9, dtype="f32", layer=3, step=5, seq_id=2,
                           ada_floor=4, head_cap=40)
    want = nexus.ada_head_budgets([out["w"][h] for h in range(h_kv)], 16, 4, cap=40)
    g = h_q // h_kv
    for h in range(h_kv):
        assert out["budgets"][h] == want[h] and len(out["w"][h]) == ns[h]
        one = nexus.evict_step(q[h * g:(h + 1) * g], [k[h]], [v[h]], 16, 2, 9, dtype="f32",
                               layer=3, step=5, seq_id=2 * h_kv + h, head_budgets=[want[h]])
        np.testing.assert_array_equal(out["keep"][h], one["keep"][0])
        np.testing.assert_array_equal(out["out_k"][h], k[h][out["keep"][h]])
        np.testing.assert_array_equal(out["out_v"][h], v[h][out["keep"][h]])
