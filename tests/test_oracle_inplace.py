"""Pins of the in-place compaction layout (streaming, [Nexus] section 2.1).

Facts checked: the first `kept` rows are a permutation of the out-of-place
result; kept rows below `kept` do not move; exactly the kept rows at or past
`kept` move, each into an evicted slot; attention of any query over the
compacted cache equals attention over the ordered one (softmax attention is
invariant under a common permutation of keys and values); a brute-force
enumeration on tiny caches.
"""

import itertools

import numpy as np
import pytest

from oracle import nexus


def _attention(q, k, v):
    logits = q @ k.T / np.sqrt(k.shape[1])
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


def test_layout_is_a_permutation_with_fixed_stayers():
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(1, 60))
        kept = int(rng.integers(1, n + 1))
        keep = np.sort(rng.choice(n, size=kept, replace=False))
        new_pos = nexus.inplace_layout(keep, n)
        assert sorted(new_pos.tolist()) == list(range(kept))
        stay = keep < kept
        np.testing.assert_array_equal(new_pos[stay], keep[stay])
        assert np.all(new_pos[~stay] < kept) and np.all(np.diff(new_pos[~stay]) > 0)


def test_rows_match_out_of_place_and_attention_is_unchanged():
    rng = np.random.default_rng(1)
    n, d, kept, a = 300, 16, 120, 40
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    keep = np.sort(rng.choice(n, size=kept, replace=False))
    app_k = rng.standard_normal((a, d))
    app_v = rng.standard_normal((a, d))
    ck = nexus.compact_inplace(k, keep, app_k)
    cv = nexus.compact_inplace(v, keep, app_v)
    order = np.argsort(nexus.inplace_layout(keep, n))
    np.testing.assert_array_equal(ck[:kept][nexus.inplace_layout(keep, n)], k[keep])
    np.testing.assert_array_equal(ck[kept:kept + a], app_k)
    ordered_k = np.concatenate([k[keep], app_k])
    ordered_v = np.concatenate([v[keep], app_v])
    q = rng.standard_normal((5, d))
    np.testing.assert_allclose(_attention(q, ck[:kept + a], cv[:kept + a]),
                               _attention(q, ordered_k, ordered_v), rtol=1e-12, atol=1e-14)
    assert order.shape == (kept,)


def test_brute_force_tiny():
    """Every keep set of a 6-row cache: the moved rows are exactly the kept rows
    at or past `kept`, and they fill the evicted slots in order."""
    n = 6
    rows = np.arange(n)[:, None] * 10.0
    for kept in range(1, n + 1):
        for keep in itertools.combinations(range(n), kept):
            keep = np.array(keep)
            out = nexus.compact_inplace(rows, keep)
            evicted_low = [i for i in range(kept) if i not in keep]
            movers = [i for i in keep if i >= kept]
            assert len(evicted_low) == len(movers)
            for h, m in zip(evicted_low, movers):
                assert out[h, 0] == rows[m, 0]
            for i in keep:
                if i < kept:
                    assert out[i, 0] == rows[i, 0]


def _block_rows(blocks, b, n):
    return np.concatenate([np.arange(k * b, min(k * b + b, n)) for k in blocks]).astype(np.int64)


@pytest.mark.parametrize("n,b,seed", [(4096, 32, 1), (1088, 32, 2), (100, 32, 3), (4001, 16, 4),
                                      (257, 8, 5)])
def test_block_hole_filling_moves_aligned_blocks_whole(n, b, seed):
    """With blocks the kept rows are the kept blocks' rows; row-level hole
    filling then moves every aligned block whole: each kept block lands as b
    consecutive rows starting at a multiple of b (a short last block, if kept,
    lands on consecutive rows too)."""
    rng = np.random.default_rng(seed)
    nu = -(-n // b)
    blocks = np.sort(rng.choice(nu, size=max(1, nu // 4), replace=False))
    rows = _block_rows(blocks, b, n)
    cache = np.arange(n)[:, None] * 10 + np.arange(3)[None, :]
    out = nexus.compact_inplace(cache, rows)
    kept = len(rows)
    got_rows = out[:kept, 0] // 10                # which original row sits in each slot
    assert sorted(got_rows.tolist()) == rows.tolist()
    full = [k for k in blocks if k * b + b <= n]
    for k in full:
        pos = np.flatnonzero(got_rows == k * b)
        assert len(pos) == 1
        p = int(pos[0])
        if kept % b == 0:
            assert p % b == 0, "an aligned block must land on a block boundary"
        np.testing.assert_array_equal(got_rows[p:p + b], np.arange(k * b, k * b + b))
