"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case monkeypatches one oracle function with a plausible slip (a dropped
term, a wrong order or index, a transposed operand) and re-runs the pin that
should catch it; the pin must fail.  Nothing here touches the GPU path.
"""

import numpy as np
import pytest

from oracle import nexus, philox
from oracle.enumerate import inclusion_probabilities_float
from tests import test_oracle_nexus as pins
from tests import test_oracle_reservoir as rpins
from tests import test_oracle_philox as ppins
from tests.test_oracle_philox import rocrand_bin  # noqa: F401  (fixture)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.fixture(scope="module")
def golden():
    import json
    with open(pins.GOLDEN) as f:
        return json.load(f)


def _walk_newest_first(P, walk_iters):
    W, N = P.shape
    C = np.zeros(N)
    for t in range(W - 1, W - walk_iters - 1, -1):
        C = C + (1.0 + P[t] @ C) * P[t]
    return C / np.abs(C).sum() if walk_iters else np.zeros(N)


def _walk_without_gamma(P, walk_iters):
    W, N = P.shape
    C = np.zeros(N)
    for t in range(W - walk_iters, W):
        C = C + P[t]
    return C / np.abs(C).sum() if walk_iters else np.zeros(N)


def _walk_gamma_after_update(P, walk_iters):
    W, N = P.shape
    C = np.zeros(N)
    for t in range(W - walk_iters, W):
        C = C + P[t]
        C = C + (P[t] @ C) * P[t]
    return C / np.abs(C).sum() if walk_iters else np.zeros(N)


def _rows_transposed_operand(q_grp, k):
    d = k.shape[-1]
    logits = np.matmul(q_grp[..., ::-1], k.T) / np.sqrt(d)
    e = np.exp(logits - logits.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).mean(axis=0)


def _rows_no_scale(q_grp, k):
    logits = np.matmul(q_grp, k.T)
    e = np.exp(logits - logits.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).mean(axis=0)


def _rows_average_logits(q_grp, k):
    d = k.shape[-1]
    logits = (np.matmul(q_grp, k.T) / np.sqrt(d)).mean(axis=0)
    e = np.exp(logits - logits.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _ramp_one_based(s, eps=nexus.EPS_TIE_DEFAULT):
    n = s.shape[-1]
    return s + eps * (np.arange(1, n + 1) / max(n - 1, 1))


def _score_no_lambda(a, c, lam=0.5):
    return a + c


@pytest.mark.parametrize("name,target,bad", [
    ("walk newest first", "nexus_walk", _walk_newest_first),
    ("walk without gamma", "nexus_walk", _walk_without_gamma),
    ("gamma after update", "nexus_walk", _walk_gamma_after_update),
    ("transposed operand", "window_rows", _rows_transposed_operand),
    ("missing 1/sqrt(D)", "window_rows", _rows_no_scale),
    ("average logits not probabilities", "window_rows", _rows_average_logits),
    ("one-based ramp", "recency_weights", _ramp_one_based),
    ("lambda dropped", "nexus_score", _score_no_lambda),
])
def test_golden_catches_scoring_slips(monkeypatch, golden, name, target, bad):
    monkeypatch.setattr(nexus, target, bad)
    assert _fails(pins.test_golden_tiny_caches, golden), name


def test_golden_catches_strided_gqa_grouping(monkeypatch, golden):
    real = nexus.evict_step

    def strided(q, k, v, budget, walk_iters, seed, **kw):
        h_kv = k.shape[0]
        g = q.shape[0] // h_kv
        order = np.concatenate([np.arange(h, q.shape[0], h_kv) for h in range(h_kv)])
        assert g * h_kv == q.shape[0]
        return real(q[order], k, v, budget, walk_iters, seed, **kw)

    monkeypatch.setattr(nexus, "evict_step", strided)
    assert _fails(pins.test_golden_gqa_mapping, golden)


def test_selection_pin_catches_older_first_ties(monkeypatch):
    def older_first(keys, budget):
        n = len(keys)
        if budget >= n:
            return np.arange(n)
        order = np.lexsort((-np.arange(n), keys))
        return np.sort(order[n - budget:])

    monkeypatch.setattr(nexus, "select_top", older_first)
    assert _fails(rpins.test_select_ties_prefer_newer_and_output_ascending)


def test_law_pin_catches_multiplied_key(monkeypatch):
    """ln(u) * w instead of ln(u) / w draws the wrong law."""
    def bad_keys(w, u, n_sink=0, n_recent=0):
        return np.log(u) * w

    monkeypatch.setattr(nexus, "reservoir_keys", bad_keys)
    w = np.array([0.1, 0.2, 0.3, 0.4])
    freq = rpins._frequencies(w, 2, 4000)
    pi = np.array(inclusion_probabilities_float(w, 2))
    assert _fails(rpins._assert_within_5_sigma, freq, pi, 4000)


def test_law_pin_catches_top_k_by_weight(monkeypatch):
    """Deterministic top-K ignores u: every draw keeps the same set."""
    def topk_keys(w, u, n_sink=0, n_recent=0):
        return np.asarray(w, dtype=np.float64)

    monkeypatch.setattr(nexus, "reservoir_keys", topk_keys)
    w = np.array([0.1, 0.2, 0.3, 0.4])
    freq = rpins._frequencies(w, 2, 2000)
    pi = np.array(inclusion_probabilities_float(w, 2))
    assert _fails(rpins._assert_within_5_sigma, freq, pi, 2000)


def test_philox_pin_catches_missing_key_bump(monkeypatch, rocrand_bin):  # noqa: F811
    def no_bump(c0, c1, c2, c3, k0, k1):
        x0, x1, x2, x3 = (philox._u32(c) for c in (c0, c1, c2, c3))
        x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
        ka, kb = philox._u32(k0), philox._u32(k1)
        for _ in range(10):
            p0, p1 = philox.M0 * x0, philox.M1 * x2
            x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ ka, p1 & philox.MASK32,
                              (p0 >> np.uint64(32)) ^ x3 ^ kb, p0 & philox.MASK32)
        return x0, x1, x2, x3

    monkeypatch.setattr(philox, "philox4x32_10", no_bump)
    assert _fails(ppins.test_matches_rocrand_on_the_token_counter_layout, rocrand_bin)


# --------------------------------------------------- n-averaged priority ----

from tests import test_oracle_navg as npins  # noqa: E402

_real_reservoir_keys = nexus.reservoir_keys
_real_uniforms_n = philox.uniforms_n


def _keys_without_log_n(w, u, n_sink=0, n_recent=0):
    """Slip: the 1/n of Eq. (6) dropped (ln pi off by ln n)."""
    keys = _real_reservoir_keys(w, u, n_sink, n_recent)
    u = np.asarray(u)
    return keys + (np.log(u.shape[1]) if u.ndim == 2 else 0.0)


def _keys_geometric_mean(w, u, n_sink=0, n_recent=0):
    """Slip: averaging the logs, (1/n) sum ln(u)/w, instead of the log of the average."""
    u = np.asarray(u, dtype=np.float64)
    if u.ndim == 1:
        return _real_reservoir_keys(w, u, n_sink, n_recent)
    return _real_reservoir_keys(w, np.exp(np.log(u).mean(axis=1)), n_sink, n_recent)


def _uniforms_n_one_block(token, unit_id, layer, step, seed, n):
    """Slip: every pair of draws from the same Philox block (no per-block key)."""
    one = _real_uniforms_n(token, unit_id, layer, step, seed, 2)
    return np.concatenate([one] * ((n + 1) // 2), axis=-1)[..., :n]


@pytest.mark.parametrize("slip, pin, args", [
    (_keys_without_log_n, npins.test_priority_is_unbiased_with_variance_over_n, (0.5, 5)),
    (_keys_geometric_mean, npins.test_priority_is_unbiased_with_variance_over_n, (0.5, 5)),
])
def test_navg_key_slips_are_caught(monkeypatch, slip, pin, args):
    monkeypatch.setattr(nexus, "reservoir_keys", slip)
    assert _fails(pin, *args)


def test_navg_shared_block_slip_is_caught(monkeypatch):
    monkeypatch.setattr(philox, "uniforms_n", _uniforms_n_one_block)
    assert _fails(npins.test_draws_come_from_independent_blocks)


# ------------------------------------------------------ block granularity ----

from tests import test_oracle_blocks as bpins  # noqa: E402

_real_block_rows = nexus.block_rows


def _block_rows_shifted(P, block):
    """Slip: token j assigned to block (j + 1) // b."""
    P = np.asarray(P, dtype=np.float64)
    return _real_block_rows(np.concatenate([np.zeros((P.shape[0], 1)), P], axis=1)[:, :-1] +
                            np.concatenate([P[:, -1:] * 0, np.zeros((P.shape[0], P.shape[1] - 1))],
                                           axis=1), block)


def _block_rows_no_partial(P, block):
    """Slip: the shorter last block dropped (floor instead of ceil)."""
    P = np.asarray(P, dtype=np.float64)
    nk = P.shape[1] // block
    S = P[:, :nk * block].reshape(P.shape[0], nk, block).sum(axis=2)
    return S / S.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("slip", [_block_rows_shifted, _block_rows_no_partial])
def test_block_slips_are_caught(monkeypatch, golden, slip):
    monkeypatch.setattr(nexus, "block_rows", slip)
    with open(bpins.GOLDEN) as f:
        import json
        g = json.load(f)
    assert _fails(bpins.test_golden_blocks, g)
