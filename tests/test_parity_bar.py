"""The GPU tests' end-to-end bar (tests/gpu_common.py) on the CPU: it must
accept exactly what the stated tolerance allows and reject the rest."""

import numpy as np
import pytest

from tests import gpu_common as gc


def _keys(n, seed):
    rng = np.random.default_rng(seed)
    return -rng.exponential(1.0, n) * 1e4          # ln(u)/w-like keys, all negative


def _top(keys, b):
    return np.sort(np.argsort(keys)[::-1][:b])


def test_identical_sets_pass_at_any_budget():
    keys = _keys(500, 1)
    keep = _top(keys, 128)
    gc.assert_kept_matches_oracle(keep, keep, keys, 128)


def test_budget_below_1000_allows_no_flip():
    keys = _keys(4096, 2)
    keep = _top(keys, 819)
    order = np.argsort(keys)[::-1]
    got = np.sort(np.concatenate([np.setdiff1d(keep, [order[818]]), [order[819]]]))
    with pytest.raises(AssertionError, match="shared"):
        gc.assert_kept_matches_oracle(got, keep, keys, 819)


def _boundary_swap(keys, b):
    order = np.argsort(keys)[::-1]
    keep = _top(keys, b)
    got = np.sort(np.concatenate([np.setdiff1d(keep, [order[b - 1]]), [order[b]]]))
    return keep, got, order


def test_boundary_flip_inside_the_band_passes_at_large_budget():
    keys = _keys(40000, 3)
    order = np.argsort(keys)[::-1]
    b = 6554
    # make the boundary pair 1e-4 apart (relative): a 1e-3 weight error can swap it
    keys[order[b]] = keys[order[b - 1]] * (1 + 1e-4)
    keep, got, _ = _boundary_swap(keys, b)
    gc.assert_kept_matches_oracle(got, keep, keys, b)


def test_flip_outside_the_band_fails():
    keys = _keys(40000, 4)
    b = 6554
    order = np.argsort(keys)[::-1]
    x = order[b]
    keys[x] = keys[order[b - 1]] * 1.01               # 1% apart: no 1e-3 weight error swaps them
    keep = _top(keys, b)
    got = np.sort(np.concatenate([np.setdiff1d(keep, [order[b - 1]]), [x]]))
    with pytest.raises(AssertionError, match="band"):
        gc.assert_kept_matches_oracle(got, keep, keys, b)


def test_flip_far_from_the_boundary_fails():
    keys = _keys(40000, 5)
    b = 6554
    keep = _top(keys, b)
    order = np.argsort(keys)[::-1]
    got = np.sort(np.concatenate([np.setdiff1d(keep, [order[10]]), [order[b]]]))
    with pytest.raises(AssertionError, match="band"):
        gc.assert_kept_matches_oracle(got, keep, keys, b)


def test_too_many_flips_fail_even_inside_the_band():
    keys = -np.full(20000, 100.0) * (1 + 1e-7 * np.arange(20000))   # all within the band
    b = 5000
    keep = _top(keys, b)
    got = np.sort(np.concatenate([keep[10:], np.setdiff1d(np.arange(20000), keep)[:10]]))
    with pytest.raises(AssertionError, match="shared"):
        gc.assert_kept_matches_oracle(got, keep, keys, b)


def test_ulp_flips():
    keys = _keys(10000, 6)
    b = 2000
    order = np.argsort(keys)[::-1]
    keys[order[b]] = np.nextafter(keys[order[b - 1]], -np.inf)
    keep, got, _ = _boundary_swap(keys, b)
    gc.assert_flips_within_ulp(got, keep, keys, b, 2)
    with pytest.raises(AssertionError):
        gc.assert_flips_within_ulp(got, keep, keys, b, 0)
    keys[order[b]] = keys[order[b - 1]] * (1 + 1e-9)
    with pytest.raises(AssertionError):
        gc.assert_flips_within_ulp(got, keep, keys, b, 2)
