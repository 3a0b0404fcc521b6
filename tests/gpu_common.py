"""Helpers for the GPU parity tests: move GPU inputs to the oracle, compare.

The oracle only ever sees host copies of the exact tensors the HIP path
consumed; no expected value is taken from the HIP path except where a test
explicitly runs the oracle's selection on the GPU's own weights.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import nexus
from workloads import bf16_bits

# Tolerance on Nexus weights: fp32 accumulation over bf16 inputs against the
# fp64 oracle (relative 1e-3, absolute floor for exp underflow).
W_RTOL = 1e-3
W_ATOL = 1e-30


def host(t):
    """(array, dtype tag) for the oracle: raw bf16 bits or fp32 values."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t), "bf16"
    return t.detach().cpu().numpy(), "f32"


def oracle_weights(q, k, n_tokens, walk, group, heads=None, lam=0.5, eps=1e-6):
    """Oracle w for KV heads `heads` of one item; q [H_q, W, D], k [H_kv, >=N, D]."""
    qh, dt = host(q)
    kh, _ = host(k[:, :n_tokens])
    heads = range(kh.shape[0]) if heads is None else heads
    out = {}
    for h in heads:
        qg = nexus.as_f64(qh[h * group:(h + 1) * group], dt)
        kk = nexus.as_f64(kh[h], dt)
        out[h] = nexus.head_weights(qg, kk, walk, lam, eps)["w"]
    return out


def assert_weights_close(w_gpu, w_ref, what=""):
    w_gpu = np.asarray(w_gpu, dtype=np.float64)
    err = np.abs(w_gpu - w_ref)
    tol = W_RTOL * np.abs(w_ref) + W_ATOL
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} weights off; worst rel "
                           f"{np.max(err / np.maximum(np.abs(w_ref), 1e-300)):.3e}")


# Relative key band implied by the weight tolerance: with |w' - w| <= 1e-3 |w|
# the key ln(u)/w' lies within a factor (1 +- 1e-3)^-1 of ln(u)/w, so two keys
# can swap order only when they are within a factor 1 + KEY_DELTA of each other.
KEY_DELTA = (1 + W_RTOL) / (1 - W_RTOL) - 1


def assert_kept_matches_oracle(got, ref_keep, ref_keys, kept, what="", n_avg=1):
    """End-to-end bar against the pure oracle for one head unit.

    At least ceil(0.999 * kept) indices shared (every index when kept < 1000);
    and every index in the symmetric difference must be a boundary token: its
    oracle key lies inside the band where a 1e-3 weight error can reorder two
    keys, [max(|t_B|, |t_B+1|) / (1 + d), min(|t_B|, |t_B+1|) * (1 + d)] with
    t_B, t_B+1 the oracle's B-th and (B+1)-th largest keys and d = KEY_DELTA
    (plus 2e-3 ln(n) absolute for the n-averaged key, whose log-sum-exp moves
    by at most ln(n) * 1e-3 beyond the scaling).
    """
    got_s = set(np.asarray(got).tolist())
    ref_s = set(np.asarray(ref_keep).tolist())
    need = math.ceil(0.999 * kept - 1e-9)
    shared = len(got_s & ref_s)
    assert shared >= need, f"{what}: {shared} of {kept} kept indices shared, need {need}"
    flips = sorted(got_s ^ ref_s)
    if not flips:
        return
    keys = np.asarray(ref_keys, dtype=np.float64)
    order = np.lexsort((np.arange(len(keys)), keys))[::-1]   # descending, larger index first
    t_b, t_b1 = keys[order[kept - 1]], keys[order[kept]]
    assert np.isfinite(t_b) and np.isfinite(t_b1), f"{what}: flip at an infinite boundary"
    slack = 2e-3 * math.log(n_avg) if n_avg > 1 else 0.0
    a, b = abs(t_b), abs(t_b1)
    lo = max(a, b) / (1 + KEY_DELTA) - slack
    hi = min(a, b) * (1 + KEY_DELTA) + slack
    for x in flips:
        kx = abs(keys[x])
        assert lo <= kx <= hi, (f"{what}: token {x} flipped with oracle key {keys[x]:.9g}, "
                                f"outside the boundary band [{lo:.9g}, {hi:.9g}]")


def assert_flips_within_ulp(got, ref_keep, ref_keys, kept, maxulp, what=""):
    """Selection on given weights against the oracle's own keys: the GPU's keys
    differ from the oracle's only by the last-place differences of the device's
    log (maxulp), so the kept sets may differ only by tokens whose oracle keys
    lie within 2 * maxulp ulp of the boundary key."""
    got_s = set(np.asarray(got).tolist())
    ref_s = set(np.asarray(ref_keep).tolist())
    flips = sorted(got_s ^ ref_s)
    if not flips:
        return
    assert maxulp > 0, f"{what}: {len(flips)} flipped tokens where the keys are exact"
    keys = np.asarray(ref_keys, dtype=np.float64)
    order = np.lexsort((np.arange(len(keys)), keys))[::-1]
    t_b = keys[order[kept - 1]]
    assert np.isfinite(t_b), f"{what}: flip at an infinite boundary"
    tol = 2 * maxulp * np.spacing(abs(t_b))
    for x in flips:
        assert abs(keys[x] - t_b) <= tol, (f"{what}: token {x} flipped, oracle key {keys[x]!r} "
                                           f"vs boundary {t_b!r}")


def oracle_map(fn, jobs, workers=None):
    """fn over jobs in threads (numpy and BLAS release the GIL), one BLAS thread
    each; results in job order."""
    from threadpoolctl import threadpool_limits
    workers = workers or min(16, os.cpu_count() or 1)
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, jobs))


def check_keep_valid(keep, n_tokens, budget):
    keep = np.asarray(keep)
    kept = min(budget, n_tokens)
    assert keep.shape[-1] >= kept
    k = keep[:kept]
    assert np.all(np.diff(k) > 0), "keep indices must be strictly ascending"
    assert k.min() >= 0 and k.max() < n_tokens
    return k


def rows_equal(out, src, keep):
    """Bitwise equality of gathered rows: out[r] == src[keep[r]] (torch tensors, one head)."""
    idx = torch.as_tensor(np.asarray(keep), dtype=torch.long, device=src.device)
    ref = src.index_select(0, idx)
    a = out[:len(keep)].contiguous().view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32)
    b = ref.contiguous().view(torch.int16 if ref.dtype == torch.bfloat16 else torch.int32)
    return torch.equal(a, b)
