"""Helpers for the GPU parity tests: move GPU inputs to the oracle, compare.

The oracle only ever sees host copies of the exact tensors the HIP path
consumed; no expected value is taken from the HIP path except where a test
explicitly runs the oracle's selection on the GPU's own weights.
"""

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


def overlap_fraction(keep_a, keep_b):
    a, b = set(np.asarray(keep_a).tolist()), set(np.asarray(keep_b).tolist())
    return len(a & b) / max(len(b), 1)


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
