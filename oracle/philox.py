"""Philox4x32-10 in plain numpy uint64 arithmetic (oracle side; test infrastructure).

Definition followed: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
easy as 1, 2, 3" (SC'11), the Philox-4x32 bijection with 10 rounds.  One round
maps the counter (x0, x1, x2, x3) under round key (k0, k1) to

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))

with multipliers M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key
is bumped by the Weyl constants W0 = 0x9E3779B9, W1 = 0xBB67AE85 (mod 2^32).

The Nexus pages fix only that a fixed random seed is used ([Nexus] section
5.1, implementation details); the counter layout and the 53-bit uniform are
this implementation's reading:

    counter = (token j, seq * H_kv + kv_head, layer, step), key = (seed lo, seed hi)
    u = (((x0 << 32) | x1) >> 11) + 1) * 2^-53  in (0, 1], exact in fp64.

For the n-averaged priority of [Nexus] section 2.3 (Eq. 6) a token needs n
draws: draws 2c and 2c + 1 come from block c, the same counter under key
(seed lo, seed hi + c mod 2^32), built from words (x0, x1) and (x2, x3).
Draw 0 is the single-draw uniform above.

Pins (tests/test_oracle_philox.py): bit-exact agreement with the independent
Philox4x32-10 engine in ROCm's rocRAND headers (compiled for the host, called
only by the test) on > 1e6 counters, plus uniformity (KS) and counter
sensitivity checks.
"""

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)


def _u32(x):
    return np.asarray(x, dtype=np.uint64) & MASK32


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply the 10-round Philox4x32 bijection; all arguments broadcast.

    Every argument is an integer array (or scalar) holding a 32-bit value.
    Returns four uint64 arrays holding the 32-bit output words.
    """
    x0, x1, x2, x3 = np.broadcast_arrays(_u32(c0), _u32(c1), _u32(c2), _u32(c3))
    x0, x1, x2, x3 = (a.copy() for a in (x0, x1, x2, x3))
    ka = _u32(k0)
    kb = _u32(k1)
    thirty_two = np.uint64(32)
    for rnd in range(10):
        # 32 x 32 -> 64-bit products are exact in uint64.
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> thirty_two, p0 & MASK32
        hi1, lo1 = p1 >> thirty_two, p1 & MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
        if rnd < 9:
            ka = (ka + W0) & MASK32
            kb = (kb + W1) & MASK32
    return x0, x1, x2, x3


def _u53(hi, lo):
    k53 = ((hi << np.uint64(32)) | lo) >> np.uint64(11)
    # k53 + 1 <= 2^53 is exactly representable, and so is the scaled result.
    return (k53 + np.uint64(1)).astype(np.float64) * (2.0 ** -53)


def uniforms_n(token, unit_id, layer, step, seed, n):
    """n draws per counter (Eq. 6): array of shape broadcast(...) + (n,)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    draws = []
    for c in range((n + 1) // 2):
        x0, x1, x2, x3 = philox4x32_10(token, unit_id, layer, step, seed & 0xFFFFFFFF,
                                       ((seed >> 32) + c) & 0xFFFFFFFF)
        draws.append(_u53(x0, x1))
        draws.append(_u53(x2, x3))
    return np.stack(draws[:n], axis=-1)


def uniforms(token, unit_id, layer, step, seed):
    """53-bit uniforms u in (0, 1] for the given counter words (broadcast).

    ``seed`` is a 64-bit integer; its low word is key k0 and its high word k1.
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    x0, x1, _, _ = philox4x32_10(token, unit_id, layer, step,
                                 seed & 0xFFFFFFFF, seed >> 32)
    k53 = ((x0 << np.uint64(32)) | x1) >> np.uint64(11)
    # k53 + 1 <= 2^53 is exactly representable, and so is the scaled result.
    return (k53 + np.uint64(1)).astype(np.float64) * (2.0 ** -53)
