"""Pins of the oracle's Philox4x32-10 (CPU).

The oracle's numpy implementation is compared bit for bit with rocRAND's own
Philox4x32-10 engine (ROCm headers, compiled for the host by this test; a
separate implementation of the same published generator) on more than 1e6
random counters and keys, then checked for uniformity.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_ref", "rocrand_philox.cpp")
BIN = os.path.join(HERE, "_bin", "rocrand_philox")
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def rocrand_bin():
    if not os.path.isdir(os.path.join(ROCM_INC, "rocrand")) or shutil.which("g++") is None:
        pytest.skip("rocRAND headers or g++ not available")
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    if not os.path.exists(BIN) or os.path.getmtime(BIN) < os.path.getmtime(SRC):
        subprocess.run(["g++", "-O2", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}", SRC,
                        "-o", BIN], check=True)
    return BIN


def _rocrand(binary, rec):
    out = subprocess.run([binary], input=rec.astype(np.uint32).tobytes(),
                         capture_output=True, check=True).stdout
    return np.frombuffer(out, dtype=np.uint32).reshape(-1, 4)


def test_matches_rocrand_on_random_counters(rocrand_bin):
    rng = np.random.default_rng(20240601)
    n = 1_100_000
    rec = rng.integers(0, 2 ** 32, size=(n, 6), dtype=np.uint64)
    rec[0] = 0
    rec[1] = 0xFFFFFFFF
    rec[2:1000, 1:] = rng.integers(0, 4, size=(998, 5))      # small words
    ref = _rocrand(rocrand_bin, rec)
    mine = np.stack(philox.philox4x32_10(*[rec[:, i] for i in range(6)]), axis=1)
    assert np.array_equal(mine.astype(np.uint32), ref)


def test_matches_rocrand_on_the_token_counter_layout(rocrand_bin):
    """The counters the eviction step uses: (token, unit, layer, step), key = seed."""
    tok = np.arange(70000, dtype=np.uint64)
    for unit, layer, step, seed in ((0, 0, 0, 0), (13, 31, 99, 0x123456789ABCDEF0)):
        rec = np.zeros((len(tok), 6), dtype=np.uint64)
        rec[:, 0] = tok
        rec[:, 1], rec[:, 2], rec[:, 3] = unit, layer, step
        rec[:, 4], rec[:, 5] = seed & 0xFFFFFFFF, seed >> 32
        ref = _rocrand(rocrand_bin, rec)
        x0, x1, _, _ = philox.philox4x32_10(tok, unit, layer, step, seed & 0xFFFFFFFF, seed >> 32)
        assert np.array_equal(x0.astype(np.uint32), ref[:, 0])
        assert np.array_equal(x1.astype(np.uint32), ref[:, 1])
        # The 53-bit uniform built from the reference words.
        k53 = ((ref[:, 0].astype(np.uint64) << np.uint64(32)) | ref[:, 1]) >> np.uint64(11)
        u_ref = (k53 + np.uint64(1)).astype(np.float64) * 2.0 ** -53
        assert np.array_equal(philox.uniforms(tok, unit, layer, step, seed), u_ref)


def test_uniforms_are_uniform_and_in_range():
    u = philox.uniforms(np.arange(200000, dtype=np.uint64), 1, 2, 3, 4)
    assert u.min() > 0.0 and u.max() <= 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    # Different counter words give unrelated streams.
    v = philox.uniforms(np.arange(200000, dtype=np.uint64), 1, 2, 4, 4)
    assert abs(np.corrcoef(u, v)[0, 1]) < 0.02


def test_uniform_extremes_are_exact():
    # k53 = 0 -> u = 2^-53; k53 = 2^53 - 1 -> u = 1 exactly (checked on the formula's
    # integer path, the only arithmetic between the Philox words and u).
    k53 = np.array([0, 2 ** 53 - 1], dtype=np.uint64)
    u = (k53 + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    assert u[0] == 2.0 ** -53 and u[1] == 1.0
