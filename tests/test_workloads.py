"""Sanity of the seeded input generators (CPU): shapes, determinism, planted structure."""

import numpy as np
import torch

from oracle import nexus
from workloads import WORKLOADS, gen_layer, ragged_lengths, budget_for, bf16_bits


def test_tiny_workload_shapes_and_determinism():
    wl = WORKLOADS["tiny_mha_f32"]
    a = gen_layer(wl)
    b = gen_layer(wl)
    assert a["q"].shape == (1, 16, 64) and a["k"].shape == (1, 512, 64)
    assert a["k"].dtype == torch.float32
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["q"], b["q"])


def test_planted_heavy_hitters_dominate_direct_score():
    wl = WORKLOADS["tiny_mha_f32"]
    x = gen_layer(wl)
    q = x["q"].double().numpy()
    k = x["k"][0].double().numpy()
    a = nexus.direct_score(nexus.window_rows(q, k))
    top = np.argsort(a)[::-1][:8]
    # The 8 planted keys have +3 sigma logits against every query; they must
    # take most of the top ranks.
    hh = set(x["planted"]["heavy"][0].tolist())
    assert len(set(top.tolist()) & hh) >= 6
    # Bridges sit off the span of the queries: logits ~ 0 against every query.
    br = x["planted"]["bridge"][0].numpy()
    assert np.abs(q[0] @ k[br].T).max() < 1e-3


def test_bf16_layer_and_budgets():
    wl = WORKLOADS["llama3_8b_layer"]
    x = gen_layer(wl, n_tokens=256)
    assert x["k"].dtype == torch.bfloat16 and x["k"].shape == (8, 256, 128)
    bits = bf16_bits(x["k"])
    assert bits.dtype == np.uint16 and bits.shape == (8, 256, 128)
    assert budget_for(32768) == 6554 and budget_for(4096) == 819
    assert budget_for(131072, 10) == 13107
    lens = ragged_lengths(WORKLOADS["ragged16_zipf"])
    assert len(lens) == 16 and all(4096 <= n <= 16384 for n in lens)
    assert lens == ragged_lengths(WORKLOADS["ragged16_zipf"])
