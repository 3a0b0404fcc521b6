"""Parity of the survival experiment ([Nexus] section 3, appendix 8.3 Lemma 1).

* The device selection, run as a stream over thousands of replicas with given
  weights, follows exactly the oracle's Monte Carlo paths on the same Philox
  counters, and its survival frequencies match the exact path-enumeration law.
* The survival driver's events are checked, teacher-forced on the device's
  pre-event caches, against the oracle: weights within 1e-3, the kept set
  equal to the oracle's selection on the device weights, at least 99.9% shared
  with the pure-oracle result, compacted rows and the appended rows byte-exact,
  and the tracked-id bookkeeping against a host recount.
"""

import dataclasses
from fractions import Fraction

import numpy as np
import pytest
import torch

import streaming_weighted_sampling_amd as nx
from oracle import nexus, survival as osurv
from streaming_weighted_sampling_amd.survival import run_survival
from tests import gpu_common as gc
from workloads import SURVIVAL, survival_event, survival_initial

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _table(seed, n_ids, events):
    rng = np.random.default_rng(seed)
    return rng.integers(1, 64, size=(events, n_ids)) / 64.0     # exact in fp32


def _device_stream(tab, n0, budget, app, events, replicas, seed):
    """The stream run with nx_reservoir_select: one KV head per replica."""
    cfg = nx.NexusConfig(replicas, replicas, 64, 4)
    ws = nx.new_workspace(cfg, n0 + app, 1, 0, device=DEV)
    res = np.tile(np.arange(n0, dtype=np.int64), (replicas, 1))
    nxt, out = n0, []
    for e in range(events):
        w = torch.from_numpy(tab[e][res].astype(np.float32)).to(DEV)
        keep, _ = nx.nx_reservoir_select(cfg, w, budget, seed, workspace=ws, step=e)
        k = keep.cpu().numpy().astype(np.int64)
        kept = np.take_along_axis(res, k, axis=1)
        new = np.tile(np.arange(nxt, nxt + app, dtype=np.int64), (replicas, 1))
        res = np.concatenate([kept, new], axis=1)
        nxt += app
        out.append(res)
    nx.nx_read_device_status(cfg, ws)
    return out


def test_device_stream_follows_the_oracle_paths_and_the_exact_law():
    n0, budget, app, events, reps = 4, 3, 1, 3, 4096
    tab = _table(3, n0 + app * events, events)
    exact = osurv.reservoir_survival_exact(lambda e, j: Fraction(float(tab[e][j])), n0, budget,
                                           app, events)
    # same seed, same counters: the very same paths
    dev = _device_stream(tab, n0, budget, app, events, reps, seed=21)
    ora = osurv.reservoir_survival_mc(lambda e, j: tab[e][j], n0, budget, app, events, reps,
                                      seed=21)
    for e in range(events):
        np.testing.assert_array_equal(dev[e], ora[e])
    # survival frequencies over 10 seeds against the exact law
    hits = [dict() for _ in range(events)]
    total = 0
    for seed in range(10):
        paths = _device_stream(tab, n0, budget, app, events, reps, seed=100 + seed)
        total += reps
        for e in range(events):
            for j in exact[e]:
                hits[e][j] = hits[e].get(j, 0) + int(np.any(paths[e] == j, axis=1).sum())
    for e in range(events):
        for j, p in exact[e].items():
            p = float(p)
            freq = hits[e][j] / total
            assert abs(freq - p) <= 5 * np.sqrt(p * (1 - p) / total) + 1e-12, (e, j, freq, p)


def _small_spec():
    return dataclasses.replace(SURVIVAL, n_streams=2, budget=1024, append=256, events=6,
                               per_class=16)


@pytest.mark.parametrize("policy", ["nexus", "topk", "topk_direct"])
def test_survival_events_teacher_forced(policy):
    spec = _small_spec()
    initial = survival_initial(spec, device=DEV)
    inputs = [survival_event(spec, e, device=DEV) for e in range(spec.events)]
    n_avg = {"nexus": 1, "topk": -1, "topk_direct": -1}[policy]
    walk = 0 if policy == "topk_direct" else spec.walk_iters
    checked = {0: (0, 0), 3: (1, 5), 5: (0, 7)}
    B, A, n0 = spec.budget, spec.append, spec.n0
    host_ids = np.tile(np.arange(n0), (spec.n_streams, spec.h_kv, 1))

    def on_event(e, sc, pre, ids):
        nonlocal host_ids
        keep = sc.keep.cpu().numpy().astype(np.int64)
        host_ids = np.concatenate(
            [np.take_along_axis(host_ids, keep, axis=2),
             np.broadcast_to(n0 + e * A + np.arange(A), (spec.n_streams, spec.h_kv, A))], axis=2)
        np.testing.assert_array_equal(ids.cpu().numpy(), host_ids)
        if e not in checked:
            return
        s, h = checked[e]
        q, k, v, n = pre
        k_post, v_post = sc.live()
        cfg = nx.NexusConfig(spec.h_q, spec.h_kv, spec.head_dim, spec.window, n_avg=n_avg)
        ws = nx.new_workspace(cfg, n, 1, walk, device=DEV)
        # The 16-stream batch and this one-item call both score in 256-token tiles
        # (too few head units for wider ones), so their fp32 sums run in the same order.
        w_gpu = nx.nx_nexus_weights(cfg, q[s], k[s], n, walk, workspace=ws).cpu().numpy()
        nx.nx_read_device_status(cfg, ws)
        w_ref = gc.oracle_weights(q[s], k[s], n, walk, spec.group, heads=[h])[h]
        gc.assert_weights_close(w_gpu[h], w_ref, f"event {e} stream {s} head {h}")
        _, on_gpu_w = nexus.select_from_weights(w_gpu, B, 0, layer=s, step=e, n_avg=n_avg)
        got = keep[s, h]
        np.testing.assert_array_equal(got, on_gpu_w[h])
        # pure oracle: its own weights, the same counters (head h of sequence 0)
        ref_keys = nexus.head_keys(w_ref, n, h, s, e, 0, n_avg)
        ref_keep = nexus.select_top(ref_keys, B)
        gc.assert_kept_matches_oracle(got, ref_keep, ref_keys, B, f"event {e} stream {s} head {h}",
                                      n_avg=max(n_avg, 1))
        assert gc.rows_equal(k_post[s, h], k[s, h], got)
        assert gc.rows_equal(v_post[s, h], v[s, h], got)
        assert torch.equal(k_post[s, h, B:].view(torch.int16),
                           inputs[e][1][s, h].view(torch.int16))

    res = run_survival(spec, policy, initial, lambda e: inputs[e], device=DEV,
                       on_event=on_event)
    # the driver's counts against a recount from the host ids
    cls = initial[2].cpu().numpy()
    alive = host_ids[:, :, :B]
    for c in range(len(spec.offsets)):
        tracked = np.stack([np.isin(np.nonzero(cls[s, h] == c)[0], alive[s, h])
                            for s in range(spec.n_streams) for h in range(spec.h_kv)])
        assert res.survival[-1, c].item() == pytest.approx(tracked.mean(), abs=1e-12)
    assert bool((res.survival[1:] <= res.survival[:-1] + 1e-12).all())


def test_survival_full_run_properties():
    """The full stream (16 Llama-3-8B-shaped streams, 400 events) under all three
    policies: survival curves are non-increasing and within [0, 1], and a rerun
    of the first 50 events reproduces them exactly (determinism)."""
    spec = SURVIVAL
    initial = survival_initial(spec, device=DEV)
    out = {}
    for policy in ("nexus", "topk", "topk_direct"):
        r = run_survival(spec, policy, initial,
                         lambda e: survival_event(spec, e, device=DEV), device=DEV)
        s = r.survival
        assert s.shape == (spec.events + 1, len(spec.offsets))
        assert bool((s[1:] <= s[:-1] + 1e-12).all()) and bool((s >= 0).all())
        out[policy] = s
    again = run_survival(spec, "nexus", initial,
                         lambda e: survival_event(spec, e, device=DEV), device=DEV, events=50)
    assert torch.equal(again.survival, out["nexus"][:51])
