"""Full-size parity of the batched path (the launch configuration bench.py times)
and of the streaming loop, on sampled head units the oracle can afford.

For every head unit of the batch the kept set is checked for its properties
(exactly min(B, N) ascending indices in range, compacted rows equal to the
gathered rows); for sampled units the weights must match the oracle within
1e-3, the kept set must equal the oracle's selection on the GPU's weights, and
it must share at least 99.9% with the pure-oracle result.
"""

import numpy as np
import pytest
import torch

import streaming_weighted_sampling_amd as nx
from oracle import nexus
from streaming_weighted_sampling_amd.stream import StreamingCache
from tests import gpu_common as gc
from workloads import (WORKLOADS, budget_for, gen_layer, gen_model, gen_stream_queries,
                       gen_stream_rows, ragged_lengths)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cfg(wl):
    return nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window,
                          torch.float32 if wl.dtype == "f32" else torch.bfloat16)


def _check_all_keeps(keep, n_tokens, budget):
    """keep: [..., budget] int32 on the GPU, all for the same n_tokens."""
    kept = min(budget, n_tokens)
    k = keep[..., :kept].long()
    assert bool((k >= 0).all()) and bool((k < n_tokens).all())
    assert bool((k[..., 1:] > k[..., :-1]).all())


def _check_unit(cfg, wl, q, k, v, keep, out_k, out_v, n, budget, walk, seed, layer, step,
                seq_id, heads):
    """Sampled-unit parity for KV heads `heads` of one (sequence, layer) item."""
    ws = nx.new_workspace(cfg, n, 1, walk, device=DEV)
    w_gpu = nx.nx_nexus_weights(cfg, q, k, n, walk, workspace=ws).cpu().numpy()
    nx.nx_read_device_status(cfg, ws)
    qh, dt = gc.host(q)
    kh, _ = gc.host(k[:, :n])
    vh, _ = gc.host(v[:, :n])
    ref = nexus.evict_step(qh, kh, vh, budget, walk, seed, dtype=dt, layer=layer, step=step,
                           seq_id=seq_id, heads=heads)
    _, on_gpu_w = nexus.select_from_weights(w_gpu, budget, seed, layer=layer, step=step,
                                            seq_id=seq_id)
    kept = min(budget, n)
    for h in heads:
        got = keep[h, :kept].cpu().numpy()
        gc.assert_weights_close(w_gpu[h], ref["w"][h], f"layer {layer} head {h}")
        np.testing.assert_array_equal(got, on_gpu_w[h])
        assert gc.overlap_fraction(got, ref["keep"][h]) >= 0.999
        assert gc.rows_equal(out_k[h], k[h], got)
        assert gc.rows_equal(out_v[h], v[h], got)


def test_stream32_event_full_size():
    """One eviction event over all 32 layers at N = 32768 (the benchmarked step)."""
    wl = WORKLOADS["llama3_8b_stream32"]
    cfg = _cfg(wl)
    n, B, L = wl.n_tokens, wl.budget, wl.n_layers
    q, k, v = gen_model(wl, device=DEV)
    keep = torch.empty(L, wl.h_kv, B, dtype=torch.int32, device=DEV)
    out_k = torch.empty(L, wl.h_kv, B, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    out_v = torch.empty_like(out_k)
    items = [dict(q=q[l], k=k[l], v=v[l], keep=keep[l], out_k=out_k[l], out_v=out_v[l],
                  kv_head_stride=n * wl.head_dim, out_head_stride=B * wl.head_dim,
                  n_tokens=n, budget=B, layer=l) for l in range(L)]
    units = nx.make_units(items, device=DEV)
    ws = nx.new_workspace(cfg, n, L, wl.walk_iters, device=DEV)
    step = 7
    nx.nx_evict_batch(cfg, units, L, n, wl.walk_iters, 0, workspace=ws, step=step,
                      max_out_rows=B)
    nx.nx_read_device_status(cfg, ws)
    _check_all_keeps(keep, n, B)
    for l, heads in ((0, [0]), (13, [5]), (31, [7])):
        _check_unit(cfg, wl, q[l], k[l], v[l], keep[l], out_k[l], out_v[l], n, B,
                    wl.walk_iters, 0, l, step, 0, heads)


def test_ragged_batch_full_size():
    """16 sequences of 4K..16K tokens x 32 layers in one call (Zipf salience)."""
    wl = WORKLOADS["ragged16_zipf"]
    cfg = _cfg(wl)
    lens = ragged_lengths(wl)
    n_max = max(lens)
    D, Hk, L = wl.head_dim, wl.h_kv, wl.n_layers
    bufs, items = [], []
    for s, n in enumerate(lens):
        B = budget_for(n)
        q, k, v = gen_model(wl, device=DEV, n_tokens=n, seq=s)
        keep = torch.empty(L, Hk, B, dtype=torch.int32, device=DEV)
        ok = torch.empty(L, Hk, B, D, dtype=torch.bfloat16, device=DEV)
        ov = torch.empty_like(ok)
        bufs.append((q, k, v, keep, ok, ov, n, B))
        for l in range(L):
            items.append(dict(q=q[l], k=k[l], v=v[l], keep=keep[l], out_k=ok[l], out_v=ov[l],
                              kv_head_stride=n * D, out_head_stride=B * D, n_tokens=n,
                              budget=B, layer=l, seq_id=s))
    units = nx.make_units(items, device=DEV)
    ws = nx.new_workspace(cfg, n_max, len(items), wl.walk_iters, device=DEV)
    nx.nx_evict_batch(cfg, units, len(items), n_max, wl.walk_iters, 11, workspace=ws, step=3,
                      max_out_rows=budget_for(n_max))
    nx.nx_read_device_status(cfg, ws)
    for (q, k, v, keep, ok, ov, n, B) in bufs:
        _check_all_keeps(keep, n, B)
    shortest = int(np.argmin(lens))
    longest = int(np.argmax(lens))
    for s, l, h in ((shortest, 0, 2), (longest, 31, 6), (5, 16, 0)):
        q, k, v, keep, ok, ov, n, B = bufs[s]
        _check_unit(cfg, wl, q[l], k[l], v[l], keep[l], ok[l], ov[l], n, B, wl.walk_iters, 11,
                    l, 3, s, [h])


def test_llama70b_share_full_size():
    """8 layers, GQA 64:8, W = 64, N = 131072 -> B = 13107 (10x reduction)."""
    wl = WORKLOADS["llama70b_share"]
    cfg = _cfg(wl)
    n, B, L = wl.n_tokens, wl.budget, wl.n_layers
    q, k, v = gen_model(wl, device=DEV)
    keep = torch.empty(L, wl.h_kv, B, dtype=torch.int32, device=DEV)
    out_k = torch.empty(L, wl.h_kv, B, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    out_v = torch.empty_like(out_k)
    items = [dict(q=q[l], k=k[l], v=v[l], keep=keep[l], out_k=out_k[l], out_v=out_v[l],
                  kv_head_stride=n * wl.head_dim, out_head_stride=B * wl.head_dim,
                  n_tokens=n, budget=B, layer=l) for l in range(L)]
    units = nx.make_units(items, device=DEV)
    ws = nx.new_workspace(cfg, n, L, wl.walk_iters, device=DEV)
    nx.nx_evict_batch(cfg, units, L, n, wl.walk_iters, 0, workspace=ws, step=0, max_out_rows=B)
    nx.nx_read_device_status(cfg, ws)
    _check_all_keeps(keep, n, B)
    for l, heads in ((0, [3]), (7, [6])):
        _check_unit(cfg, wl, q[l], k[l], v[l], keep[l], out_k[l], out_v[l], n, B,
                    wl.walk_iters, 0, l, 0, 0, heads)


def _stream_setup(wl, layers, n0, steps_seen=()):
    cfg = _cfg(wl)
    B, A = wl.budget, wl.stream_append
    sc = StreamingCache(cfg, len(layers), max(n0 + A, B + A), B, A, wl.walk_iters, seed=0,
                        device=DEV)
    q, k, v = gen_model(wl, device=DEV, n_tokens=n0, layers=layers)
    # The rows that arrive before the first event complete the initial cache.
    k0 = torch.empty(len(layers), wl.h_kv, n0 + A, wl.head_dim, dtype=k.dtype, device=DEV)
    v0 = torch.empty_like(k0)
    k0[:, :, :n0] = k
    v0[:, :, :n0] = v
    for i, l in enumerate(layers):
        k0[i, :, n0:], v0[i, :, n0:] = gen_stream_rows(wl, layer=l, step=0, n_new=A, device=DEV)
    sc.load(k0, v0, n0 + A)
    return sc


def _stream_inputs(sc, wl, layers, step):
    for i, l in enumerate(layers):
        sc.q[i].copy_(gen_stream_queries(wl, layer=l, step=step, device=DEV))
        nk, nv = gen_stream_rows(wl, layer=l, step=step + 1, n_new=wl.stream_append, device=DEV)
        sc.app_k[i].copy_(nk)
        sc.app_v[i].copy_(nv)


def test_streaming_100_events_teacher_forced():
    """All 32 layers: 100 append-256 / evict-to-6554 events; the oracle re-runs
    sampled events on the GPU's own pre-event caches."""
    wl = WORKLOADS["llama3_8b_stream32"]
    layers = list(range(wl.n_layers))
    sc = _stream_setup(wl, layers, wl.n_tokens)
    B, A = wl.budget, wl.stream_append
    checked = {0: (0, 0), 1: (21, 3), 50: (9, 4), 99: (31, 7)}
    for step in range(wl.stream_steps):
        _stream_inputs(sc, wl, layers, step)
        pre = None
        if step in checked:
            li, h = checked[step]
            k_pre, v_pre = sc.live()
            pre = (li, h, sc.q[li].clone(), k_pre[li].clone(), v_pre[li].clone(), sc.n_tokens,
                   sc.app_k[li].clone(), sc.app_v[li].clone())
        sc.step()
        if pre is not None:
            li, h, q, kp, vp, n, ak, av = pre
            nx.nx_read_device_status(sc.cfg, sc.ws)
            k_post, v_post = sc.live()
            assert sc.n_tokens == min(B, n) + A
            keep = sc.keep[li]
            _check_all_keeps(keep, n, B)
            _check_unit(sc.cfg, wl, q, kp, vp, keep, k_post[li], v_post[li], n, B,
                        wl.walk_iters, 0, layers[li], step, 0, [h])
            kept = min(B, n)
            assert torch.equal(k_post[li][:, kept:].view(torch.int16), ak.view(torch.int16))
            assert torch.equal(v_post[li][:, kept:].view(torch.int16), av.view(torch.int16))
    nx.nx_read_device_status(sc.cfg, sc.ws)


def test_streaming_resume_is_bitwise_equal():
    wl = WORKLOADS["llama3_8b_stream32"]
    layers = [0, 1, 2, 3]
    n0 = 8192

    def run(split):
        sc = _stream_setup(wl, layers, n0)
        for step in range(6):
            if step == split:
                st = sc.state()
                sc = StreamingCache(sc.cfg, len(layers), sc.capacity, sc.budget, sc.n_append,
                                    sc.walk_iters, seed=0, device=DEV)
                sc.restore(st)
            _stream_inputs(sc, wl, layers, step)
            sc.step()
        nx.nx_read_device_status(sc.cfg, sc.ws)
        return sc.live()

    k_a, v_a = run(split=None)
    k_b, v_b = run(split=3)
    assert torch.equal(k_a.view(torch.int16), k_b.view(torch.int16))
    assert torch.equal(v_a.view(torch.int16), v_b.view(torch.int16))
