"""Per-head budgets on the device ([Nexus] appendix 10; allocation rule of the
cited Ada-KV, as the oracle states it).

* nx_head_budgets on given weights equals the oracle's allocation exactly
  (ties, non-positive weights, floors, capacities, many heads).
* nx_evict_batch with given budgets and with allocated budgets: the budgets
  equal the oracle's allocation on the device's own weights, each head's kept
  set equals the oracle's selection on those weights with its budget, at least
  99.9% of it is shared with the pure-oracle result, keep entries past a head's
  count are -1, and the compacted rows are the gathered rows.
* Per-head resident counts (head_tokens / head_tokens_out): one event on
  ragged heads, and streaming decode with allocated budgets (copy and in
  place), every event against the oracle on the device's pre-event cache.
"""

import numpy as np
import pytest
import torch

import streaming_weighted_sampling_amd as nx
from oracle import nexus
from tests import gpu_common as gc
from workloads import WORKLOADS, gen_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _weights(rng, h, n, kind):
    if kind == "smooth":
        return rng.exponential(size=(h, n)).astype(np.float32) ** 3 * 1e-4
    if kind == "ties":
        return rng.choice(np.float32([0.5, 0.25, 0.125, 0.0, -1.0]), size=(h, n))
    # a concentrated head, a spread head and random ones
    w = rng.exponential(size=(h, n)).astype(np.float32) * 1e-5
    w[0, :50] = 0.01
    if h > 1:
        w[1, :] = 3e-5
    return w


@pytest.mark.parametrize("h,n", [(8, 4096), (8, 40000), (1, 3000), (64, 1000)])
@pytest.mark.parametrize("kind", ["smooth", "ties", "mixed"])
def test_allocation_on_given_weights_is_exact(h, n, kind):
    rng = np.random.default_rng(h * 1000 + n + len(kind))
    w = _weights(rng, h, n, kind)
    wt = torch.from_numpy(w).to(DEV)
    cfg = nx.NexusConfig(h, h, 64, 4, head_alloc=nx.NX_HEADS_ALLOC)
    for budget, floor, cap in [(n // 5, 0, 0), (n // 5, n // 25, 2 * n // 5), (n // 3, n // 3, 0),
                               (1, 0, 0), (n + 7, 3, n), (max(1, n // 7), 2, n // 6)]:
        cfg.head_floor = floor
        ws = nx.new_workspace(cfg, n, 1, 0, device=DEV)
        got = nx.nx_head_budgets(cfg, wt, budget, workspace=ws, head_cap=cap).cpu().numpy()
        nx.nx_read_device_status(cfg, ws)
        want = nexus.ada_head_budgets(w, budget, floor, cap=cap if cap > 0 else budget)
        np.testing.assert_array_equal(got, want, err_msg=f"B={budget} f={floor} cap={cap}")


def _layer(n):
    wl = WORKLOADS["llama3_8b_layer"]
    return wl, gen_layer(wl, n_tokens=n, device=DEV)


def _run_batch(cfg, wl, lay, n, budget, cap, walk, hb_in=None, seed=3, ws=None):
    H, D = wl.h_kv, wl.head_dim
    rows = min(cap * cfg.block, n)
    keep = torch.full((H, cap), 12345, dtype=torch.int32, device=DEV)
    out_k = torch.zeros(H, rows, D, dtype=cfg.dtype, device=DEV)
    out_v = torch.zeros_like(out_k)
    hb = (torch.zeros(H, dtype=torch.int32, device=DEV) if hb_in is None else
          torch.tensor(hb_in, dtype=torch.int32, device=DEV))
    k = lay["k"][:, :n].contiguous()
    v = lay["v"][:, :n].contiguous()
    w_sel = torch.full((H, cfg.units(n)), float("nan"), device=DEV)
    units = nx.make_units([dict(q=lay["q"], k=k, v=v, keep=keep, out_k=out_k, out_v=out_v,
                                kv_head_stride=n * D, out_head_stride=rows * D, n_tokens=n,
                                budget=budget, head_cap=cap, head_budget=hb, layer=5,
                                out_w=w_sel)],
                          device=DEV)
    if ws is None:
        ws = nx.new_workspace(cfg, n, 1, walk, device=DEV)
    nx.nx_evict_batch(cfg, units, 1, n, walk, seed, workspace=ws, step=2, max_out_rows=rows)
    nx.nx_read_device_status(cfg, ws)
    return k, v, keep, out_k, out_v, hb.cpu().numpy(), w_sel.cpu().numpy()


def _check(cfg, wl, lay, k, v, keep, out_k, out_v, budgets, n, walk, w_gpu, seed=3):
    """w_gpu: the weights the batch exported (its selection's weights)."""
    _, on_gpu_w = nexus.select_from_weights(w_gpu, 0, seed, layer=5, step=2,
                                            head_budgets=budgets)
    qh, dt = gc.host(lay["q"])
    kh, _ = gc.host(k)
    vh, _ = gc.host(v)
    ref = nexus.evict_step(qh, kh, vh, int(max(budgets)), walk, seed, dtype=dt, layer=5,
                           step=2, block=cfg.block, head_budgets=budgets)
    keep = keep.cpu().numpy()
    for h in range(wl.h_kv):
        nu = w_gpu.shape[1]
        kept = min(int(budgets[h]), nu)
        np.testing.assert_array_equal(keep[h, :kept], on_gpu_w[h], err_msg=f"head {h}")
        assert np.all(keep[h, kept:] == -1)
        gc.assert_weights_close(w_gpu[h], ref["w"][h], f"head {h}")
        gc.assert_kept_matches_oracle(keep[h, :kept], ref["keep"][h], ref["keys"][h], kept,
                                      f"head {h}")
        rows = np.concatenate([np.arange(b * cfg.block, min((b + 1) * cfg.block, n))
                               for b in keep[h, :kept]])
        assert gc.rows_equal(out_k[h], k[h], rows)
        assert gc.rows_equal(out_v[h], v[h], rows)
    return w_gpu


@pytest.mark.parametrize("n", [4096, 40000])
def test_batch_with_given_budgets(n):
    wl, lay = _layer(n)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_GIVEN)
    B = n // 5
    cap = 2 * B + n // 2
    given = [B, 1, B // 3, 2 * B, B + 17, cap, 5, B // 2]
    k, v, keep, ok, ov, hb, w = _run_batch(cfg, wl, lay, n, B, cap, wl.walk_iters, hb_in=given)
    np.testing.assert_array_equal(hb, given)
    _check(cfg, wl, lay, k, v, keep, ok, ov, np.array(given), n, wl.walk_iters, w)


@pytest.mark.parametrize("n,floor,cap_mult", [(4096, 0, 2), (4096, 100, 3), (40000, 800, 2),
                                              (20001, 0, 1)])
def test_batch_with_allocated_budgets(n, floor, cap_mult):
    wl, lay = _layer(n)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_ALLOC, head_floor=floor)
    B = n // 5
    cap = cap_mult * B
    k, v, keep, ok, ov, hb, w = _run_batch(cfg, wl, lay, n, B, cap, wl.walk_iters)
    w_gpu = _check(cfg, wl, lay, k, v, keep, ok, ov, hb, n, wl.walk_iters, w)
    np.testing.assert_array_equal(hb, nexus.ada_head_budgets(w_gpu, B, floor, cap=cap))
    if cap_mult > 1:
        assert hb.sum() == wl.h_kv * B
    assert hb.min() >= floor


def test_batch_allocated_budgets_with_blocks():
    n, b = 8192, 32
    wl, lay = _layer(n)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16, block=b,
                         head_alloc=nx.NX_HEADS_ALLOC, head_floor=4)
    B = 51
    k, v, keep, ok, ov, hb, w = _run_batch(cfg, wl, lay, n, B, 3 * B, wl.walk_iters)
    w_gpu = _check(cfg, wl, lay, k, v, keep, ok, ov, hb, n, wl.walk_iters, w)
    np.testing.assert_array_equal(hb, nexus.ada_head_budgets(w_gpu, B, 4, cap=3 * B))


def test_given_budget_above_capacity_marks_the_item_bad():
    n = 2048
    wl, lay = _layer(n)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_GIVEN)
    with pytest.raises(nx.NexusError) as e:
        _run_batch(cfg, wl, lay, n, 400, 400, wl.walk_iters, hb_in=[400] * 7 + [401])
    assert e.value.code == nx.NX_EINVAL


# ------------------------------------------------ per-head resident counts --


def test_uniform_budget_on_ragged_heads():
    """One event on heads of different lengths (head_tokens): each head's
    weights, selection and rows follow the oracle on its own rows, and
    head_tokens_out holds min(B, n_h) + n_append."""
    n, B, A = 4096, 700, 64
    wl, lay = _layer(n)
    H, D = wl.h_kv, wl.head_dim
    cfg = nx.NexusConfig(wl.h_q, H, D, wl.window, torch.bfloat16)
    counts = [4096, 3000, 701, 700, 1, 2048, 4095, 1500]
    tin = torch.tensor(counts, dtype=torch.int32, device=DEV)
    tout = torch.full((H,), -7, dtype=torch.int32, device=DEV)
    keep = torch.full((H, B), 12345, dtype=torch.int32, device=DEV)
    out_k = torch.zeros(H, B + A, D, dtype=cfg.dtype, device=DEV)
    out_v = torch.zeros_like(out_k)
    app_k = torch.randn(H, A, D, device=DEV).to(cfg.dtype)
    app_v = torch.randn_like(app_k)
    w_sel = torch.full((H, n), float("nan"), device=DEV)
    units = nx.make_units([dict(q=lay["q"], k=lay["k"], v=lay["v"], keep=keep, out_k=out_k,
                                out_v=out_v, app_k=app_k, app_v=app_v, kv_head_stride=n * D,
                                out_head_stride=(B + A) * D, n_tokens=n, budget=B, n_append=A,
                                layer=1, out_w=w_sel, head_tokens=tin, head_tokens_out=tout)],
                          device=DEV)
    ws = nx.new_workspace(cfg, n, 1, wl.walk_iters, device=DEV)
    nx.nx_evict_batch(cfg, units, 1, n, wl.walk_iters, 11, workspace=ws, step=3,
                      max_out_rows=B + A)
    nx.nx_read_device_status(cfg, ws)
    np.testing.assert_array_equal(tout.cpu().numpy(), [min(B, c) + A for c in counts])
    qh, dt = gc.host(lay["q"])
    kh, _ = gc.host(lay["k"])
    vh, _ = gc.host(lay["v"])
    ref = nexus.evict_step(qh, [kh[h, :c] for h, c in enumerate(counts)],
                           [vh[h, :c] for h, c in enumerate(counts)], B, wl.walk_iters, 11,
                           dtype=dt, layer=1, step=3)
    w = w_sel.cpu().numpy()
    keep = keep.cpu().numpy()
    _, on_gpu_w = nexus.select_from_weights([w[h, :c] for h, c in enumerate(counts)], B, 11,
                                            layer=1, step=3)
    for h, c in enumerate(counts):
        kept = min(B, c)
        assert np.all(np.isnan(w[h, c:])), f"head {h}: weights written past its count"
        gc.assert_weights_close(w[h, :c], ref["w"][h], f"head {h}")
        np.testing.assert_array_equal(keep[h, :kept], on_gpu_w[h], err_msg=f"head {h}")
        gc.assert_kept_matches_oracle(keep[h, :kept], ref["keep"][h], ref["keys"][h], kept,
                                      f"head {h}")
        assert gc.rows_equal(out_k[h, :kept], lay["k"][h], keep[h, :kept])
        assert gc.rows_equal(out_v[h, :kept], lay["v"][h], keep[h, :kept])
        assert torch.equal(out_k[h, kept:kept + A].view(torch.int16), app_k[h].view(torch.int16))
        assert torch.equal(out_v[h, kept:kept + A].view(torch.int16), app_v[h].view(torch.int16))


@pytest.mark.parametrize("bad", ["same_array", "above_n_tokens", "zero"])
def test_bad_head_tokens_mark_the_item_bad(bad):
    n, B = 1024, 200
    wl, lay = _layer(n)
    H, D = wl.h_kv, wl.head_dim
    cfg = nx.NexusConfig(wl.h_q, H, D, wl.window, torch.bfloat16)
    vals = [n] * H
    if bad == "above_n_tokens":
        vals[3] = n + 1
    if bad == "zero":
        vals[5] = 0
    tin = torch.tensor(vals, dtype=torch.int32, device=DEV)
    tout = tin if bad == "same_array" else torch.zeros(H, dtype=torch.int32, device=DEV)
    keep = torch.zeros(H, B, dtype=torch.int32, device=DEV)
    out_k = torch.zeros(H, B, D, dtype=cfg.dtype, device=DEV)
    out_v = torch.zeros_like(out_k)
    units = nx.make_units([dict(q=lay["q"], k=lay["k"], v=lay["v"], keep=keep, out_k=out_k,
                                out_v=out_v, kv_head_stride=n * D, out_head_stride=B * D,
                                n_tokens=n, budget=B, head_tokens=tin, head_tokens_out=tout)],
                          device=DEV)
    ws = nx.new_workspace(cfg, n, 1, wl.walk_iters, device=DEV)
    with pytest.raises(nx.NexusError) as e:
        nx.nx_evict_batch(cfg, units, 1, n, wl.walk_iters, 1, workspace=ws, max_out_rows=B)
        nx.nx_read_device_status(cfg, ws)
    assert e.value.code == nx.NX_EINVAL
    if bad == "same_array":
        np.testing.assert_array_equal(tin.cpu().numpy(), vals)


@pytest.mark.parametrize("inplace", [False, True])
def test_streaming_decode_with_allocated_budgets(inplace):
    """Four append-128 / evict events on two layers with allocated per-head
    budgets (floor 32, capacity 2B): the heads' row counts drift apart and
    travel on the device from one event to the next.  Every event is checked
    against the oracle on the device's pre-event cache: the allocation exactly
    on the device's weights, the selection exactly on them, the weights and
    kept sets against the pure oracle, the new counts and the new rows."""
    from streaming_weighted_sampling_amd.stream import StreamingCache
    wl = WORKLOADS["llama3_8b_layer"]
    L, n0, A, B, floor, seed = 2, 2048, 128, 400, 32, 5
    cap = 2 * B
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_ALLOC, head_floor=floor)
    sc = StreamingCache(cfg, L, max(n0, cap + A), B, A, wl.walk_iters, seed=seed, device=DEV,
                        inplace=inplace, export_w=True, head_cap=cap)
    g = torch.Generator(device="cpu").manual_seed(23)
    k0 = torch.randn((L, wl.h_kv, n0, wl.head_dim), generator=g).to(torch.bfloat16)
    # Heads with different spreads so that the allocation moves budget between them.
    k0 = k0 * torch.linspace(0.3, 3.0, wl.h_kv).view(1, -1, 1, 1).to(torch.bfloat16)
    sc.load(k0.to(DEV), torch.randn_like(k0).to(DEV), n0)
    drift = False
    for step in range(4):
        sc.q.copy_(torch.randn(sc.q.shape, generator=g).to(torch.bfloat16))
        sc.app_k.copy_(torch.randn(sc.app_k.shape, generator=g).to(torch.bfloat16))
        sc.app_v.copy_(torch.randn(sc.app_v.shape, generator=g).to(torch.bfloat16))
        pre = sc.head_tokens().numpy()
        kp, vp = (gc.host(t)[0] for t in sc.live())
        sc.step()
        nx.nx_read_device_status(sc.cfg, sc.ws)
        post = sc.head_tokens().numpy()
        hb_all = sc.head_budget.cpu().numpy()
        kl, vl = (gc.host(t)[0] for t in sc.live())
        app_k, app_v = gc.host(sc.app_k)[0], gc.host(sc.app_v)[0]
        for l in range(L):
            what = f"step {step} layer {l}"
            counts = pre[l]
            hb = hb_all[l]
            w_all = sc.weights(l).cpu().numpy()
            w_gpu = [w_all[h, :c] for h, c in enumerate(counts)]
            np.testing.assert_array_equal(hb, nexus.ada_head_budgets(w_gpu, B, floor, cap=cap),
                                          err_msg=what)
            _, on_gpu_w = nexus.select_from_weights(w_gpu, 0, seed, layer=l, step=step,
                                                    head_budgets=hb)
            qh, dt = gc.host(sc.q[l])
            ref = nexus.evict_step(qh, [kp[l, h, :c] for h, c in enumerate(counts)],
                                   [vp[l, h, :c] for h, c in enumerate(counts)], B,
                                   wl.walk_iters, seed, dtype=dt, layer=l, step=step,
                                   head_budgets=hb)
            keep = sc.keep[l].cpu().numpy()
            for h, c in enumerate(counts):
                kept = min(int(hb[h]), int(c))
                np.testing.assert_array_equal(keep[h, :kept], on_gpu_w[h], err_msg=f"{what} head {h}")
                assert np.all(keep[h, kept:] == -1)
                gc.assert_weights_close(w_gpu[h], ref["w"][h], f"{what} head {h}")
                gc.assert_kept_matches_oracle(keep[h, :kept], ref["keep"][h], ref["keys"][h],
                                              kept, f"{what} head {h}")
                assert post[l, h] == kept + A
                if inplace:   # all pre-event rows of the buffer: they hold kept + A
                    exp_k = nexus.compact_inplace(kp[l, h], keep[h, :kept], app_k[l, h])
                    exp_v = nexus.compact_inplace(vp[l, h], keep[h, :kept], app_v[l, h])
                else:
                    exp_k = np.concatenate([kp[l, h][keep[h, :kept]], app_k[l, h]])
                    exp_v = np.concatenate([vp[l, h][keep[h, :kept]], app_v[l, h]])
                np.testing.assert_array_equal(kl[l, h, :kept + A], exp_k[:kept + A])
                np.testing.assert_array_equal(vl[l, h, :kept + A], exp_v[:kept + A])
        drift = drift or len(set(post.ravel().tolist())) > 1
    assert drift, "the allocation never moved budget between heads"


def test_allocated_budgets_on_a_reused_workspace():
    """Two allocated-budget events of different sizes on one workspace: the
    allocation histograms sit at another offset in the second call (over the
    first call's keys and scores), so each call must clear them itself.  Both
    calls' budgets equal the oracle's allocation on their exported weights."""
    wl, lay = _layer(4096)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_ALLOC, head_floor=40)
    ws = nx.new_workspace(cfg, 4096, 1, wl.walk_iters, device=DEV)
    for n in (4096, 1536):
        B = n // 5
        k, v, keep, ok, ov, hb, w = _run_batch(cfg, wl, lay, n, B, 2 * B, wl.walk_iters, ws=ws)
        w_gpu = _check(cfg, wl, lay, k, v, keep, ok, ov, hb, n, wl.walk_iters, w)
        np.testing.assert_array_equal(hb, nexus.ada_head_budgets(w_gpu, B, 40, cap=2 * B),
                                      err_msg=f"n = {n}")


def test_allocated_budgets_with_a_deep_walk():
    """Allocated per-head budgets on the weights of a deep walk (H = 16: walk
    rows stored by the second sweep, Gram pass): the budgets equal the
    oracle's allocation on the exported weights, the kept sets the oracle's
    selection on them, and the weights the pure oracle's within 1e-3."""
    n = 4096
    wl, lay = _layer(n)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_ALLOC, head_floor=40)
    B = n // 5
    k, v, keep, ok, ov, hb, w = _run_batch(cfg, wl, lay, n, B, 2 * B, 16)
    w_gpu = _check(cfg, wl, lay, k, v, keep, ok, ov, hb, n, 16, w)
    np.testing.assert_array_equal(hb, nexus.ada_head_budgets(w_gpu, B, 40, cap=2 * B))


def test_streaming_decode_deep_walk_inplace():
    """Three in-place append-64 / evict events with a deep walk (H = 12) and
    allocated per-head budgets: every event against the oracle on the
    device's pre-event cache."""
    from streaming_weighted_sampling_amd.stream import StreamingCache
    wl = WORKLOADS["llama3_8b_layer"]
    L, n0, A, B, floor, seed, walk = 1, 1500, 64, 300, 20, 9, 12
    cap = 2 * B
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         head_alloc=nx.NX_HEADS_ALLOC, head_floor=floor)
    sc = StreamingCache(cfg, L, max(n0, cap + A), B, A, walk, seed=seed, device=DEV,
                        inplace=True, export_w=True, head_cap=cap)
    g = torch.Generator(device="cpu").manual_seed(31)
    k0 = torch.randn((L, wl.h_kv, n0, wl.head_dim), generator=g).to(torch.bfloat16)
    k0 = k0 * torch.linspace(0.4, 2.5, wl.h_kv).view(1, -1, 1, 1).to(torch.bfloat16)
    sc.load(k0.to(DEV), torch.randn_like(k0).to(DEV), n0)
    for step in range(3):
        sc.q.copy_(torch.randn(sc.q.shape, generator=g).to(torch.bfloat16))
        sc.app_k.copy_(torch.randn(sc.app_k.shape, generator=g).to(torch.bfloat16))
        sc.app_v.copy_(torch.randn(sc.app_v.shape, generator=g).to(torch.bfloat16))
        pre = sc.head_tokens().numpy()
        kp, vp = (gc.host(t)[0] for t in sc.live())
        sc.step()
        nx.nx_read_device_status(sc.cfg, sc.ws)
        post = sc.head_tokens().numpy()
        hb = sc.head_budget.cpu().numpy()[0]
        kl, _ = (gc.host(t)[0] for t in sc.live())
        app_k = gc.host(sc.app_k)[0]
        counts = pre[0]
        w_all = sc.weights(0).cpu().numpy()
        w_gpu = [w_all[h, :c] for h, c in enumerate(counts)]
        np.testing.assert_array_equal(hb, nexus.ada_head_budgets(w_gpu, B, floor, cap=cap))
        _, on_gpu_w = nexus.select_from_weights(w_gpu, 0, seed, layer=0, step=step,
                                                head_budgets=hb)
        qh, dt = gc.host(sc.q[0])
        ref = nexus.evict_step(qh, [kp[0, h, :c] for h, c in enumerate(counts)],
                               [vp[0, h, :c] for h, c in enumerate(counts)], B, walk, seed,
                               dtype=dt, layer=0, step=step, head_budgets=hb)
        keep = sc.keep[0].cpu().numpy()
        for h, c in enumerate(counts):
            kept = min(int(hb[h]), int(c))
            what = f"step {step} head {h}"
            np.testing.assert_array_equal(keep[h, :kept], on_gpu_w[h], err_msg=what)
            gc.assert_weights_close(w_gpu[h], ref["w"][h], what)
            gc.assert_kept_matches_oracle(keep[h, :kept], ref["keep"][h], ref["keys"][h], kept, what)
            assert post[0, h] == kept + A
            exp_k = nexus.compact_inplace(kp[0, h], keep[h, :kept], app_k[0, h])
            np.testing.assert_array_equal(kl[0, h, :kept + A], exp_k[:kept + A])
