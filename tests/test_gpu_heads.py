"""Per-head budgets on the device ([Nexus] appendix 10; allocation rule of the
cited Ada-KV, as the oracle states it).

* nx_head_budgets on given weights equals the oracle's allocation exactly
  (ties, non-positive weights, floors, capacities, many heads).
* nx_evict_batch with given budgets and with allocated budgets: the budgets
  equal the oracle's allocation on the device's own weights, each head's kept
  set equals the oracle's selection on those weights with its budget, at least
  99.9% of it is shared with the pure-oracle result, keep entries past a head's
  count are -1, and the compacted rows are the gathered rows.
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


def _run_batch(cfg, wl, lay, n, budget, cap, walk, hb_in=None, seed=3):
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
