"""Parity of the HIP path (through the C ABI) with the fp64 oracle, stage by stage.

Tolerances: Nexus weights within 1e-3 relative; reservoir selection on given
weights bit-exact; compaction byte-exact; end to end at least 99.9% of the
kept set shared with the oracle, and bit-exact when the oracle selects on the
GPU's own weights.
"""

import zlib

import numpy as np
import pytest
import torch

import streaming_weighted_sampling_amd as nx
from oracle import nexus, philox
from tests import gpu_common as gc
from workloads import WORKLOADS, gen_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cfg(h_q, h_kv, d, w, dtype=torch.bfloat16, **kw):
    return nx.NexusConfig(h_q, h_kv, d, w, dtype, **kw)


def _ws(cfg, n, units=1, walk=3):
    return nx.new_workspace(cfg, n, units, walk, device=DEV)


# ---------------------------------------------------------------- reservoir --

def test_philox_keys_bitexact_over_a_million_counters():
    """Keys ln(u)/1 expose the Philox uniform; compare with the oracle's generator."""
    h_kv, n = 8, 131072
    cfg = _cfg(8, h_kv, 128, 4)
    ws = _ws(cfg, n, walk=0)
    w = torch.ones(h_kv, n, dtype=torch.float32, device=DEV)
    seed = 0x0123456789ABCDEF
    keep, keys = nx.nx_reservoir_select(cfg, w, 10, seed, workspace=ws, layer=7, step=3,
                                        seq_id=2, with_keys=True)
    nx.nx_read_device_status(cfg, ws)
    keys = keys.cpu().numpy()
    for h in range(h_kv):
        u = philox.uniforms(np.arange(n, dtype=np.uint64), 2 * h_kv + h, 7, 3, seed)
        ref = np.log(u)
        # A wrong uniform would move ln(u) by far more than an ulp; the device
        # log (ocml) and glibc's may differ in the last place (a few percent of
        # inputs), which is all this allows.
        same = keys[h] == ref
        assert same.mean() > 0.9, same.mean()
        np.testing.assert_array_max_ulp(keys[h], ref, maxulp=1)


@pytest.mark.parametrize("n,budget,sink,recent", [
    (1, 1, 0, 0), (7, 3, 0, 0), (100, 100, 0, 0), (100, 250, 0, 0), (1000, 1, 0, 0),
    (4097, 819, 0, 0), (32768, 6554, 0, 0), (5000, 1000, 4, 8), (70000, 13107, 0, 0),
])
def test_reservoir_select_bitexact_on_given_weights(n, budget, sink, recent):
    h_kv = 4
    cfg = _cfg(8, h_kv, 128, 8, n_sink=sink, n_recent=recent)
    ws = _ws(cfg, n, walk=0)
    g = torch.Generator(device="cpu").manual_seed(n * 31 + budget)
    w = (torch.rand(h_kv, n, generator=g) ** 3 / n).float()
    seed = 12345
    keep, keys = nx.nx_reservoir_select(cfg, w.to(DEV), budget, seed, workspace=ws, layer=5,
                                        step=9, seq_id=1, with_keys=True)
    nx.nx_read_device_status(cfg, ws)
    keep = keep.cpu().numpy()
    keys = keys.cpu().numpy()
    ref_keys, ref_keep = nexus.select_from_weights(w.numpy(), budget, seed, layer=5, step=9,
                                                   seq_id=1, n_sink=sink, n_recent=recent)
    for h in range(h_kv):
        # 1 ulp from the device log, 1 more from the correctly rounded divide by w
        np.testing.assert_array_max_ulp(keys[h], ref_keys[h], maxulp=2)
        kept = min(budget, n)
        got = gc.check_keep_valid(keep[h], n, budget)
        # The selection is a function of the keys: select on the GPU's keys ...
        np.testing.assert_array_equal(got, nexus.select_top(keys[h], budget))
        # ... and it matches the oracle's own keys (device log against glibc's: a
        # boundary pair within 2 ulp could swap, nothing else).
        assert len(got) == kept
        gc.assert_flips_within_ulp(got, ref_keep[h], ref_keys[h], kept, 2)


def _weights(kind, h_kv, n, gen):
    """Weight rows that stress the order estimate of the fused select."""
    u = torch.rand(h_kv, n, generator=gen, dtype=torch.float64)
    if kind == "cubic":
        w = u ** 3 / n
    elif kind == "zeros_negative":
        w = u / n
        w[:, ::7] = 0.0
        w[:, 3::11] = -1.0
    elif kind == "subnormal":
        w = u / n
        w[:, ::5] = 1e-40 * (1 + u[:, ::5])
        w[:, 1::13] = 1e-44
    elif kind == "wide_range":
        w = 10.0 ** (-30 * u)
    elif kind == "equal":
        w = torch.full((h_kv, n), 1.0 / n, dtype=torch.float64)
    else:
        raise ValueError(kind)
    return w.float()


@pytest.mark.parametrize("kind", ["cubic", "zeros_negative", "subnormal", "wide_range", "equal"])
@pytest.mark.parametrize("n,budget,sink,recent", [
    (32768, 6554, 0, 0), (20001, 1, 0, 0), (5000, 4999, 0, 0), (9000, 3000, 7, 9), (1000, 250, 0, 0),
    (32769, 6554, 0, 0), (131072, 13107, 5, 7), (262144, 52429, 0, 0), (100003, 99000, 0, 0),
])
def test_estimate_select_equals_exact_select(kind, n, budget, sink, recent):
    """Without a key export the select kernel ranks tokens by an fp32 estimate
    (codes in registers up to 32768 tokens, re-read from memory above) and
    computes fp64 keys only near the boundary; with the export every key is
    exact.  Both must keep exactly the same tokens."""
    h_kv = 8
    cfg = _cfg(8, h_kv, 128, 8, n_sink=sink, n_recent=recent)
    ws = _ws(cfg, n, walk=0)
    gen = torch.Generator(device="cpu").manual_seed(zlib.crc32(f"{kind}/{n}/{budget}".encode()))
    w = _weights(kind, h_kv, n, gen)
    wd = w.to(DEV)
    for step in range(3):
        fast, _ = nx.nx_reservoir_select(cfg, wd, budget, 77, workspace=ws, layer=2, step=step)
        exact, keys = nx.nx_reservoir_select(cfg, wd, budget, 77, workspace=ws, layer=2, step=step,
                                             with_keys=True)
        nx.nx_read_device_status(cfg, ws)
        assert torch.equal(fast, exact), (kind, step)
        k = keys.cpu().numpy()
        for h in range(h_kv):
            np.testing.assert_array_equal(exact[h].cpu().numpy(), nexus.select_top(k[h], budget))


@pytest.mark.parametrize("n", [3000, 40000])
def test_reservoir_select_ties_and_nonpositive_weights(n):
    """Many -inf keys (w <= 0) and duplicates: ties go to the larger index.
    n = 3000 runs the fused keys + select kernel, n = 40000 the two-kernel path."""
    h_kv = 2
    cfg = _cfg(2, h_kv, 64, 4)
    ws = _ws(cfg, n, walk=0)
    w = np.zeros((h_kv, n), dtype=np.float32)
    w[:, ::3] = 1e-3                      # a third positive, the rest -inf keys
    w[1, 5] = -1.0
    for budget in (n // 6, n // 3, n // 2, n - 1):
        keep, _ = nx.nx_reservoir_select(cfg, torch.from_numpy(w).to(DEV), budget, 7, workspace=ws)
        nx.nx_read_device_status(cfg, ws)
        _, ref = nexus.select_from_weights(w, budget, 7)
        for h in range(h_kv):
            np.testing.assert_array_equal(keep[h].cpu().numpy(), ref[h])


def test_reservoir_inclusion_frequencies_match_enumeration():
    """1.2e5 draws of N = 6, B = 2 over independent KV heads and steps vs the exact law."""
    from oracle.enumerate import inclusion_probabilities_float
    n, budget, h_kv = 6, 2, 4096
    cfg = _cfg(h_kv, h_kv, 64, 4)
    ws = _ws(cfg, n, walk=0)
    wv = np.array([0.02, 0.05, 0.1, 0.15, 0.3, 0.38], dtype=np.float32)
    w = torch.from_numpy(np.tile(wv, (h_kv, 1))).to(DEV)
    counts = np.zeros(n)
    draws = 0
    for step in range(30):
        keep, _ = nx.nx_reservoir_select(cfg, w, budget, 99, workspace=ws, step=step)
        k = keep.cpu().numpy()
        np.add.at(counts, k.ravel(), 1)
        draws += h_kv
    nx.nx_read_device_status(cfg, ws)
    freq = counts / draws
    pi = np.array(inclusion_probabilities_float(wv.astype(np.float64), budget))
    sigma = np.sqrt(pi * (1 - pi) / draws)
    assert np.all(np.abs(freq - pi) < 5 * sigma), (freq, pi)


@pytest.mark.parametrize("kind", ["cubic", "zeros_negative", "wide_range", "equal"])
@pytest.mark.parametrize("n_avg", [2, 5, 64, nx.TOPK])
@pytest.mark.parametrize("n,budget,sink,recent", [(32768, 6554, 0, 0), (131072, 13107, 5, 7), (9000, 3000, 7, 9)])
def test_estimate_select_equals_exact_select_averaged(kind, n_avg, n, budget, sink, recent):
    """n >= 2 draws per token (Eq. 6), or the top-B-by-weight limit: the
    select ranks tokens by an fp32 estimate of the key and computes exact keys
    only near the boundary; with the key export every key is exact.  Both
    keep the same tokens."""
    h_kv = 4
    cfg = _cfg(8, h_kv, 128, 8, n_sink=sink, n_recent=recent, n_avg=n_avg)
    ws = _ws(cfg, n, walk=0)
    gen = torch.Generator(device="cpu").manual_seed(zlib.crc32(f"{kind}/{n}/{n_avg}".encode()))
    w = _weights(kind, h_kv, n, gen)
    wd = w.to(DEV)
    for step in range(2):
        fast, _ = nx.nx_reservoir_select(cfg, wd, budget, 31, workspace=ws, layer=1, step=step)
        exact, keys = nx.nx_reservoir_select(cfg, wd, budget, 31, workspace=ws, layer=1, step=step,
                                             with_keys=True)
        nx.nx_read_device_status(cfg, ws)
        assert torch.equal(fast, exact), (kind, n_avg, step)
        k = keys.cpu().numpy()
        for h in range(h_kv):
            np.testing.assert_array_equal(exact[h].cpu().numpy(), nexus.select_top(k[h], budget))


@pytest.mark.parametrize("n", [32768, 20001])
def test_fused_and_two_kernel_selection_agree(n):
    """The selection runs on estimate codes held in registers when max_tokens
    <= 32768, on codes re-read from memory up to 262144, and as exact keys plus
    a global radix select above; the same items must give the same kept rows
    on all three paths."""
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    budget = n // 5
    layers = 2
    data = [gen_layer(wl, device=DEV, n_tokens=n, layer=l) for l in range(layers)]
    outs = []
    for max_tokens in (n, 32769, 262145):
        keep = torch.full((layers, wl.h_kv, budget), -1, dtype=torch.int32, device=DEV)
        ok = torch.empty(layers, wl.h_kv, budget, wl.head_dim, dtype=torch.bfloat16, device=DEV)
        ov = torch.empty_like(ok)
        items = [dict(q=q, k=k, v=v, keep=keep[l], out_k=ok[l], out_v=ov[l],
                      kv_head_stride=n * wl.head_dim, out_head_stride=budget * wl.head_dim,
                      n_tokens=n, budget=budget, layer=l)
                 for l, (q, k, v) in enumerate((d["q"], d["k"], d["v"]) for d in data)]
        units = nx.make_units(items, device=DEV)
        ws = _ws(cfg, max_tokens, layers, wl.walk_iters)
        nx.nx_evict_batch(cfg, units, layers, max_tokens, wl.walk_iters, 3, workspace=ws, step=2,
                          max_out_rows=budget)
        nx.nx_read_device_status(cfg, ws)
        outs.append((keep.clone(), ok.clone(), ov.clone()))
    for l in range(layers):
        for h in range(wl.h_kv):
            gc.check_keep_valid(outs[0][0][l, h].cpu().numpy(), n, budget)
    for other in outs[1:]:
        assert torch.equal(outs[0][0], other[0])
        assert torch.equal(outs[0][1].view(torch.int16), other[1].view(torch.int16))
        assert torch.equal(outs[0][2].view(torch.int16), other[2].view(torch.int16))


# ------------------------------------------ n-averaged priority (Eq. 6) --


@pytest.mark.parametrize("n_avg", [2, 5, 64, nx.TOPK])
@pytest.mark.parametrize("n,budget,sink,recent", [
    (4097, 819, 0, 0), (32768, 6554, 0, 0), (40000, 8000, 3, 5), (50, 7, 0, 0),
])
def test_averaged_priority_on_given_weights(n_avg, n, budget, sink, recent):
    """Keys of Eq. (6) with n draws (and its top-B-by-weight limit) against the
    oracle; the selection is exactly the oracle's selection on the GPU's keys."""
    h_kv = 4
    cfg = _cfg(8, h_kv, 128, 8, n_sink=sink, n_recent=recent, n_avg=n_avg)
    ws = _ws(cfg, n, walk=0)
    g = torch.Generator(device="cpu").manual_seed(zlib.crc32(f"navg/{n_avg}/{n}".encode()))
    w = (torch.rand(h_kv, n, generator=g) ** 3 / n).float()
    w[:, ::17] = 0.0
    keep, keys = nx.nx_reservoir_select(cfg, w.to(DEV), budget, 31, workspace=ws, layer=3,
                                        step=4, seq_id=2, with_keys=True)
    nx.nx_read_device_status(cfg, ws)
    keep, keys = keep.cpu().numpy(), keys.cpu().numpy()
    ref_keys, ref_keep = nexus.select_from_weights(w.numpy(), budget, 31, layer=3, step=4,
                                                   seq_id=2, n_sink=sink, n_recent=recent,
                                                   n_avg=n_avg)
    kept = min(budget, n)
    for h in range(h_kv):
        if n_avg == nx.TOPK:
            np.testing.assert_array_equal(keys[h], ref_keys[h])
        else:
            # device log / exp against glibc: a few ulp after the log-sum-exp
            np.testing.assert_array_max_ulp(keys[h], ref_keys[h], maxulp=16)
        got = gc.check_keep_valid(keep[h], n, budget)
        np.testing.assert_array_equal(got, nexus.select_top(keys[h], budget))
        gc.assert_flips_within_ulp(got, ref_keep[h], ref_keys[h], kept,
                                   0 if n_avg == nx.TOPK else 16)


@pytest.mark.parametrize("n_avg", [5, nx.TOPK])
def test_averaged_priority_end_to_end(n_avg):
    """One event of the llama3 8B layer workload with Eq. (6) at n = 5 and with
    the deterministic limit, through the batched path."""
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, n_avg=n_avg)
    d = gen_layer(wl, device=DEV)
    n, B = wl.n_tokens, wl.budget
    keep = torch.full((wl.h_kv, B), -1, dtype=torch.int32, device=DEV)
    ok = torch.empty(wl.h_kv, B, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    ov = torch.empty_like(ok)
    w_sel = torch.full((wl.h_kv, n), float("nan"), device=DEV)
    units = nx.make_units([dict(q=d["q"], k=d["k"], v=d["v"], keep=keep, out_k=ok, out_v=ov,
                                kv_head_stride=n * wl.head_dim, out_head_stride=B * wl.head_dim,
                                n_tokens=n, budget=B, layer=4, out_w=w_sel)], device=DEV)
    ws = _ws(cfg, n, 1, wl.walk_iters)
    nx.nx_evict_batch(cfg, units, 1, n, wl.walk_iters, 9, workspace=ws, step=6, max_out_rows=B)
    nx.nx_read_device_status(cfg, ws)
    w_gpu = w_sel.cpu().numpy()
    qh, dt = gc.host(d["q"])
    kh, _ = gc.host(d["k"])
    vh, _ = gc.host(d["v"])
    ref = nexus.evict_step(qh, kh, vh, B, wl.walk_iters, 9, dtype=dt, layer=4, step=6,
                           n_avg=n_avg)
    _, on_gpu_w = nexus.select_from_weights(w_gpu, B, 9, layer=4, step=6, n_avg=n_avg)
    for h in range(wl.h_kv):
        got = gc.check_keep_valid(keep[h].cpu().numpy(), n, B)
        gc.assert_weights_close(w_gpu[h], ref["w"][h], f"n_avg {n_avg} head {h}")
        np.testing.assert_array_equal(got, on_gpu_w[h])
        gc.assert_kept_matches_oracle(got, ref["keep"][h], ref["keys"][h], B, f"n_avg {n_avg} head {h}",
                                      n_avg=max(n_avg, 1))
        assert gc.rows_equal(ok[h], d["k"][h], got)
        assert gc.rows_equal(ov[h], d["v"][h], got)


# ------------------------------------------------- block granularity (f2) --


@pytest.mark.parametrize("block,n", [(32, 4096), (8, 4096), (2, 1000), (32, 4001), (16, 300)])
def test_block_mode_end_to_end(block, n):
    """Blocks of b tokens (Eq. 1's BlockSum_b): block weights against the oracle,
    the kept blocks equal the oracle's selection on the GPU's weights, whole
    kept blocks compacted (a short last block when b does not divide N)."""
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, block=block)
    d = gen_layer(wl, device=DEV, n_tokens=n)
    nu = cfg.units(n)
    budget = max(1, round(nu / 5))
    ws = _ws(cfg, n, 1, wl.walk_iters)
    w_only = nx.nx_nexus_weights(cfg, d["q"], d["k"], n, wl.walk_iters, workspace=ws)
    nx.nx_read_device_status(cfg, ws)
    assert tuple(w_only.shape) == (wl.h_kv, nu)
    w_gpu = torch.full((wl.h_kv, nu), float("nan"), device=DEV)
    keep, ok, ov = nx.nx_evict_step(cfg, d["q"], d["k"], d["v"], n, budget, wl.walk_iters, 5,
                                    workspace=ws, layer=1, step=2, out_w=w_gpu)
    nx.nx_read_device_status(cfg, ws)
    qh, dt = gc.host(d["q"])
    kh, _ = gc.host(d["k"])
    vh, _ = gc.host(d["v"])
    ref = nexus.evict_step(qh, kh, vh, budget, wl.walk_iters, 5, dtype=dt, layer=1, step=2,
                           block=block)
    _, on_gpu_w = nexus.select_from_weights(w_gpu.cpu().numpy(), budget, 5, layer=1, step=2)
    for h in range(wl.h_kv):
        gc.assert_weights_close(w_gpu[h].cpu().numpy(), ref["w"][h], f"block {block} head {h}")
        gc.assert_weights_close(w_only[h].cpu().numpy(), ref["w"][h], f"block {block} head {h}")
        got = gc.check_keep_valid(keep[h].cpu().numpy(), nu, budget)
        np.testing.assert_array_equal(got, on_gpu_w[h])
        gc.assert_kept_matches_oracle(got, ref["keep"][h], ref["keys"][h], min(budget, nu),
                                      f"block {block} head {h}")
        rows = np.concatenate([np.arange(b * block, min(b * block + block, n)) for b in got])
        assert gc.rows_equal(ok[h][:len(rows)], d["k"][h], rows)
        assert gc.rows_equal(ov[h][:len(rows)], d["v"][h], rows)


@pytest.mark.parametrize("h_q,window,block,n", [(64, 32, 16, 3000), (64, 64, 32, 2000)])
def test_block_mode_wide_groups(h_q, window, block, n):
    """Blocks with G = 8 query heads per KV head and 256 or 512 window rows:
    the score sweeps run 16-wavefront workgroups (one row tile each)."""
    h_kv, walk = 8, 3
    cfg = _cfg(h_q, h_kv, 128, window, block=block)
    q, k = _synthetic(h_q, h_kv, 128, window, torch.bfloat16, n, seed=4000 + window + block)
    v = torch.randn(k.shape, device=DEV).bfloat16()
    nu = cfg.units(n)
    budget = max(1, round(nu / 5))
    ws = _ws(cfg, n, 1, walk)
    w_gpu = torch.full((h_kv, nu), float("nan"), device=DEV)
    keep, ok, ov = nx.nx_evict_step(cfg, q, k, v, n, budget, walk, 9, workspace=ws, layer=2, step=1,
                                    out_w=w_gpu)
    nx.nx_read_device_status(cfg, ws)
    qh, dt = gc.host(q)
    kh, _ = gc.host(k)
    vh, _ = gc.host(v)
    ref = nexus.evict_step(qh, kh, vh, budget, walk, 9, dtype=dt, layer=2, step=1, block=block,
                           heads=[0, 7])
    _, on_gpu_w = nexus.select_from_weights(w_gpu.cpu().numpy(), budget, 9, layer=2, step=1)
    for h in (0, 7):
        gc.assert_weights_close(w_gpu[h].cpu().numpy(), ref["w"][h], f"block {block} head {h}")
        got = gc.check_keep_valid(keep[h].cpu().numpy(), nu, budget)
        np.testing.assert_array_equal(got, on_gpu_w[h])
        gc.assert_kept_matches_oracle(got, ref["keep"][h], ref["keys"][h], min(budget, nu),
                                      f"block {block} head {h}")
        rows = np.concatenate([np.arange(b * block, min(b * block + block, n)) for b in got])
        assert gc.rows_equal(ok[h][:len(rows)], k[h], rows)
        assert gc.rows_equal(ov[h][:len(rows)], v[h], rows)


def test_block_mode_streaming_appends_after_whole_blocks():
    """Four events of append-256 / evict with blocks of 32 on four layers."""
    from streaming_weighted_sampling_amd.stream import StreamingCache
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, block=32)
    L, n0, A, budget = 4, 4096, 256, 26          # 26 blocks = 832 rows kept
    sc = StreamingCache(cfg, L, n0 + A, budget, A, wl.walk_iters, seed=4, device=DEV)
    k0 = torch.randn(L, wl.h_kv, n0 + A, wl.head_dim, device=DEV).to(torch.bfloat16)
    v0 = torch.randn_like(k0)
    sc.load(k0, v0, n0 + A)
    for step in range(4):
        sc.q.copy_(torch.randn_like(sc.q))
        sc.app_k.copy_(torch.randn_like(sc.app_k))
        sc.app_v.copy_(torch.randn_like(sc.app_v))
        kp, vp = (t.clone() for t in sc.live())
        n_pre = sc.n_tokens
        app_k, app_v = sc.app_k.clone(), sc.app_v.clone()
        sc.step()
        nx.nx_read_device_status(sc.cfg, sc.ws)
        assert sc.n_tokens == budget * 32 + A
        kl, vl = sc.live()
        for l in range(L):
            for h in range(wl.h_kv):
                blocks = sc.keep[l, h].cpu().numpy()
                gc.check_keep_valid(blocks, n_pre // 32, budget)
                rows = np.concatenate([np.arange(b * 32, b * 32 + 32) for b in blocks])
                assert gc.rows_equal(kl[l, h, :budget * 32], kp[l, h], rows)
                assert gc.rows_equal(vl[l, h, :budget * 32], vp[l, h], rows)
            assert torch.equal(kl[l, :, budget * 32:].view(torch.int16), app_k[l].view(torch.int16))


# ------------------------------------------- in-place compaction (f4) --


def test_inplace_step_matches_copy_and_oracle_layout():
    """Same kept set as the copy mode; the caches afterwards equal the oracle's
    hole-filling layout of the original rows (movers from beyond kept)."""
    wl = WORKLOADS["llama3_8b_layer"]
    d = gen_layer(wl, device=DEV)
    n, B = wl.n_tokens, wl.budget
    cfg_copy = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    cfg_in = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, compact=nx.NX_COMPACT_INPLACE)
    ws = _ws(cfg_copy, n, 1, wl.walk_iters)
    keep_c, ok, ov = nx.nx_evict_step(cfg_copy, d["q"], d["k"], d["v"], n, B, wl.walk_iters, 3,
                                      workspace=ws, layer=2, step=1)
    k_in, v_in = d["k"].clone(), d["v"].clone()
    keep_i, k_out, v_out = nx.nx_evict_step(cfg_in, d["q"], k_in, v_in, n, B, wl.walk_iters, 3,
                                            workspace=ws, layer=2, step=1)
    nx.nx_read_device_status(cfg_in, ws)
    assert k_out.data_ptr() == k_in.data_ptr()
    assert torch.equal(keep_c, keep_i)
    kh = d["k"].view(torch.int16).cpu().numpy()
    vh = d["v"].view(torch.int16).cpu().numpy()
    for h in range(wl.h_kv):
        keep = keep_i[h].cpu().numpy()
        exp_k = nexus.compact_inplace(kh[h], keep)
        exp_v = nexus.compact_inplace(vh[h], keep)
        np.testing.assert_array_equal(k_in[h].view(torch.int16).cpu().numpy()[:B], exp_k[:B])
        np.testing.assert_array_equal(v_in[h].view(torch.int16).cpu().numpy()[:B], exp_v[:B])
        # the same rows as the copy mode, permuted
        pos = nexus.inplace_layout(keep, n)
        np.testing.assert_array_equal(exp_k[pos], ok[h].view(torch.int16).cpu().numpy())


def test_inplace_streaming_events_match_oracle():
    """Six append-256 / evict events, in place, on two layers: every event's
    cache equals the oracle's hole filling of the pre-event cache with the GPU's
    keep, and the keep matches the oracle's selection on the GPU's weights."""
    from streaming_weighted_sampling_amd.stream import StreamingCache
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    L, A, B = 2, 256, 819
    n0 = 2048
    sc = StreamingCache(cfg, L, n0, B, A, wl.walk_iters, seed=8, device=DEV, inplace=True,
                        export_w=True)
    k0 = torch.randn(L, wl.h_kv, n0, wl.head_dim, device=DEV).to(torch.bfloat16)
    v0 = torch.randn_like(k0)
    sc.load(k0, v0, n0)
    g = torch.Generator(device="cpu").manual_seed(17)
    for step in range(6):
        sc.q.copy_(torch.randn(sc.q.shape, generator=g).to(torch.bfloat16))
        sc.app_k.copy_(torch.randn(sc.app_k.shape, generator=g).to(torch.bfloat16))
        sc.app_v.copy_(torch.randn(sc.app_v.shape, generator=g).to(torch.bfloat16))
        kp, vp = (t.clone() for t in sc.live())
        n_pre = sc.n_tokens
        sc.step()
        nx.nx_read_device_status(sc.cfg, sc.ws)
        assert sc.n_tokens == B + A
        kl, vl = sc.live()
        for l in range(L):
            keep = sc.keep[l].cpu().numpy()
            w_gpu = sc.weights(l).cpu().numpy()
            qh, dt = gc.host(sc.q[l])
            kh, _ = gc.host(kp[l])
            vh, _ = gc.host(vp[l])
            ref = nexus.evict_step(qh, kh, vh, B, wl.walk_iters, 8, dtype=dt, layer=l, step=step)
            _, on_gpu_w = nexus.select_from_weights(w_gpu, B, 8, layer=l, step=step)
            for h in range(wl.h_kv):
                gc.assert_weights_close(w_gpu[h], ref["w"][h], f"step {step} layer {l} head {h}")
                np.testing.assert_array_equal(keep[h], on_gpu_w[h])
                gc.assert_kept_matches_oracle(keep[h], ref["keep"][h], ref["keys"][h], B,
                                              f"step {step} layer {l} head {h}")
                exp_k = nexus.compact_inplace(kp[l, h].view(torch.int16).cpu().numpy(), keep[h],
                                              sc.app_k[l, h].view(torch.int16).cpu().numpy())
                np.testing.assert_array_equal(kl[l, h].view(torch.int16).cpu().numpy(),
                                              exp_k[:B + A])
                exp_v = nexus.compact_inplace(vp[l, h].view(torch.int16).cpu().numpy(), keep[h],
                                              sc.app_v[l, h].view(torch.int16).cpu().numpy())
                np.testing.assert_array_equal(vl[l, h].view(torch.int16).cpu().numpy(),
                                              exp_v[:B + A])


def _block_rows(blocks, b, n):
    return np.concatenate([np.arange(k * b, min(k * b + b, n)) for k in blocks])


@pytest.mark.parametrize("block,n", [(32, 4096), (32, 4001), (8, 1000)])
def test_inplace_blocks_step_matches_copy_and_oracle_layout(block, n):
    """In-place compaction of kept blocks (a short last block when b does not
    divide N): the same kept blocks and weights as the copy mode, and the caches
    afterwards equal the oracle's hole filling of the kept blocks' rows."""
    wl = WORKLOADS["llama3_8b_layer"]
    d = gen_layer(wl, device=DEV, n_tokens=n)
    cfg_copy = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, block=block)
    cfg_in = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, block=block, compact=nx.NX_COMPACT_INPLACE)
    nu = cfg_copy.units(n)
    B = max(1, round(nu / 5))
    ws = _ws(cfg_copy, n, 1, wl.walk_iters)
    w_c = torch.empty(wl.h_kv, nu, device=DEV)
    w_i = torch.empty_like(w_c)
    keep_c, ok, ov = nx.nx_evict_step(cfg_copy, d["q"], d["k"], d["v"], n, B, wl.walk_iters, 3,
                                      workspace=ws, layer=2, step=1, out_w=w_c)
    k_in, v_in = d["k"].clone(), d["v"].clone()
    keep_i, k_out, v_out = nx.nx_evict_step(cfg_in, d["q"], k_in, v_in, n, B, wl.walk_iters, 3,
                                            workspace=ws, layer=2, step=1, out_w=w_i)
    nx.nx_read_device_status(cfg_in, ws)
    assert k_out.data_ptr() == k_in.data_ptr()
    assert torch.equal(keep_c, keep_i)
    assert torch.equal(w_c.view(torch.int32), w_i.view(torch.int32))
    kh = d["k"].view(torch.int16).cpu().numpy()
    vh = d["v"].view(torch.int16).cpu().numpy()
    kept_rows = cfg_in.kept_rows(n, B)
    for h in range(wl.h_kv):
        rows = _block_rows(keep_i[h].cpu().numpy(), block, n)
        assert len(rows) == kept_rows
        exp_k = nexus.compact_inplace(kh[h], rows)
        exp_v = nexus.compact_inplace(vh[h], rows)
        np.testing.assert_array_equal(k_in[h].view(torch.int16).cpu().numpy()[:kept_rows], exp_k[:kept_rows])
        np.testing.assert_array_equal(v_in[h].view(torch.int16).cpu().numpy()[:kept_rows], exp_v[:kept_rows])
        pos = nexus.inplace_layout(rows, n)
        np.testing.assert_array_equal(exp_k[pos], ok[h][:kept_rows].view(torch.int16).cpu().numpy())


def test_inplace_blocks_streaming_events_match_oracle():
    """Four append-256 / evict-to-26-blocks events with blocks of 32, in place,
    on two layers: each event's kept blocks equal the oracle's selection on the
    exported block weights and share the stated bar with the pure oracle, and
    the cache equals the oracle's hole filling with the new rows after it."""
    from streaming_weighted_sampling_amd.stream import StreamingCache
    wl = WORKLOADS["llama3_8b_layer"]
    b = 32
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, block=b)
    L, A, B, n0 = 2, 256, 26, 4096
    sc = StreamingCache(cfg, L, n0, B, A, wl.walk_iters, seed=12, device=DEV, inplace=True,
                        export_w=True)
    g = torch.Generator(device="cpu").manual_seed(21)
    k0 = torch.randn(L, wl.h_kv, n0, wl.head_dim, generator=g).to(torch.bfloat16).to(DEV)
    v0 = torch.randn(L, wl.h_kv, n0, wl.head_dim, generator=g).to(torch.bfloat16).to(DEV)
    sc.load(k0, v0, n0)
    for step in range(4):
        sc.q.copy_(torch.randn(sc.q.shape, generator=g).to(torch.bfloat16))
        sc.app_k.copy_(torch.randn(sc.app_k.shape, generator=g).to(torch.bfloat16))
        sc.app_v.copy_(torch.randn(sc.app_v.shape, generator=g).to(torch.bfloat16))
        kp, vp = (t.clone() for t in sc.live())
        n_pre = sc.n_tokens
        sc.step()
        nx.nx_read_device_status(sc.cfg, sc.ws)
        assert sc.n_tokens == B * b + A
        kl, vl = sc.live()
        for l in range(L):
            keep = sc.keep[l].cpu().numpy()
            w_gpu = sc.weights(l).cpu().numpy()
            qh, dt = gc.host(sc.q[l])
            kh, _ = gc.host(kp[l])
            vh, _ = gc.host(vp[l])
            ref = nexus.evict_step(qh, kh, vh, B, wl.walk_iters, 12, dtype=dt, layer=l, step=step,
                                   block=b)
            _, on_gpu_w = nexus.select_from_weights(w_gpu, B, 12, layer=l, step=step)
            for h in range(wl.h_kv):
                gc.assert_weights_close(w_gpu[h], ref["w"][h], f"step {step} layer {l} head {h}")
                np.testing.assert_array_equal(keep[h], on_gpu_w[h])
                gc.assert_kept_matches_oracle(keep[h], ref["keep"][h], ref["keys"][h], B,
                                              f"step {step} layer {l} head {h}")
                rows = _block_rows(keep[h], b, n_pre)
                for src, dst, app in ((kp, kl, sc.app_k), (vp, vl, sc.app_v)):
                    exp = nexus.compact_inplace(src[l, h].view(torch.int16).cpu().numpy(), rows,
                                                app[l, h].view(torch.int16).cpu().numpy())
                    np.testing.assert_array_equal(dst[l, h].view(torch.int16).cpu().numpy(),
                                                  exp[:B * b + A])


# --------------------------------------------------------------- compaction --

@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_kv_compact_bitexact(dtype, d):
    h_kv, n, budget = 8, 5000, 1001
    cfg = _cfg(8, h_kv, d, 4, dtype)
    ws = _ws(cfg, n, walk=0)
    k = torch.randn(h_kv, n, d, device=DEV).to(dtype)
    v = torch.randn(h_kv, n, d, device=DEV).to(dtype)
    g = torch.Generator(device="cpu").manual_seed(1)
    keep = torch.stack([torch.randperm(n, generator=g)[:budget].sort().values for _ in range(h_kv)])
    keep = keep.to(torch.int32).to(DEV)
    out_k, out_v = nx.nx_kv_compact(cfg, k, v, keep, n, budget, workspace=ws)
    nx.nx_read_device_status(cfg, ws)
    for h in range(h_kv):
        assert gc.rows_equal(out_k[h], k[h], keep[h].cpu())
        assert gc.rows_equal(out_v[h], v[h], keep[h].cpu())


def test_kv_compact_rejects_out_of_range_index():
    cfg = _cfg(2, 2, 128, 4)
    ws = _ws(cfg, 100, walk=0)
    k = torch.randn(2, 100, 128, device=DEV).bfloat16()
    keep = torch.arange(20, dtype=torch.int32, device=DEV).repeat(2, 1)
    keep[1, 7] = 100
    nx.nx_kv_compact(cfg, k, k.clone(), keep, 100, 20, workspace=ws)
    with pytest.raises(nx.NexusError) as e:
        nx.nx_read_device_status(cfg, ws)
    assert e.value.code == nx.NX_EINVAL


# ------------------------------------------------------------------ scoring --

SCORE_CASES = [
    # name, h_q, h_kv, d, W, dtype, N, walk
    ("tiny_f32", 1, 1, 64, 16, torch.float32, 512, 3),
    ("tiny_f32_ragged", 1, 1, 64, 16, torch.float32, 1000, 3),
    ("llama_layer", 32, 8, 128, 32, torch.bfloat16, 4096, 3),
    ("llama_ragged_h0", 32, 8, 128, 32, torch.bfloat16, 4100, 0),
    ("llama_h1", 32, 8, 128, 32, torch.bfloat16, 777, 1),
    ("llama_h5", 32, 8, 128, 32, torch.bfloat16, 3000, 5),
    ("llama_h6", 32, 8, 128, 32, torch.bfloat16, 2222, 6),
    ("llama_h7", 32, 8, 128, 32, torch.bfloat16, 1999, 7),
    ("g8_w64", 64, 8, 128, 64, torch.bfloat16, 2000, 3),
    ("g8_w32_h4", 64, 8, 128, 32, torch.bfloat16, 2500, 4),
    ("g4_w48_h8", 32, 8, 128, 48, torch.bfloat16, 1700, 8),
    ("g8_w32_lds_h6", 64, 8, 128, 32, torch.bfloat16, 1900, 6),
    ("g2_w16_h5", 16, 8, 128, 16, torch.bfloat16, 3000, 5),
    ("g16_w8_h4_64walkrows", 128, 8, 128, 8, torch.bfloat16, 2100, 4),
    ("mha_w32_h3", 8, 8, 128, 32, torch.bfloat16, 2600, 3),
    ("f32_d128_g4", 32, 8, 128, 32, torch.float32, 1500, 3),
    # fp32 above 4 row tiles: eight wavefronts of two tiles each (the fp32
    # D = 128 forms of these kernels hold part of their state in scratch)
    ("f32_d128_g8_w32", 64, 8, 128, 32, torch.float32, 1300, 3),
    ("f32_d64_g8_w64_h5", 64, 8, 64, 64, torch.float32, 900, 5),
    ("bf16_d64_g8_w64", 64, 8, 64, 64, torch.bfloat16, 1800, 3),
    ("bf16_d64", 16, 4, 64, 8, torch.bfloat16, 1500, 8),
    ("one_token", 4, 2, 128, 4, torch.bfloat16, 1, 2),
    # 64 KV heads x 3 tiles of 2048 tokens, ragged tail: many workgroups per head unit
    ("many_heads_ragged", 256, 64, 128, 32, torch.bfloat16, 5000, 3),
    # deep walks (section 2.2 Eq. 4 with any H <= W): walk rows stored by the
    # second sweep, Gram in its own pass
    ("deep_g4_h12", 32, 8, 128, 32, torch.bfloat16, 3000, 12),
    ("deep_g4_h32_every_row", 32, 8, 128, 32, torch.bfloat16, 2100, 32),
    ("deep_g8_h16", 64, 8, 128, 32, torch.bfloat16, 1800, 16),
    ("deep_g16_h5_80_walk_rows", 128, 8, 128, 8, torch.bfloat16, 1500, 5),
    ("deep_g1_h40", 8, 8, 128, 48, torch.bfloat16, 2600, 40),
    ("deep_g2_h64", 16, 8, 64, 64, torch.bfloat16, 2000, 64),
    ("deep_g32_h9", 32, 1, 128, 16, torch.bfloat16, 1000, 9),
    ("deep_f32_g4_h10", 8, 2, 64, 16, torch.float32, 1500, 10),
    ("deep_ragged_many_chunks", 32, 8, 128, 32, torch.bfloat16, 9001, 20),
]


def _synthetic(h_q, h_kv, d, W, dtype, n, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(h_q, W, d, generator=g, device=DEV)
    k = torch.randn(h_kv, n, d, generator=g, device=DEV)
    k[:, :, :4] *= 8.0                     # outlier channels
    return q.to(dtype), k.to(dtype)


@pytest.mark.parametrize("case", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_nexus_weights_match_oracle(case):
    name, h_q, h_kv, d, W, dtype, n, walk = case
    cfg = _cfg(h_q, h_kv, d, W, dtype)
    ws = _ws(cfg, n, walk=walk)
    q, k = _synthetic(h_q, h_kv, d, W, dtype, n, seed=zlib.crc32(name.encode()))
    w = nx.nx_nexus_weights(cfg, q, k, n, walk, workspace=ws)
    nx.nx_read_device_status(cfg, ws)
    heads = range(h_kv) if h_kv <= 8 else [0, 1, h_kv // 2, h_kv - 2, h_kv - 1]
    ref = gc.oracle_weights(q, k, n, walk, h_q // h_kv, heads=heads)
    for h in heads:
        gc.assert_weights_close(w[h].cpu().numpy(), ref[h], f"{name} head {h}")


def test_workload_weights_match_oracle():
    """The planted tiny and Llama-layer workloads, through nx_nexus_weights."""
    for name in ("tiny_mha_f32", "llama3_8b_layer"):
        wl = WORKLOADS[name]
        x = gen_layer(wl, device=DEV)
        cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window,
                   torch.float32 if wl.dtype == "f32" else torch.bfloat16)
        ws = _ws(cfg, wl.n_tokens, walk=wl.walk_iters)
        w = nx.nx_nexus_weights(cfg, x["q"], x["k"], wl.n_tokens, wl.walk_iters, workspace=ws)
        nx.nx_read_device_status(cfg, ws)
        ref = gc.oracle_weights(x["q"], x["k"], wl.n_tokens, wl.walk_iters, wl.group)
        for h in range(wl.h_kv):
            gc.assert_weights_close(w[h].cpu().numpy(), ref[h], f"{name} head {h}")


# -------------------------------------------------------------- end to end --

def _end_to_end(wl_name, n=None, budget=None, walk=None, seed=0, layer=0, step=0, sink=0, recent=0):
    """One nx_evict_step against the oracle: the exported weights within 1e-3,
    the kept set equal to the oracle's selection on those weights, the pure
    oracle's kept set within the stated bar, compacted rows byte-exact."""
    wl = WORKLOADS[wl_name]
    n = wl.n_tokens if n is None else n
    budget = wl.budget if budget is None else budget
    walk = wl.walk_iters if walk is None else walk
    dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    x = gen_layer(wl, device=DEV, n_tokens=n)
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, dtype, n_sink=sink, n_recent=recent)
    ws = _ws(cfg, n, walk=walk)
    w_sel = torch.full((wl.h_kv, n), float("nan"), device=DEV)
    keep, ok, ov = nx.nx_evict_step(cfg, x["q"], x["k"], x["v"], n, budget, walk, seed,
                                    workspace=ws, layer=layer, step=step, out_w=w_sel)
    nx.nx_read_device_status(cfg, ws)
    # The weights-only entry point scores the same way.
    w_only = nx.nx_nexus_weights(cfg, x["q"], x["k"], n, walk, workspace=ws)
    nx.nx_read_device_status(cfg, ws)
    qh, dt = gc.host(x["q"])
    kh, _ = gc.host(x["k"])
    vh, _ = gc.host(x["v"])
    ref = nexus.evict_step(qh, kh, vh, budget, walk, seed, dtype=dt, layer=layer, step=step,
                           n_sink=sink, n_recent=recent)
    w_sel = w_sel.cpu().numpy()
    _, on_gpu_w = nexus.select_from_weights(w_sel, budget, seed, layer=layer, step=step,
                                            n_sink=sink, n_recent=recent)
    keep = keep.cpu().numpy()
    kept = min(budget, n)
    for h in range(wl.h_kv):
        got = gc.check_keep_valid(keep[h], n, budget)
        gc.assert_weights_close(w_sel[h], ref["w"][h], f"{wl_name} head {h}")
        gc.assert_weights_close(w_only[h].cpu().numpy(), ref["w"][h], f"{wl_name} head {h} (weights only)")
        np.testing.assert_array_equal(got, on_gpu_w[h])
        gc.assert_kept_matches_oracle(got, ref["keep"][h], ref["keys"][h], kept, f"{wl_name} head {h}")
        assert gc.rows_equal(ok[h], x["k"][h], got)
        assert gc.rows_equal(ov[h], x["v"][h], got)
    return keep


def test_evict_step_tiny_f32():
    _end_to_end("tiny_mha_f32")


def test_evict_step_llama_layer():
    _end_to_end("llama3_8b_layer", layer=3, step=11, seed=42)


def test_evict_step_forced_slots_and_edges():
    _end_to_end("llama3_8b_layer", n=2000, budget=400, sink=4, recent=16)
    _end_to_end("llama3_8b_layer", n=300, budget=300)       # B == N keeps all
    _end_to_end("llama3_8b_layer", n=300, budget=1000)      # B > N keeps all
    _end_to_end("llama3_8b_layer", n=1, budget=1)
    _end_to_end("llama3_8b_layer", n=999, budget=1)
    _end_to_end("tiny_mha_f32", walk=0)


@pytest.mark.parametrize("walk", [12, 32])
def test_evict_step_deep_walk(walk):
    """Walks deeper than the register-held forms (H = 12, and H = W = 32: every
    window row), end to end."""
    _end_to_end("llama3_8b_layer", n=4096, walk=walk, seed=13, layer=2, step=4)


@pytest.mark.parametrize("block,walk,n", [(32, 16, 4096), (8, 24, 3001)])
def test_block_mode_deep_walk(block, walk, n):
    """Blocks with a deep walk: the stored walk rows are block sums, the Gram
    pass runs over block units."""
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = _cfg(wl.h_q, wl.h_kv, wl.head_dim, wl.window, block=block)
    d = gen_layer(wl, device=DEV, n_tokens=n)
    nu = cfg.units(n)
    budget = max(1, round(nu / 5))
    ws = _ws(cfg, n, 1, walk)
    w_gpu = torch.full((wl.h_kv, nu), float("nan"), device=DEV)
    keep, ok, ov = nx.nx_evict_step(cfg, d["q"], d["k"], d["v"], n, budget, walk, 6,
                                    workspace=ws, layer=1, step=3, out_w=w_gpu)
    nx.nx_read_device_status(cfg, ws)
    qh, dt = gc.host(d["q"])
    kh, _ = gc.host(d["k"])
    vh, _ = gc.host(d["v"])
    ref = nexus.evict_step(qh, kh, vh, budget, walk, 6, dtype=dt, layer=1, step=3, block=block)
    _, on_gpu_w = nexus.select_from_weights(w_gpu.cpu().numpy(), budget, 6, layer=1, step=3)
    for h in range(wl.h_kv):
        gc.assert_weights_close(w_gpu[h].cpu().numpy(), ref["w"][h], f"block {block} head {h}")
        got = gc.check_keep_valid(keep[h].cpu().numpy(), nu, budget)
        np.testing.assert_array_equal(got, on_gpu_w[h])
        gc.assert_kept_matches_oracle(got, ref["keep"][h], ref["keys"][h], min(budget, nu),
                                      f"block {block} head {h}")
        rows = np.concatenate([np.arange(b * block, min(b * block + block, n)) for b in got])
        assert gc.rows_equal(ok[h][:len(rows)], d["k"][h], rows)
        assert gc.rows_equal(ov[h][:len(rows)], d["v"][h], rows)


def test_evict_step_is_deterministic():
    a = _end_to_end("llama3_8b_layer", n=4096, seed=5)
    b = _end_to_end("llama3_8b_layer", n=4096, seed=5)
    np.testing.assert_array_equal(a, b)


def test_nonfinite_input_sets_device_status():
    cfg = _cfg(8, 2, 128, 8)
    n = 1000
    ws = _ws(cfg, n)
    q, k = _synthetic(8, 2, 128, 8, torch.bfloat16, n, seed=3)
    k[1, 17, 5] = float("nan")
    nx.nx_evict_step(cfg, q, k, k.clone(), n, 100, 3, 0, workspace=ws)
    with pytest.raises(nx.NexusError) as e:
        nx.nx_read_device_status(cfg, ws)
    assert e.value.code == nx.NX_ENONFINITE
    nx.nx_read_device_status(cfg, ws)       # the status word was cleared


def test_stats_overflow_fallback():
    """Logits far above the first tile's max take the exact fallback sweep."""
    cfg = _cfg(4, 1, 128, 4)
    n = 600
    ws = _ws(cfg, n)
    q = torch.zeros(4, 4, 128, device=DEV)
    q[:, :, 0] = 1.0
    k = torch.zeros(1, n, 128, device=DEV)
    k[0, :, 0] = torch.linspace(-50, 1100, n, device=DEV)   # logits up to ~97 nats apart per row
    q, k = q.bfloat16(), k.bfloat16()
    w = nx.nx_nexus_weights(cfg, q, k, n, 2, workspace=ws)
    nx.nx_read_device_status(cfg, ws)
    ref = gc.oracle_weights(q, k, n, 2, 4)
    gc.assert_weights_close(w[0].cpu().numpy(), ref[0], "overflow fallback")


@pytest.mark.parametrize("n_hi", [4000, 8000, 16000])
def test_many_small_head_units_select(n_hi):
    """Batches of 512 head units (64 items x 8 KV heads) with ragged N up to
    4000, 8000 and 16000: the selection runs 512-lane workgroups (8, 16 and 32
    codes per lane).  Every head's kept set equals the oracle's selection on
    the weights the batch exported, and each item's first head matches the
    pure oracle at the stated bar."""
    h_q, h_kv, d, W, walk = 32, 8, 128, 32, 3
    cfg = _cfg(h_q, h_kv, d, W)
    rng = np.random.default_rng(n_hi)
    lens = rng.integers(n_hi // 4, n_hi + 1, size=64)
    lens[0] = n_hi
    items, bufs = [], []
    for i, n in enumerate(lens.tolist()):
        q, k = _synthetic(h_q, h_kv, d, W, torch.bfloat16, n, seed=7000 + i)
        v = torch.randn(k.shape, device=DEV).bfloat16()
        B = max(1, round(n / 5))
        keep = torch.full((h_kv, B), -7, dtype=torch.int32, device=DEV)
        ok = torch.empty(h_kv, B, d, dtype=torch.bfloat16, device=DEV)
        ov = torch.empty_like(ok)
        w = torch.full((h_kv, n), float("nan"), device=DEV)
        bufs.append((q, k, v, keep, w, n, B))
        items.append(dict(q=q, k=k, v=v, keep=keep, out_k=ok, out_v=ov, kv_head_stride=n * d,
                          out_head_stride=B * d, n_tokens=n, budget=B, layer=i % 7, seq_id=i,
                          out_w=w))
    units = nx.make_units(items, device=DEV)
    ws = _ws(cfg, n_hi, len(items), walk)
    nx.nx_evict_batch(cfg, units, len(items), n_hi, walk, 21, workspace=ws, step=4,
                      max_out_rows=round(n_hi / 5))
    nx.nx_read_device_status(cfg, ws)
    for i, (q, k, v, keep, w, n, B) in enumerate(bufs):
        wh = w.cpu().numpy()
        _, on_w = nexus.select_from_weights(wh, B, 21, layer=i % 7, step=4, seq_id=i)
        kh = keep.cpu().numpy()
        for h in range(h_kv):
            np.testing.assert_array_equal(kh[h], on_w[h], err_msg=f"item {i} head {h}")
        if i % 8 == 0:
            qh, dt = gc.host(q)
            kk, _ = gc.host(k)
            vv, _ = gc.host(v)
            ref = nexus.evict_step(qh, kk, vv, B, walk, 21, dtype=dt, layer=i % 7, step=4,
                                   seq_id=i, heads=[0])
            gc.assert_weights_close(wh[0], ref["w"][0], f"item {i}")
            gc.assert_kept_matches_oracle(kh[0], ref["keep"][0], ref["keys"][0], min(B, n),
                                          f"item {i}")
