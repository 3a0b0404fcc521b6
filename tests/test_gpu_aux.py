"""Auxiliary checks on the GPU: canary-padded output buffers (no call writes
outside what it owns) and the NX_DEBUG synchronous-check mode."""

import os

import numpy as np
import pytest
import torch

import streaming_weighted_sampling_amd as nx
from workloads import WORKLOADS, gen_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
PAD = 4096          # canary bytes on each side of every output
CANARY = 0xA5


class Padded:
    """A tensor of `shape` carved out of a byte buffer with canaries around it."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((PAD + n + PAD,), CANARY, dtype=torch.uint8, device=DEV)
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)

    def intact(self):
        head, tail = self.raw[:PAD], self.raw[-PAD:]
        return bool((head == CANARY).all()) and bool((tail == CANARY).all())


def _layer(n):
    wl = WORKLOADS["llama3_8b_layer"]
    return wl, gen_layer(wl, device=DEV, n_tokens=n)


@pytest.mark.parametrize("n,budget", [(4096, 819), (300, 500), (1000, 1)])
def test_evict_step_writes_only_its_outputs(n, budget):
    wl, x = _layer(n)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    kept = min(budget, n)
    keep = Padded((wl.h_kv, budget), torch.int32)
    keep.t.fill_(-77)
    ok = Padded((wl.h_kv, kept, wl.head_dim), torch.bfloat16)
    ov = Padded((wl.h_kv, kept, wl.head_dim), torch.bfloat16)
    w = Padded((wl.h_kv, n), torch.float32)
    ws = nx.new_workspace(cfg, n, 1, wl.walk_iters, device=DEV)
    nx.nx_evict_step(cfg, x["q"], x["k"], x["v"], n, budget, wl.walk_iters, 1, workspace=ws,
                     keep=keep.t, out_k=ok.t, out_v=ov.t, out_w=w.t)
    nx.nx_read_device_status(cfg, ws)
    for name, p in (("keep", keep), ("out_k", ok), ("out_v", ov), ("out_w", w)):
        assert p.intact(), name
    # keep entries past the kept count are left as they were
    assert bool((keep.t[:, kept:] == -77).all())
    assert bool((keep.t[:, :kept] >= 0).all())


def test_ragged_batch_writes_only_its_outputs():
    """Items of different lengths whose outputs sit back to back in shared
    buffers, each slice separated from the next by a canary gap."""
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    lens = [4096, 1500, 33, 2047]
    buffers, items = [], []
    for i, n in enumerate(lens):
        x = gen_layer(wl, device=DEV, n_tokens=n, layer=i)
        b = max(1, n // 5)
        keep = Padded((wl.h_kv, b), torch.int32)
        ok = Padded((wl.h_kv, b, wl.head_dim), torch.bfloat16)
        ov = Padded((wl.h_kv, b, wl.head_dim), torch.bfloat16)
        w = Padded((wl.h_kv, n), torch.float32)
        buffers += [keep, ok, ov, w]
        items.append(dict(q=x["q"], k=x["k"], v=x["v"], keep=keep.t, out_k=ok.t, out_v=ov.t,
                          out_w=w.t, kv_head_stride=n * wl.head_dim,
                          out_head_stride=b * wl.head_dim, n_tokens=n, budget=b, layer=i))
    units = nx.make_units(items, device=DEV)
    ws = nx.new_workspace(cfg, max(lens), len(lens), wl.walk_iters, device=DEV)
    nx.nx_evict_batch(cfg, units, len(lens), max(lens), wl.walk_iters, 4, workspace=ws,
                      max_out_rows=max(lens) // 5)
    nx.nx_read_device_status(cfg, ws)
    assert all(p.intact() for p in buffers)


def test_stage_entry_points_write_only_their_outputs():
    wl, x = _layer(3000)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    n, b = 3000, 600
    ws = nx.new_workspace(cfg, n, 1, wl.walk_iters, device=DEV)
    w = Padded((wl.h_kv, n), torch.float32)
    nx.nx_nexus_weights(cfg, x["q"], x["k"], n, wl.walk_iters, workspace=ws, out_w=w.t)
    keep = Padded((wl.h_kv, b), torch.int32)
    ok = Padded((wl.h_kv, b, wl.head_dim), torch.bfloat16)
    ov = Padded((wl.h_kv, b, wl.head_dim), torch.bfloat16)
    k2, _ = nx.nx_reservoir_select(cfg, w.t.contiguous(), b, 2, workspace=ws)
    keep.t.copy_(k2)
    nx.nx_kv_compact(cfg, x["k"], x["v"], keep.t, n, b, workspace=ws, out_k=ok.t, out_v=ov.t)
    nx.nx_read_device_status(cfg, ws)
    assert w.intact() and keep.intact() and ok.intact() and ov.intact()


@pytest.fixture
def debug_env():
    old = os.environ.get("NX_DEBUG")
    os.environ["NX_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["NX_DEBUG"]
    else:
        os.environ["NX_DEBUG"] = old


def test_debug_mode_matches_the_asynchronous_results(debug_env):
    wl, x = _layer(4096)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    ws = nx.new_workspace(cfg, 4096, 1, wl.walk_iters, device=DEV)
    keep_d, ok_d, _ = nx.nx_evict_step(cfg, x["q"], x["k"], x["v"], 4096, 819, 3, 5, workspace=ws)
    os.environ["NX_DEBUG"] = "0"
    keep_a, ok_a, _ = nx.nx_evict_step(cfg, x["q"], x["k"], x["v"], 4096, 819, 3, 5, workspace=ws)
    nx.nx_read_device_status(cfg, ws)
    assert torch.equal(keep_d, keep_a)
    assert torch.equal(ok_d.view(torch.int16), ok_a.view(torch.int16))


def test_debug_mode_reports_a_device_error_from_the_call_itself(debug_env):
    wl, x = _layer(1000)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window)
    ws = nx.new_workspace(cfg, 1000, 1, wl.walk_iters, device=DEV)
    k = x["k"].clone()
    k[3, 17, 5] = float("nan")
    with pytest.raises(nx.NexusError) as e:
        nx.nx_evict_step(cfg, x["q"], k, x["v"], 1000, 100, 3, 0, workspace=ws)
    assert e.value.code == nx.NX_ENONFINITE
    with pytest.raises(nx.NexusError):
        nx.nx_read_device_status(cfg, ws)      # the word stays set until read
    nx.nx_read_device_status(cfg, ws)          # ... and is cleared by the read
