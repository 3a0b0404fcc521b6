"""nx_evict_step_noalloc (static scratch, nothing allocated by the call) against
nx_evict_step with a caller workspace: identical kept indices, compacted rows
and exported weights, bit for bit, on two calls in a row, the second smaller."""

import pytest
import torch

import streaming_weighted_sampling_amd as nx
from workloads import WORKLOADS, gen_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(cfg, x, n, budget, walk, seed, layer, step):
    """Run both entry points on the same inputs; return their outputs."""
    outs = []
    for noalloc in (False, True):
        keep = torch.full((cfg.n_kv_heads, budget), -7, dtype=torch.int32, device=DEV)
        kept = cfg.kept_rows(n, budget)
        ok = torch.zeros(cfg.n_kv_heads, kept, cfg.head_dim, dtype=cfg.dtype, device=DEV)
        ov = torch.zeros_like(ok)
        w = torch.full((cfg.n_kv_heads, n), float("nan"), device=DEV)
        k, v = x["k"][:, :n].contiguous(), x["v"][:, :n].contiguous()
        if noalloc:
            nx.nx_evict_step_noalloc(cfg, x["q"], k, v, n, budget, walk, seed, out_k=ok, out_v=ov,
                                     keep=keep, layer=layer, step=step, out_w=w)
            nx.nx_read_device_status(cfg, None)
        else:
            ws = nx.new_workspace(cfg, n, 1, walk, device=DEV)
            nx.nx_evict_step(cfg, x["q"], k, v, n, budget, walk, seed, workspace=ws, layer=layer,
                             step=step, out_k=ok, out_v=ov, keep=keep, out_w=w)
            nx.nx_read_device_status(cfg, ws)
        outs.append((keep, ok, ov, w))
    return outs


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16)
    x = gen_layer(wl, device=DEV)
    for n, budget, walk, seed, layer, step in ((wl.n_tokens, wl.budget, wl.walk_iters, 5, 2, 9),
                                               (1000, 200, 1, 6, 3, 10)):
        (k0, ok0, ov0, w0), (k1, ok1, ov1, w1) = _both(cfg, x, n, budget, walk, seed, layer, step)
        assert torch.equal(k0, k1), n
        assert torch.equal(ok0.view(torch.int16), ok1.view(torch.int16)), n
        assert torch.equal(ov0.view(torch.int16), ov1.view(torch.int16)), n
        assert torch.equal(w0.view(torch.int32), w1.view(torch.int32)), n


def test_noalloc_rejects_shapes_beyond_the_scratch():
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16)
    n, budget = 131072, 26214         # 8 heads x 128K tokens need more than 16 MiB
    assert nx.workspace_bytes(cfg, n, 1, 3) > nx.NX_SCRATCH_BYTES
    q = torch.zeros(wl.h_q, wl.window, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(wl.h_kv, n, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    ok = torch.empty(wl.h_kv, budget, wl.head_dim, dtype=torch.bfloat16, device=DEV)
    ov = torch.empty_like(ok)
    keep = torch.empty(wl.h_kv, budget, dtype=torch.int32, device=DEV)
    with pytest.raises(nx.NexusError) as e:
        nx.nx_evict_step_noalloc(cfg, q, k, v, n, budget, 3, 0, out_k=ok, out_v=ov, keep=keep)
    assert e.value.code == nx.NX_EWORKSPACE
