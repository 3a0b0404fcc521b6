"""Eviction steps captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: every replay must reproduce the eager results bit for bit, with
eager work and synchronisation between replays.  The library records no
memset nodes (its scratch clears are kernels), which this checks in practice."""

import pytest
import torch

import streaming_weighted_sampling_amd as nx
from workloads import WORKLOADS, gen_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager_steps():
    wl = WORKLOADS["llama3_8b_layer"]
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16)
    n, B, H, D = wl.n_tokens, wl.budget, wl.h_kv, wl.head_dim
    x = gen_layer(wl, device=DEV)
    copies = 3
    ks = [x["k"].clone() for _ in range(copies)]
    vs = [x["v"].clone() for _ in range(copies)]
    for c in range(1, copies):           # different caches per copy
        ks[c][:, c::7] = ks[c][:, c::7] * 0.5
    keep = torch.empty(copies, H, B, dtype=torch.int32, device=DEV)
    ok = torch.empty(copies, H, B, D, dtype=torch.bfloat16, device=DEV)
    ov = torch.empty_like(ok)
    w = torch.empty(copies, H, n, device=DEV)
    ws = nx.new_workspace(cfg, n, 1, wl.walk_iters, device=DEV)

    def steps():
        for c in range(copies):
            nx.nx_evict_step(cfg, x["q"], ks[c], vs[c], n, B, wl.walk_iters, 3, workspace=ws,
                             step=c, out_k=ok[c], out_v=ov[c], keep=keep[c], out_w=w[c])

    steps()
    nx.nx_read_device_status(cfg, ws)
    ref = [t.clone() for t in (keep, ok, ov, w)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            steps()
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        for t in (keep, ok, ov, w):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (keep, ok, ov, w)
        for name, a, b in zip(("keep", "out_k", "out_v", "w"), got, ref):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), (r, name)
        # eager work between replays: another step on a different budget
        k2, _, _ = nx.nx_evict_step(cfg, x["q"], ks[0], vs[0], n, B // 2, wl.walk_iters, 9,
                                    workspace=ws)
        nx.nx_read_device_status(cfg, ws)
