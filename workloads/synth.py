"""Seeded synthetic KV caches and query windows shaped like the pages' workloads.

The pages evaluate on LongBench, RULER and an agentic coding benchmark with
trained models ([Nexus] section 5.1); none of that is used here.  Instead these
generators draw i.i.d. Gaussian queries and keys and plant the structure the
method is about: heavy hitters (keys aligned with every window query),
bridge keys (aligned with the heavy hitters but nearly orthogonal to the
queries), a few large outlier channels in K, and for the ragged batch a
heavy-tailed Zipf(1.1) salience (about 80% of the attention mass on ~15% of
the positions, the shape of [Nexus] Figure 1).

All generation runs in torch on the requested device with a seeded
torch.Generator, so it is deterministic per (workload, layer, sequence, step)
and device.  bf16 workloads are rounded to bf16 once; consumers that need
exact values read the rounded tensors back.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # data seed
    n_layers: int
    n_seqs: int
    h_q: int
    h_kv: int
    head_dim: int
    window: int
    walk_iters: int
    dtype: str                 # "bf16" or "f32"
    n_tokens: int              # resident tokens (0 for ragged: see ragged_lengths)
    budget: int                # kept tokens per KV head (0: derived per sequence)
    heavy_hitters: int = 0     # planted per KV head
    bridges: int = 0           # planted per KV head
    outlier_channels: int = 0  # K channels scaled by `outlier_scale`
    outlier_scale: float = 8.0
    zipf: float = 0.0          # Zipf exponent of token salience (0: none)
    ragged_range: tuple = ()   # (lo, hi) inclusive, for ragged batches
    stream_steps: int = 0      # streaming events (append then evict)
    stream_append: int = 0     # tokens appended per event
    budget_divisor: int = 5    # ragged budget = round(N / divisor)
    notes: str = field(default="", compare=False)

    @property
    def group(self):
        return self.h_q // self.h_kv


WORKLOADS = {
    # 1: one head, fp32, tiny; the size the oracle finishes instantly.
    "tiny_mha_f32": Workload(
        "tiny_mha_f32", 1, 1, 1, 1, 1, 64, 16, 3, "f32", 512, 128,
        heavy_hitters=8, bridges=8),
    # 2: one Llama-3-8B-shaped layer (GQA 32:8, head_dim 128).
    "llama3_8b_layer": Workload(
        "llama3_8b_layer", 2, 1, 1, 32, 8, 128, 32, 3, "bf16", 4096, 819,
        heavy_hitters=41, bridges=41, outlier_channels=4),
    # 3: all 32 layers, cache at 32K, then 100 append-256 / evict events.
    "llama3_8b_stream32": Workload(
        "llama3_8b_stream32", 3, 32, 1, 32, 8, 128, 32, 3, "bf16", 32768, 6554,
        heavy_hitters=328, bridges=328, outlier_channels=4,
        stream_steps=100, stream_append=256),
    # 4: 16 ragged sequences of 4K..16K tokens, 32 layers, Zipf salience.
    "ragged16_zipf": Workload(
        "ragged16_zipf", 4, 32, 16, 32, 8, 128, 32, 5, "bf16", 0, 0,
        zipf=1.1, ragged_range=(4096, 16384)),
    # 5: one GPU's share of a 70B-shaped model: 8 layers, GQA 64:8, 128K tokens.
    "llama70b_share": Workload(
        "llama70b_share", 5, 8, 1, 64, 8, 128, 64, 3, "bf16", 131072, 13107,
        bridges=655, outlier_channels=4, budget_divisor=10),
}


def budget_for(n_tokens, divisor=5):
    """Budget of a ragged sequence: N / divisor rounded half up (80% eviction)."""
    return int(math.floor(n_tokens / divisor + 0.5))


def _seed(*parts):
    """Stable 63-bit seed from small integers."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h ^= (int(p) + 0x632BE59BD9B4E019 + ((h << 6) & 0xFFFFFFFFFFFFFFFF) + (h >> 2))
        h &= 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def ragged_lengths(wl):
    """Per-sequence resident lengths of a ragged workload (seeded, CPU)."""
    lo, hi = wl.ragged_range
    g = _gen("cpu", wl.index, 0xA11, 0)
    return [int(x) for x in torch.randint(lo, hi + 1, (wl.n_seqs,), generator=g)]


def _torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def _plant_head(k, qm, wl, hh_pos, br_pos, zipf_delta, g):
    """Plant heavy hitters, bridges and salience into one KV head's keys (fp32).

    k: [N, D]; qm: [G*W, D] the group's window queries.
    """
    n, d = k.shape
    rows = qm.shape[0]
    m = qm.mean(dim=0)
    m_dir = m / m.norm()
    if rows < d:
        # small [rows, D] pseudo-inverse, computed on the host in fp64
        pinv = torch.linalg.pinv(qm.double().cpu()).float().to(qm.device)   # [D, rows]
        proj_q = pinv @ qm                                       # projector onto span(Q)
    else:
        pinv, proj_q = None, None

    def off_queries(x):
        if proj_q is not None:
            return x - x @ proj_q.T
        return x - (x @ m_dir)[..., None] * m_dir

    if len(hh_pos):
        sigma = ((qm @ k.T) / math.sqrt(d)).std()
        target = 3.0 * sigma * math.sqrt(d)
        if pinv is not None:
            delta = pinv @ torch.full((rows,), float(target), device=k.device)
        else:
            delta = target * m / (m @ m)
        k[hh_pos] += delta
    if len(br_pos):
        if len(hh_pos):
            base = k[hh_pos].mean(dim=0)
        else:
            base = torch.randn(d, generator=g, device=k.device)
        noise = torch.randn(len(br_pos), d, generator=g, device=k.device) * 0.25
        br = off_queries(base[None, :] + noise)
        br = br / br.norm(dim=1, keepdim=True) * math.sqrt(d)
        k[br_pos] = br
    if zipf_delta is not None:
        k += zipf_delta[:, None] * (math.sqrt(d) * m / (m @ m))[None, :]


def fill_layer_(wl, q_out, k_out, v_out, *, layer=0, seq=0, n_tokens=None):
    """Fill preallocated tensors with one (layer, sequence) of the workload.

    q_out: [H_q, W, D]; k_out, v_out: [H_kv, >= N, D] (rows N.. are untouched).
    Everything is drawn on q_out's device.  Returns the planted positions:
    {"heavy": [per-head index tensors], "bridge": [...]}.
    """
    dev = q_out.device
    n = wl.n_tokens if n_tokens is None else n_tokens
    d, W, G = wl.head_dim, wl.window, wl.group
    g = _gen(dev, wl.index, layer, seq, 1)
    q = torch.randn(wl.h_q, W, d, generator=g, device=dev)
    n_hh = wl.heavy_hitters if wl.n_tokens == 0 or n == wl.n_tokens else \
        int(round(wl.heavy_hitters * n / wl.n_tokens))
    n_br = wl.bridges if wl.n_tokens == 0 or n == wl.n_tokens else \
        int(round(wl.bridges * n / wl.n_tokens))
    zipf_delta = None
    if wl.zipf:
        gz = _gen(dev, wl.index, 0xF00, seq, 2)                  # shared by layers, heads
        rank = torch.randperm(n, generator=gz, device=dev).float() + 1.0
        zipf_delta = wl.zipf * torch.log(n / rank)
    planted = {"heavy": [], "bridge": []}
    for h in range(wl.h_kv):
        k = torch.randn(n, d, generator=g, device=dev)
        if wl.outlier_channels:
            ch = torch.randperm(d, generator=g, device=dev)[:wl.outlier_channels]
            k[:, ch] *= wl.outlier_scale
        pos = torch.randperm(n, generator=g, device=dev)
        hh_pos = pos[:min(n_hh, n)]
        br_pos = pos[min(n_hh, n):min(n_hh + n_br, n)]
        qm = q[h * G:(h + 1) * G].reshape(G * W, d)
        _plant_head(k, qm, wl, hh_pos, br_pos, zipf_delta, g)
        k_out[h, :n].copy_(k)
        v_out[h, :n].copy_(torch.randn(n, d, generator=g, device=dev))
        planted["heavy"].append(hh_pos)
        planted["bridge"].append(br_pos)
    q_out.copy_(q)
    return planted


def gen_layer(wl, *, layer=0, seq=0, n_tokens=None, device="cpu", capacity=None):
    """One (layer, sequence) of the workload: dict(q, k, v) in the workload dtype.

    k, v have `capacity` rows per head (default N); rows N.. are zero.
    """
    n = wl.n_tokens if n_tokens is None else n_tokens
    cap = n if capacity is None else capacity
    dt = _torch_dtype(wl)
    q32 = torch.empty(wl.h_q, wl.window, wl.head_dim, device=device)
    k32 = torch.zeros(wl.h_kv, cap, wl.head_dim, device=device)
    v32 = torch.zeros(wl.h_kv, cap, wl.head_dim, device=device)
    planted = fill_layer_(wl, q32, k32, v32, layer=layer, seq=seq, n_tokens=n)
    return {"q": q32.to(dt), "k": k32.to(dt), "v": v32.to(dt), "n_tokens": n,
            "planted": planted}


def gen_model(wl, *, device="cpu", n_tokens=None, seq=0, layers=None, capacity=None):
    """Every layer of one sequence: q [L, H_q, W, D], k and v [L, H_kv, cap, D].

    Rows N.. of each head (up to `capacity`) are zero.  Drawn layer by layer
    through fp32 staging buffers, then rounded to the workload dtype.
    """
    n = wl.n_tokens if n_tokens is None else n_tokens
    cap = n if capacity is None else capacity
    layers = range(wl.n_layers) if layers is None else layers
    L, dt = len(layers), _torch_dtype(wl)
    q = torch.empty(L, wl.h_q, wl.window, wl.head_dim, dtype=dt, device=device)
    k = torch.zeros(L, wl.h_kv, cap, wl.head_dim, dtype=dt, device=device)
    v = torch.zeros_like(k)
    q32 = torch.empty(wl.h_q, wl.window, wl.head_dim, device=device)
    k32 = torch.empty(wl.h_kv, n, wl.head_dim, device=device)
    v32 = torch.empty_like(k32)
    for i, layer in enumerate(layers):
        fill_layer_(wl, q32, k32, v32, layer=layer, seq=seq, n_tokens=n)
        q[i].copy_(q32)
        k[i, :, :n].copy_(k32)
        v[i, :, :n].copy_(v32)
    return q, k, v


def gen_stream_rows(wl, *, layer, step, n_new, device="cpu"):
    """The N(0,1) K and V rows appended at a streaming event: [H_kv, n_new, D] each."""
    g = _gen(device, wl.index, layer, step, 3)
    dt = _torch_dtype(wl)
    k = torch.randn(wl.h_kv, n_new, wl.head_dim, generator=g, device=device)
    v = torch.randn(wl.h_kv, n_new, wl.head_dim, generator=g, device=device)
    return k.to(dt), v.to(dt)


def gen_stream_queries(wl, *, layer, step, device="cpu"):
    """Fresh N(0,1) window queries for a streaming event: [H_q, W, D]."""
    g = _gen(device, wl.index, layer, step, 4)
    q = torch.randn(wl.h_q, wl.window, wl.head_dim, generator=g, device=device)
    return q.to(_torch_dtype(wl))


def bf16_bits(t):
    """Raw bit patterns of a bf16 tensor as a numpy uint16 array (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- survival ----

@dataclass(frozen=True)
class SurvivalSpec:
    """A long streaming run with tracked tokens ([Nexus] section 3; the check its
    summary proposes: survival of low-direct-attention tokens over hundreds of
    eviction events, Nexus against top-K on the same stream).

    Every stream is one Llama-3-8B-shaped layer (GQA 32:8, head_dim 128, bf16)
    that starts with budget + append resident tokens and then runs `events`
    append-then-evict events.  All window queries of KV head h carry a common
    component sqrt(D) * mu_h along a seeded unit direction mu_h, so every key
    has a persistent logit offset k . mu_h (N(0, 1) for ordinary keys).  The
    tracked tokens of class c have that offset set to exactly offsets[c];
    per_class of them per class and KV head sit at seeded positions of the
    initial cache.
    """
    name: str = "survival_stream"
    index: int = 6
    n_streams: int = 16
    h_q: int = 32
    h_kv: int = 8
    head_dim: int = 128
    window: int = 32
    walk_iters: int = 3
    dtype: str = "bf16"
    budget: int = 2048
    append: int = 256
    events: int = 400
    offsets: tuple = (-1.0, -0.5, 0.0, 0.5, 1.0)
    per_class: int = 32

    @property
    def group(self):
        return self.h_q // self.h_kv

    @property
    def n0(self):
        return self.budget + self.append


SURVIVAL = SurvivalSpec()


def _survival_dirs(spec, device):
    """mu [S, H_kv, D]: the seeded unit directions of every stream and KV head."""
    g = _gen(device, spec.index, 0x5A, 0)
    mu = torch.randn(spec.n_streams, spec.h_kv, spec.head_dim, generator=g, device=device)
    return mu / mu.norm(dim=-1, keepdim=True)


def survival_initial(spec, device="cpu"):
    """Initial caches and class labels of a survival run.

    Returns k, v [S, H_kv, n0, D] (spec dtype) and cls [S, H_kv, n0] int64:
    the tracked class of each initial token, -1 for ordinary tokens.
    """
    S, H, D, n0 = spec.n_streams, spec.h_kv, spec.head_dim, spec.n0
    n_cls = len(spec.offsets)
    if n_cls * spec.per_class > n0:
        raise ValueError("more tracked tokens than initial tokens")
    mu = _survival_dirs(spec, device)
    g = _gen(device, spec.index, 0x5B, 0)
    k = torch.randn(S, H, n0, D, generator=g, device=device)
    v = torch.randn(S, H, n0, D, generator=g, device=device)
    cls = torch.full((S, H, n0), -1, dtype=torch.int64, device=device)
    off = torch.tensor(spec.offsets, dtype=torch.float32, device=device)
    for s in range(S):
        for h in range(H):
            pos = torch.randperm(n0, generator=g, device=device)[:n_cls * spec.per_class]
            c = torch.arange(n_cls * spec.per_class, device=device) // spec.per_class
            m = mu[s, h]
            kt = k[s, h, pos]
            kt = kt - (kt @ m)[:, None] * m[None, :] + off[c][:, None] * m[None, :]
            k[s, h, pos] = kt
            cls[s, h, pos] = c
    dt = _torch_dtype(spec)
    return k.to(dt), v.to(dt), cls


def survival_event(spec, step, device="cpu"):
    """Inputs of event `step`: window queries q [S, H_q, W, D] and the rows that
    arrive after it, app_k and app_v [S, H_kv, append, D] (N(0, 1))."""
    S, D, G = spec.n_streams, spec.head_dim, spec.group
    mu = _survival_dirs(spec, device)
    g = _gen(device, spec.index, 0x5C, step)
    q = torch.randn(S, spec.h_q, spec.window, D, generator=g, device=device)
    q += math.sqrt(D) * mu.repeat_interleave(G, dim=1)[:, :, None, :]
    app_k = torch.randn(S, spec.h_kv, spec.append, D, generator=g, device=device)
    app_v = torch.randn(S, spec.h_kv, spec.append, D, generator=g, device=device)
    dt = _torch_dtype(spec)
    return q.to(dt), app_k.to(dt), app_v.to(dt)
