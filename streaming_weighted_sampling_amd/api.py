"""Torch-facing binding of libnexus.so: checks and marshalling, no arithmetic.

Each function mirrors one C entry point of include/nexus.h and takes torch
device tensors; every step of the eviction path runs in the library's HIP
kernels.  Buffers are passed by data_ptr() and work is enqueued on the current
torch stream (or the given one).
"""

import ctypes
from dataclasses import dataclass

import torch

from ._lib import NX_BF16, NX_F32, NxDesc, NxUnit, check, load

_DTYPES = {torch.bfloat16: NX_BF16, torch.float32: NX_F32}


TOPK = -1                     # n_avg value of the deterministic top-B-by-weight limit


@dataclass
class NexusConfig:
    """Shape and parameters shared by the calls of one eviction event."""
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    dtype: torch.dtype = torch.bfloat16
    lam: float = 0.5          # [Nexus] section 5.1 mixing weight
    eps_tie: float = 1e-6     # [Nexus] section 5.1 tie-break magnitude
    n_sink: int = 0
    n_recent: int = 0
    n_avg: int = 1            # [Nexus] Eq. 6 averaging count; TOPK (-1) = deterministic limit
    block: int = 1            # [Nexus] Eq. 1 block size b: 1 = tokens, else 2..32 (power of 2)
    compact: int = 0          # 0: copy kept rows to new buffers; 1: compact k / v in place
    head_alloc: int = 0       # appendix 10 per-head budgets: 0 uniform, 1 given, 2 allocated
    head_floor: int = 0       # per-head floor of the allocation (head_alloc = 2)

    def units(self, n_tokens):
        """Selection units of a head: tokens, or ceil(n_tokens / block) blocks."""
        return -(-n_tokens // self.block)

    def kept_rows(self, n_tokens, budget):
        """Rows of the kept units (at most budget whole blocks, a short last one shorter)."""
        return min(min(budget, self.units(n_tokens)) * self.block, n_tokens)

    def desc(self, workspace=None, *, layer=0, step=0, seq_id=0, kv_head_stride=0,
             out_head_stride=0, max_out_rows=0, stream=None, out_w=None):
        d = NxDesc()
        d.n_q_heads = self.n_q_heads
        d.n_kv_heads = self.n_kv_heads
        d.head_dim = self.head_dim
        d.window = self.window
        d.dtype = _DTYPES.get(self.dtype, 99)
        d.lambda_ = self.lam
        d.eps_tie = self.eps_tie
        d.n_sink = self.n_sink
        d.n_recent = self.n_recent
        d.n_avg = self.n_avg
        d.block = self.block
        d.compact = self.compact
        d.head_alloc = self.head_alloc
        d.head_floor = self.head_floor
        d.out_w = _ptr(out_w)
        d.layer = layer
        d.step = step
        d.seq_id = seq_id
        d.max_out_rows = max_out_rows
        d.kv_head_stride = kv_head_stride
        d.out_head_stride = out_head_stride
        if workspace is not None:
            d.workspace = workspace.data_ptr()
            d.workspace_bytes = workspace.numel() * workspace.element_size()
        d.stream = _stream_handle(stream)
        return d


def _stream_handle(stream):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_cache(cfg, t, name):
    if t.dtype != cfg.dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {cfg.dtype}")
    if t.dim() != 3 or t.shape[0] != cfg.n_kv_heads or t.shape[2] != cfg.head_dim:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [n_kv_heads, rows, head_dim]")
    if t.stride(2) != 1 or t.stride(1) != cfg.head_dim:
        raise ValueError(f"{name}: rows must be contiguous")
    return t.stride(0)


def _check_weights(cfg, w, n_tokens, name):
    if w.dtype != torch.float32 or not w.is_contiguous() or \
            tuple(w.shape) != (cfg.n_kv_heads, cfg.units(n_tokens)):
        raise ValueError(f"{name} must be a contiguous float32 [n_kv_heads, units] tensor")


def workspace_bytes(cfg, max_tokens, max_units=1, walk_iters=3):
    d = cfg.desc()
    n = load().nx_evict_workspace_bytes(ctypes.byref(d), max_tokens, max_units, walk_iters)
    if n == 0:
        raise ValueError("invalid shape for the workspace query")
    return n


def new_workspace(cfg, max_tokens, max_units=1, walk_iters=3, device="cuda"):
    """Zero-filled workspace (the status word must start at zero)."""
    return torch.zeros(workspace_bytes(cfg, max_tokens, max_units, walk_iters),
                       dtype=torch.uint8, device=device)


def nx_evict_step(cfg, q, k, v, n_tokens, budget, walk_iters, seed, *, workspace, layer=0,
                  step=0, seq_id=0, out_k=None, out_v=None, keep=None, out_w=None, stream=None):
    """One eviction event; returns (keep [H_kv, B] int32, out_k, out_v).

    out_w: optional float32 [H_kv, units] tensor that receives the Nexus weights
    the selection used."""
    kst = _check_cache(cfg, k, "k")
    if _check_cache(cfg, v, "v") != kst:
        raise ValueError("k and v must share the head stride")
    if q.dtype != cfg.dtype or not q.is_contiguous() or \
            tuple(q.shape) != (cfg.n_q_heads, cfg.window, cfg.head_dim):
        raise ValueError("q must be a contiguous [n_q_heads, window, head_dim] tensor")
    kept = cfg.kept_rows(n_tokens, budget)
    if cfg.compact:
        # In place: k and v are compacted themselves (their first `kept` rows).
        if out_k is not None or out_v is not None:
            raise ValueError("in-place compaction takes no out_k / out_v")
        ost = 0
    else:
        if out_k is None:
            out_k = torch.empty(cfg.n_kv_heads, max(kept, 1), cfg.head_dim, dtype=cfg.dtype,
                                device=k.device)
        if out_v is None:
            out_v = torch.empty_like(out_k)
        ost = _check_cache(cfg, out_k, "out_k")
        if _check_cache(cfg, out_v, "out_v") != ost:
            raise ValueError("out_k and out_v must share the head stride")
    if keep is None:
        keep = torch.empty(cfg.n_kv_heads, budget, dtype=torch.int32, device=k.device)
    if out_w is not None:
        _check_weights(cfg, out_w, n_tokens, "out_w")
    d = cfg.desc(workspace, layer=layer, step=step, seq_id=seq_id, kv_head_stride=kst,
                 out_head_stride=ost, stream=stream, out_w=out_w)
    check(load().nx_evict_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), n_tokens, budget,
                               walk_iters, seed, _ptr(keep), _ptr(out_k), _ptr(out_v)),
          "nx_evict_step")
    if cfg.compact:
        return keep, k, v
    return keep, out_k, out_v


def nx_evict_step_noalloc(cfg, q, k, v, n_tokens, budget, walk_iters, seed, *, out_k, out_v,
                          keep, layer=0, step=0, seq_id=0, out_w=None, stream=None):
    """nx_evict_step on the library's static scratch (no workspace, nothing
    allocated by the call); every output tensor is given by the caller."""
    kst = _check_cache(cfg, k, "k")
    if _check_cache(cfg, v, "v") != kst:
        raise ValueError("k and v must share the head stride")
    if q.dtype != cfg.dtype or not q.is_contiguous() or \
            tuple(q.shape) != (cfg.n_q_heads, cfg.window, cfg.head_dim):
        raise ValueError("q must be a contiguous [n_q_heads, window, head_dim] tensor")
    ost = 0
    if not cfg.compact:
        ost = _check_cache(cfg, out_k, "out_k")
        if _check_cache(cfg, out_v, "out_v") != ost:
            raise ValueError("out_k and out_v must share the head stride")
    if keep.dtype != torch.int32 or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous int32 tensor")
    if out_w is not None:
        _check_weights(cfg, out_w, n_tokens, "out_w")
    d = cfg.desc(None, layer=layer, step=step, seq_id=seq_id, kv_head_stride=kst,
                 out_head_stride=ost, stream=stream, out_w=out_w)
    check(load().nx_evict_step_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), n_tokens,
                                       budget, walk_iters, seed, _ptr(keep), _ptr(out_k),
                                       _ptr(out_v)), "nx_evict_step_noalloc")
    return keep, out_k, out_v


def nx_nexus_weights(cfg, q, k, n_tokens, walk_iters, *, workspace, out_w=None, stream=None):
    """Nexus weights w [H_kv, units] fp32 (units = n_tokens, or blocks)."""
    kst = _check_cache(cfg, k, "k")
    if out_w is None:
        out_w = torch.empty(cfg.n_kv_heads, cfg.units(n_tokens), dtype=torch.float32, device=k.device)
    d = cfg.desc(workspace, kv_head_stride=kst, stream=stream)
    check(load().nx_nexus_weights(ctypes.byref(d), _ptr(q), _ptr(k), n_tokens, walk_iters,
                                  _ptr(out_w)), "nx_nexus_weights")
    return out_w


def nx_reservoir_select(cfg, w, budget, seed, *, workspace, layer=0, step=0, seq_id=0,
                        with_keys=False, stream=None):
    """Reservoir selection on weights w [H_kv, N] fp32; returns (keep, keys or None)."""
    if w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous [n_kv_heads, n_tokens] float32 tensor")
    n = w.shape[1]
    keep = torch.empty(cfg.n_kv_heads, budget, dtype=torch.int32, device=w.device)
    keys = torch.empty(cfg.n_kv_heads, n, dtype=torch.float64, device=w.device) if with_keys else None
    d = cfg.desc(workspace, layer=layer, step=step, seq_id=seq_id, stream=stream)
    check(load().nx_reservoir_select(ctypes.byref(d), _ptr(w), n, budget, seed, _ptr(keep),
                                     _ptr(keys)), "nx_reservoir_select")
    return keep, keys


def nx_head_budgets(cfg, w, budget, *, workspace, head_cap=0, out=None, stream=None):
    """Per-head budgets allocated on given weights w [H_kv, N] fp32 of one item
    (cfg.head_alloc must be 2); returns int32 [H_kv] on w's device."""
    if w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous [n_kv_heads, n_tokens] float32 tensor")
    if out is None:
        out = torch.empty(cfg.n_kv_heads, dtype=torch.int32, device=w.device)
    d = cfg.desc(workspace, stream=stream)
    check(load().nx_head_budgets(ctypes.byref(d), _ptr(w), w.shape[1], budget, head_cap,
                                 _ptr(out)), "nx_head_budgets")
    return out


def nx_kv_compact(cfg, k, v, keep, n_tokens, budget, *, workspace, out_k=None, out_v=None,
                  stream=None):
    kst = _check_cache(cfg, k, "k")
    kept = cfg.kept_rows(n_tokens, budget)
    if out_k is None:
        out_k = torch.empty(cfg.n_kv_heads, kept, cfg.head_dim, dtype=cfg.dtype, device=k.device)
    if out_v is None:
        out_v = torch.empty_like(out_k)
    ost = _check_cache(cfg, out_k, "out_k")
    if keep.dtype != torch.int32 or not keep.is_contiguous():
        raise ValueError("keep must be contiguous int32 [n_kv_heads, budget]")
    d = cfg.desc(workspace, kv_head_stride=kst, out_head_stride=ost, stream=stream)
    check(load().nx_kv_compact(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(keep), n_tokens, budget,
                               _ptr(out_k), _ptr(out_v)), "nx_kv_compact")
    return out_k, out_v


def make_units(items, device="cuda"):
    """Device array of nx_unit records from a list of dicts (see nx_unit in nexus.h)."""
    arr = (NxUnit * len(items))()
    for rec, it in zip(arr, items):
        for key in ("q", "k", "v", "keep", "out_k", "out_v", "app_k", "app_v", "out_w",
                    "head_tokens", "head_tokens_out"):
            setattr(rec, key, _ptr(it.get(key)))
        rec.kv_head_stride = it["kv_head_stride"]
        rec.out_head_stride = it["out_head_stride"]
        rec.n_tokens = it["n_tokens"]
        rec.budget = it["budget"]
        rec.n_append = it.get("n_append", 0)
        rec.layer = it.get("layer", 0)
        rec.seq_id = it.get("seq_id", 0)
        rec.head_cap = it.get("head_cap", 0)
        rec.head_budget = _ptr(it.get("head_budget"))
    host = torch.frombuffer(bytearray(arr), dtype=torch.uint8)
    return host.to(device)


def nx_evict_batch(cfg, units_dev, n_units, max_tokens, walk_iters, seed, *, workspace, step=0,
                   max_out_rows=0, stream=None):
    d = cfg.desc(workspace, step=step, max_out_rows=max_out_rows, stream=stream)
    check(load().nx_evict_batch(ctypes.byref(d), _ptr(units_dev), n_units, max_tokens,
                                walk_iters, seed), "nx_evict_batch")


def nx_read_device_status(cfg, workspace, stream=None):
    """Synchronises the stream and raises NexusError on a recorded device error
    (workspace None: the status of nx_evict_step_noalloc calls on this device)."""
    d = cfg.desc(workspace, stream=stream)
    check(load().nx_read_device_status(ctypes.byref(d)), "device status")


def profile_enable(on=True, stages=None):
    """Start (clearing earlier records) or stop per-stage HIP-event timing.

    stages: names of the stages to time (None: every stage)."""
    lib = load()
    if not on:
        mask = 0
    elif stages is None:
        mask = -1
    else:
        names = [lib.nx_stage_name(i).decode() for i in range(32)]
        mask = 0
        for st in stages:
            if st not in names:
                raise ValueError(f"unknown stage {st!r}")
            mask |= 1 << names.index(st)
    lib.nx_profile_enable(mask)


def profile_read():
    """{stage name: (total ms, launches)} for the launches recorded since enabling."""
    lib = load()
    ms = (ctypes.c_float * 16)()
    cnt = (ctypes.c_int32 * 16)()
    n = lib.nx_profile_read(ms, cnt, 16)
    return {lib.nx_stage_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}
