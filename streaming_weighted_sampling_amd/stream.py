"""Streaming eviction over every layer: append new rows, then evict back to B.

[Nexus] ("Forget Without Compromise: Nexus Sampling for Streaming KV-Cache
Eviction Under Fixed Budgets", section 2.1) treats eviction as a stream: the
cache grows as tokens arrive and, whenever the budget is hit, keeps B
positions and continues with those rows.  This driver holds two capacity
buffers per layer and ping-pongs between them.  One `step()` is one
nx_evict_batch call over all layers; its compaction also writes the rows
that arrive before the next event right after the kept ones, so a step reads
each resident row once and writes the next cache once.  Marshalling only:
every byte of the path moves inside libnexus.so.
"""

from dataclasses import replace

import torch

from ._lib import NX_HEADS_UNIFORM
from .api import NexusConfig, make_units, new_workspace, nx_evict_batch


class StreamingCache:
    """K/V capacity buffers for `n_layers` layers of one sequence.

    Layout of each buffer: [n_layers, n_kv_heads, capacity, head_dim].
    `capacity` must hold max(initial tokens, budget + n_append).  With
    inplace=False two buffers ping-pong and the kept rows stay in cache
    order; with inplace=True one buffer is compacted in place (hole filling:
    only the kept rows past the kept count move, then the new rows follow), so
    an event writes about n_append rows per head instead of budget.
    With export_w=True every event also writes the Nexus weights its selection
    used (read them back with weights()).

    Per-head budgets ([Nexus] appendix 10; cfg.head_alloc = 2 allocates them
    every event, 1 reads them from head_budget[layer]): each head keeps up to
    head_cap units (0: budget), so after an event the heads hold different
    row counts.  Those counts stay on the device (two [n_layers, n_kv_heads]
    int32 arrays, written by one event and read by the next); n_tokens is
    then the host's bound on them and head_tokens() reads them back.
    """

    def __init__(self, cfg: NexusConfig, n_layers, capacity, budget, n_append, walk_iters,
                 seed=0, seq_id=0, device="cuda", inplace=False, export_w=False, head_cap=0):
        if inplace:
            cfg = replace(cfg, compact=1)
        self.inplace = inplace
        self.cfg, self.n_layers, self.capacity = cfg, n_layers, capacity
        self.budget, self.n_append, self.walk_iters = budget, n_append, walk_iters
        self.seed, self.seq_id, self.device = seed, seq_id, device
        self.per_head = cfg.head_alloc != NX_HEADS_UNIFORM
        self.cap = (head_cap if head_cap > 0 else budget) if self.per_head else budget
        shape = (n_layers, cfg.n_kv_heads, capacity, cfg.head_dim)
        nbuf = 1 if inplace else 2
        self.k = [torch.zeros(shape, dtype=cfg.dtype, device=device) for _ in range(nbuf)]
        self.v = [torch.zeros(shape, dtype=cfg.dtype, device=device) for _ in range(nbuf)]
        self.q = torch.zeros(n_layers, cfg.n_q_heads, cfg.window, cfg.head_dim, dtype=cfg.dtype,
                             device=device)
        self.app_k = torch.zeros(n_layers, cfg.n_kv_heads, n_append, cfg.head_dim,
                                 dtype=cfg.dtype, device=device)
        self.app_v = torch.zeros_like(self.app_k)
        self.keep = torch.zeros(n_layers, cfg.n_kv_heads, self.cap, dtype=torch.int32,
                                device=device)
        if self.per_head:
            self.head_budget = torch.zeros(n_layers, cfg.n_kv_heads, dtype=torch.int32,
                                           device=device)
            self.tokens = [torch.zeros(n_layers, cfg.n_kv_heads, dtype=torch.int32, device=device)
                           for _ in range(2)]
        self.tcur = 0         # which count array holds the live per-head counts
        self.w = (torch.zeros(n_layers, cfg.n_kv_heads * cfg.units(capacity), dtype=torch.float32,
                              device=device) if export_w else None)
        self.last_units = 0   # selection units per head of the last event
        self.ws = new_workspace(cfg, capacity, n_layers, walk_iters, device=device)
        self.cur = 0          # which buffer holds the live cache
        self.n_tokens = 0     # live rows per head
        self.step_no = 0
        self._units = {}

    def load(self, k, v, n_tokens):
        """Initial cache: k, v [n_layers, n_kv_heads, n_tokens, head_dim]."""
        self.k[self.cur][:, :, :n_tokens].copy_(k)
        self.v[self.cur][:, :, :n_tokens].copy_(v)
        self.n_tokens = n_tokens
        if self.per_head:
            self.tokens[self.tcur].fill_(n_tokens)

    def _units_for(self, src, n_tokens):
        key = (src, n_tokens, self.tcur)
        if key not in self._units:
            dst = src if self.inplace else 1 - src
            rows = self.capacity * self.cfg.head_dim
            out_k = None if self.inplace else self.k[dst]
            out_v = None if self.inplace else self.v[dst]
            items = [dict(q=self.q[l], k=self.k[src][l], v=self.v[src][l], keep=self.keep[l],
                          out_k=None if out_k is None else out_k[l],
                          out_v=None if out_v is None else out_v[l], app_k=self.app_k[l],
                          app_v=self.app_v[l], kv_head_stride=rows, out_head_stride=rows,
                          n_tokens=n_tokens, budget=self.budget, n_append=self.n_append,
                          layer=l, seq_id=self.seq_id,
                          out_w=None if self.w is None else self.w[l])
                     for l in range(self.n_layers)]
            if self.per_head:
                for l, it in enumerate(items):
                    it.update(head_cap=self.cap, head_budget=self.head_budget[l],
                              head_tokens=self.tokens[self.tcur][l],
                              head_tokens_out=self.tokens[1 - self.tcur][l])
            self._units[key] = make_units(items, device=self.device)
        return self._units[key]

    def step(self):
        """One eviction event: q, app_k and app_v must hold this event's window
        queries and the rows that arrive before the next event."""
        kept = self.cfg.kept_rows(self.n_tokens, self.cap)
        if kept + self.n_append > self.capacity:
            raise ValueError("capacity too small for budget (head_cap) + n_append")
        units = self._units_for(self.cur, self.n_tokens)
        nx_evict_batch(self.cfg, units, self.n_layers, self.n_tokens, self.walk_iters, self.seed,
                       workspace=self.ws, step=self.step_no, max_out_rows=kept + self.n_append)
        if not self.inplace:
            self.cur = 1 - self.cur
        if self.per_head:
            self.tcur = 1 - self.tcur
        self.last_units = self.cfg.units(self.n_tokens)
        self.n_tokens = kept + self.n_append
        self.step_no += 1

    def head_tokens(self):
        """Live rows of every head, int64 [n_layers, n_kv_heads] on the host (synchronises)."""
        if not self.per_head:
            return torch.full((self.n_layers, self.cfg.n_kv_heads), self.n_tokens,
                              dtype=torch.int64)
        return self.tokens[self.tcur].cpu().long()

    def weights(self, layer):
        """The weights [n_kv_heads, units] the last event selected on (export_w=True);
        with per-head budgets head h's row holds units(its count before the event)
        valid entries."""
        if self.w is None:
            raise ValueError("StreamingCache was built without export_w")
        nu = self.last_units
        return self.w[layer][:self.cfg.n_kv_heads * nu].view(self.cfg.n_kv_heads, nu)

    def live(self):
        """(k, v) views of the live cache: [n_layers, n_kv_heads, n_tokens, head_dim]
        (with per-head budgets, head h's rows past head_tokens()[layer, h] are stale)."""
        return self.k[self.cur][:, :, :self.n_tokens], self.v[self.cur][:, :, :self.n_tokens]

    def state(self):
        """Host copy of everything a resumed stream needs."""
        k, v = self.live()
        return {"k": k.cpu(), "v": v.cpu(), "n_tokens": self.n_tokens, "step": self.step_no,
                "head_tokens": self.head_tokens()}

    def restore(self, st):
        self.cur = 0
        self.load(st["k"].to(self.device), st["v"].to(self.device), st["n_tokens"])
        if self.per_head:
            self.tokens[self.tcur].copy_(st["head_tokens"].to(torch.int32))
        self.step_no = st["step"]
