"""Long-run survival of tracked tokens under streaming eviction.

[Nexus] ("Forget Without Compromise: Nexus Sampling for Streaming KV-Cache
Eviction Under Fixed Budgets") section 3 and appendix 8.3 (Lemma 1): under
deterministic top-K a token survives only while it clears the cutoff at every
event, under the weighted reservoir its survival is a product of per-event
inclusion probabilities that stay positive while its weight does.  This
driver runs the same stream of queries and arriving rows under several
selection policies and counts, after every event, how many tokens of each
tracked class are still resident.

Policies:
  nexus        Nexus weights (walk depth of the run), reservoir keys ln(u)/w
  topk         the same weights, deterministic top-B (the n -> infinity limit)
  topk_direct  the direct score alone (walk depth 0), deterministic top-B

Every event is one nx_evict_batch call over all streams (one stream = one
item); the id bookkeeping that follows the kept rows is torch gathers on
the device, outside the eviction path.
"""

from dataclasses import dataclass

import torch

from .api import TOPK, NexusConfig, nx_read_device_status
from .stream import StreamingCache

POLICIES = ("nexus", "topk", "topk_direct")


@dataclass
class SurvivalResult:
    policy: str
    survival: torch.Tensor      # [events + 1, n_classes] fraction of tracked tokens resident
    ms_per_event: float         # eviction calls only (HIP events around them)
    events: int


def _policy(policy, walk_iters):
    if policy == "nexus":
        return 1, walk_iters
    if policy == "topk":
        return TOPK, walk_iters
    if policy == "topk_direct":
        return TOPK, 0
    raise ValueError(f"unknown policy {policy!r}; expected one of {POLICIES}")


def run_survival(spec, policy, initial, event_inputs, *, events=None, seed=0, device="cuda",
                 on_event=None):
    """Run one policy over the stream.

    initial: (k, v, cls) from the workload's survival_initial on `device`;
    event_inputs(e) -> (q, app_k, app_v) of event e.  on_event(e, cache,
    pre) is called after each event with the StreamingCache and the pre-event
    (q, k, v, n_tokens) host-visible tensors when it is given (for checks).
    """
    events = spec.events if events is None else events
    n_avg, walk = _policy(policy, spec.walk_iters)
    dtype = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    cfg = NexusConfig(spec.h_q, spec.h_kv, spec.head_dim, spec.window, dtype=dtype, n_avg=n_avg)
    S, H, n0, A, B = spec.n_streams, spec.h_kv, spec.n0, spec.append, spec.budget
    sc = StreamingCache(cfg, S, n0, B, A, walk, seed=seed, device=device)
    k0, v0, cls = initial
    sc.load(k0, v0, n0)
    n_cls = len(spec.offsets)
    ids = torch.arange(n0, device=device).expand(S, H, n0).contiguous()
    counts = torch.zeros(events + 1, n_cls, dtype=torch.int64, device=device)
    counts[0] = torch.bincount(cls[cls >= 0], minlength=n_cls)
    start = [torch.cuda.Event(enable_timing=True) for _ in range(events)]
    stop = [torch.cuda.Event(enable_timing=True) for _ in range(events)]
    arange_a = torch.arange(A, device=device)
    for e in range(events):
        q, ak, av = event_inputs(e)
        sc.q.copy_(q)
        sc.app_k.copy_(ak)
        sc.app_v.copy_(av)
        pre = None
        if on_event is not None:
            k_pre, v_pre = sc.live()
            pre = (sc.q.clone(), k_pre.clone(), v_pre.clone(), sc.n_tokens)
        start[e].record()
        sc.step()
        stop[e].record()
        kept = ids.gather(2, sc.keep.long())
        ids = torch.cat([kept, (n0 + e * A + arange_a).expand(S, H, A)], dim=2)
        tracked = kept < n0
        c = cls.gather(2, kept.clamp(max=n0 - 1))
        c = c[tracked & (c >= 0)]
        counts[e + 1] = torch.bincount(c, minlength=n_cls)
        if on_event is not None:
            on_event(e, sc, pre, ids)
    nx_read_device_status(sc.cfg, sc.ws)
    ms = sum(a.elapsed_time(b) for a, b in zip(start, stop)) / max(events, 1)
    surv = counts.double() / counts[0].double().clamp(min=1)
    return SurvivalResult(policy, surv.cpu(), ms, events)
