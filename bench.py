"""Benchmark of the Nexus Sampling eviction step on one MI355X.

One step = one eviction event over every layer of the headline workload: a
Llama-3-8B-shaped model (32 layers, 32 query heads sharing 8 KV heads, head_dim
128, bf16) whose cache holds N = 32768 tokens per KV head, evicted to B = 6554
with a window of W = 32 queries and walk depth H = 3.  All stages run in one
nx_evict_batch call: scoring (two MFMA sweeps over K), walk and keys, radix
select, compaction.  Inputs are synthetic and resident in HBM before timing.

Prints one JSON line: KV tokens scored and sampled per second (256 head units
x 32768 tokens per step), step latency (mean, and median / p10 / p90 of
per-step HIP events), the scoring stage against HBM with the algorithmic K
bytes counted once over both sweeps (HIP events inside the timed loop), the
compaction against HBM, and the fp64 CPU oracle timed on the host.

Other modes: --workload tiny_mha_f32 / llama3_8b_layer (single-layer latency,
eager and graph-replayed), ragged16_zipf / llama70b_share (the other full-size
events), --steady, --survival, --read-ceiling, --copy-calibration.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import streaming_weighted_sampling_amd as nx  # noqa: E402
from workloads import WORKLOADS, fill_layer_, bf16_bits, gen_layer  # noqa: E402

METRIC = "KV tokens scored+sampled/sec and eviction-step latency at N=32K, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
SCORE_STAGES = ("score_stats", "score_combine", "score_probs")

PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "eviction_step_llama3_8b_stream32_hbm_bytes.txt")
CSRC = os.path.join(ROOT, "streaming_weighted_sampling_amd", "csrc")


def csrc_digest():
    """sha256 over the kernel sources (sorted names and contents)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def counter_traffic(kernels, path=PROFILE_COUNTERS):
    """HBM bytes per launch summed over `kernels`, from a committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy calibration),
    or None when the summary is missing, lacks a kernel, or was taken on other
    kernel sources."""
    try:
        with open(path) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    digest, found = None, {}
    for line in lines:
        parts = line.split()
        if len(parts) == 2 and parts[0] == "csrc_sha256:":
            digest = parts[1]
        if len(parts) == 4 and parts[0] == "traffic_bytes_per_launch:":
            found[parts[1]] = int(parts[2]) + int(parts[3])
    if digest != csrc_digest() or any(k not in found for k in kernels):
        return None
    return {"bytes": sum(found[k] for k in kernels), "source": os.path.relpath(path, ROOT)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def budget_units(wl, block):
    """Kept units per head: B tokens, or round(B / b) blocks of b tokens."""
    return wl.budget if block == 1 else max(1, round(wl.budget / block))


def build_batch(wl, device, block=1, head_cap=0):
    """The headline batch; head_cap > 0 sizes keep and output rows for per-head
    budgets of up to head_cap units (head_budget arrays included)."""
    L, H, N, D = wl.n_layers, wl.h_kv, wl.n_tokens, wl.head_dim
    B = budget_units(wl, block)
    C = head_cap if head_cap > 0 else B
    R = min(C * block, N)            # kept rows per head (capacity)
    q = torch.empty(L, wl.h_q, wl.window, D, dtype=torch.bfloat16, device=device)
    k = torch.empty(L, H, N, D, dtype=torch.bfloat16, device=device)
    v = torch.empty(L, H, N, D, dtype=torch.bfloat16, device=device)
    q32 = torch.empty(wl.h_q, wl.window, D, device=device)
    k32 = torch.empty(H, N, D, device=device)
    v32 = torch.empty(H, N, D, device=device)
    for layer in range(L):
        fill_layer_(wl, q32, k32, v32, layer=layer)
        q[layer].copy_(q32)
        k[layer].copy_(k32)
        v[layer].copy_(v32)
    del q32, k32, v32
    keep = torch.empty(L, H, C, dtype=torch.int32, device=device)
    out_k = torch.empty(L, H, R, D, dtype=torch.bfloat16, device=device)
    out_v = torch.empty_like(out_k)
    head_budget = torch.zeros(L, H, dtype=torch.int32, device=device)
    items = [dict(q=q[l], k=k[l], v=v[l], keep=keep[l], out_k=out_k[l], out_v=out_v[l],
                  kv_head_stride=N * D, out_head_stride=R * D, n_tokens=N, budget=B, layer=l,
                  head_cap=head_cap, head_budget=head_budget[l] if head_cap > 0 else None)
             for l in range(L)]
    units = nx.make_units(items, device=device)
    return dict(q=q, k=k, v=v, keep=keep, out_k=out_k, out_v=out_v, units=units, budget=B,
                rows=R, head_budget=head_budget)


def _oracle_layer_seconds(wl, qb, kb, vb, budget, layer, threads=None):
    """Wall seconds of the oracle's full step on one (sequence, layer): every
    KV head (threads=1 pins BLAS to one thread)."""
    from oracle import nexus
    dt = "bf16" if wl.dtype == "bf16" else "f32"
    if threads is None:
        t0 = time.perf_counter()
        nexus.evict_step(qb, kb, vb, budget, wl.walk_iters, 0, dtype=dt, layer=layer)
        return time.perf_counter() - t0
    from threadpoolctl import threadpool_limits
    with threadpool_limits(threads):
        t0 = time.perf_counter()
        nexus.evict_step(qb, kb, vb, budget, wl.walk_iters, 0, dtype=dt, layer=layer)
        return time.perf_counter() - t0


def cpu_baseline(wl, data, budget_s, n_avg=1, block=1, extra=True):
    """The fp64 oracle as it stands, on the host: whole KV heads of the headline
    event in layer order until ~budget_s seconds pass; then (extra) one
    Llama-3-8B layer (N = 4096) on every BLAS thread and on one, and one layer
    of the 70B-shaped share (N = 131072, G*W = 512)."""
    from oracle import nexus
    threads = blas_threads()
    heads_done, t0 = 0, time.perf_counter()
    while heads_done < wl.n_layers * wl.h_kv and time.perf_counter() - t0 < budget_s:
        layer, h = divmod(heads_done, wl.h_kv)
        q = bf16_bits(data["q"][layer, h * wl.group:(h + 1) * wl.group])
        k = bf16_bits(data["k"][layer, h:h + 1])
        v = bf16_bits(data["v"][layer, h:h + 1])
        nexus.evict_step(q, k, v, data["budget"], wl.walk_iters, 0, dtype="bf16", layer=layer,
                         n_avg=n_avg, block=block)
        heads_done += 1
    dt = time.perf_counter() - t0
    out = {"value": round(heads_done * wl.n_tokens / dt, 1), "unit": "KV tokens/s",
           "cores": threads, "kind": "oracle",
           "sample": f"{heads_done} of {wl.n_layers * wl.h_kv} KV heads of the same step "
                     f"({heads_done * wl.n_tokens} tokens, full oracle step per head) in "
                     f"{dt:.1f} s; BLAS threads {threads} (numpy elementwise work runs on one), "
                     f"{os.cpu_count()} host CPUs visible",
           "cpu_model": cpu_model()}
    if not extra:
        return out
    runs = []
    for name, th in (("llama3_8b_layer", None), ("llama3_8b_layer", 1), ("llama70b_share", None)):
        w2 = WORKLOADS[name]
        x = gen_layer(w2, device="cuda")
        qb, kb, vb = bf16_bits(x["q"]), bf16_bits(x["k"]), bf16_bits(x["v"])
        del x
        sec = _oracle_layer_seconds(w2, qb, kb, vb, w2.budget, 0, threads=th)
        toks = w2.h_kv * w2.n_tokens
        runs.append({"workload": f"{name} one layer ({w2.h_kv} KV heads x {w2.n_tokens} tokens)",
                     "blas_threads": th or threads, "seconds_per_layer": round(sec, 4),
                     "kv_tokens_per_s": round(toks / sec, 1)})
    out["runs"] = runs
    return out


def timed_batch(step, steps, stages):
    """Runs step(i) for i < steps with HIP events around each step and around
    the given stages' launches; returns (wall ms per step, per-step event ms,
    {stage: (ms per launch, launches)})."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    nx.profile_enable(True, stages=list(stages))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nx.profile_enable(False)
    st = nx.profile_read()
    per = {s: (st[s][0] / max(st[s][1], 1), st[s][1]) for s in stages if st[s][1]}
    return (t1 - t0) * 1e3 / steps, [a.elapsed_time(b) for a, b in ev], per


def stage_pass(step, steps):
    """Per-stage ms per launch from a pass with events around every stage
    (outside the timed region: each recorded launch adds two event records)."""
    nx.profile_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    nx.profile_enable(False)
    return {name: (ms / max(cnt, 1), cnt) for name, (ms, cnt) in nx.profile_read().items() if cnt}


def roofline_obj(amount, unit, peak, bound, kernel_ms, launches, kernel, traffic):
    achieved = amount / (kernel_ms * 1e-3)
    return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": None if traffic is None else traffic["bytes"],
            "kernel": kernel, "kernel_ms_per_launch": round(kernel_ms, 4),
            "launches_timed": launches,
            "traffic_source": None if traffic is None else traffic["source"]}


def steady_run(wl, compact, steps, warmup):
    """Streaming steady state: every event holds N = B + A rows per head, keeps
    B and appends A new rows (queries and new rows synthetic, fixed).  Returns
    (ms per event, per-stage ms per launch, rows per head)."""
    from streaming_weighted_sampling_amd.stream import StreamingCache
    dev = "cuda"
    L, B, A = wl.n_layers, wl.budget, wl.stream_append
    n = B + A
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16)
    sc = StreamingCache(cfg, L, n, B, A, wl.walk_iters, seed=0, device=dev,
                        inplace=compact == "inplace")
    q32 = torch.empty(wl.h_q, wl.window, wl.head_dim, device=dev)
    k32 = torch.empty(wl.h_kv, n, wl.head_dim, device=dev)
    v32 = torch.empty(wl.h_kv, n, wl.head_dim, device=dev)
    k0 = torch.empty(L, wl.h_kv, n, wl.head_dim, dtype=torch.bfloat16, device=dev)
    v0 = torch.empty_like(k0)
    for layer in range(L):
        fill_layer_(wl, q32, k32, v32, layer=layer, n_tokens=n)
        sc.q[layer].copy_(q32)
        k0[layer].copy_(k32)
        v0[layer].copy_(v32)
    sc.load(k0, v0, n)
    del k0, v0
    g = torch.Generator(device=dev).manual_seed(5)
    sc.app_k.copy_(torch.randn(sc.app_k.shape, generator=g, device=dev).to(torch.bfloat16))
    sc.app_v.copy_(torch.randn(sc.app_v.shape, generator=g, device=dev).to(torch.bfloat16))
    for _ in range(warmup):
        sc.step()
    torch.cuda.synchronize()
    nx.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        sc.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    nx.profile_enable(False)
    stages = nx.profile_read()
    nx.nx_read_device_status(sc.cfg, sc.ws)
    ms = (t1 - t0) * 1e3 / steps
    return ms, {k: round(v[0] / max(v[1], 1), 4) for k, v in stages.items() if v[1]}, n


def steady(wl, args):
    """The streaming steady state as its own JSON line (--steady)."""
    ms, stages, n = steady_run(wl, args.compact, args.steps, args.warmup)
    units = wl.n_layers * wl.h_kv
    B, A = wl.budget, wl.stream_append
    print(json.dumps({
        "metric": METRIC, "value": round(units * n / (ms * 1e-3), 1), "unit": "KV tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"llama3_8b_stream32 steady-state event N={n} -> {B} + {A} "
                               f"appended, 32 layers x 8 KV heads", "compact": args.compact},
        "stage_ms_per_launch": stages,
    }))


def survival_bench(args):
    """The survival stream: the same queries and arriving rows under each
    selection policy; reports the Nexus policy's event rate and every policy's
    survival of the tracked classes at a few event counts."""
    from streaming_weighted_sampling_amd.survival import POLICIES, run_survival
    from workloads import SURVIVAL, survival_event, survival_initial
    spec = SURVIVAL
    dev = "cuda"
    initial = survival_initial(spec, device=dev)
    curves, ms = {}, {}
    for policy in POLICIES:
        r = run_survival(spec, policy, initial, lambda e: survival_event(spec, e, device=dev),
                         device=dev)
        at = [e for e in (1, 10, 50, 100, 200, 300, 400) if e <= spec.events]
        curves[policy] = {f"{off:+.1f}": [round(float(r.survival[e, c]), 5) for e in at]
                          for c, off in enumerate(spec.offsets)}
        ms[policy] = r.ms_per_event
    units = spec.n_streams * spec.h_kv
    print(json.dumps({
        "metric": "survival-stream eviction events/sec (16 streams x 8 KV heads), 1 MI355X",
        "value": round(1e3 / ms["nexus"], 1), "unit": "events/s", "n_gpus": 1,
        "steps": spec.events, "warmup": 0, "ms_per_step": round(ms["nexus"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"survival_stream {spec.n_streams} streams x {spec.h_kv} KV heads, "
                               f"N = {spec.n0} -> {spec.budget} + {spec.append}, "
                               f"{spec.events} events", "head_units": units},
        "ms_per_event": {p: round(v, 4) for p, v in ms.items()},
        "survival_at_events": at,
        "survival": curves,
    }))


def headline(args):
    """The 32-layer event at N = 32768 (optionally n-averaged, blocks or per-head budgets)."""
    dev = "cuda"
    wl = WORKLOADS["llama3_8b_stream32"]
    heads = args.heads == "alloc"
    cap = 2 * budget_units(wl, args.block) if heads else 0
    data = build_batch(wl, dev, args.block, head_cap=cap)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, torch.bfloat16,
                         n_avg=args.n_avg, block=args.block,
                         head_alloc=nx.NX_HEADS_ALLOC if heads else nx.NX_HEADS_UNIFORM,
                         head_floor=data["budget"] // 5 if heads else 0)
    ws = nx.new_workspace(cfg, wl.n_tokens, wl.n_layers, wl.walk_iters, device=dev)

    def step(i):
        nx.nx_evict_batch(cfg, data["units"], wl.n_layers, wl.n_tokens, wl.walk_iters, 0,
                          workspace=ws, step=i, max_out_rows=data["rows"])

    for i in range(args.warmup):
        step(i)
    nx.nx_read_device_status(cfg, ws)
    torch.cuda.synchronize()
    per_launch = stage_pass(lambda i: step(args.warmup + i), args.steps)

    units = wl.n_layers * wl.h_kv
    tokens = units * wl.n_tokens
    # Algorithmic work per launch (one launch per stage per step covers every
    # layer): per (KV head, resident token) d*e bytes of K read once and
    # 2*G*W*d flops; per kept row 4*d*e bytes (K and V read and written) plus a
    # 4-byte index.  The second sweep over K is not counted.
    d, e = wl.head_dim, 2
    k_bytes = tokens * d * e
    kept_rows = min(data["budget"] * args.block, wl.n_tokens)   # per head on average
    compact_bytes = units * (kept_rows * 4 * d * e + data["budget"] * 4)
    qk_flops = tokens * 2 * wl.group * wl.window * d

    # Timed region: events around each step and around the three score stages
    # and the compaction, on the stream they are launched on.
    timed = SCORE_STAGES + ("kv_compact",)
    ms_per_step, step_ms, per = timed_batch(lambda i: step(args.warmup + args.steps + i),
                                            args.steps, timed)
    nx.nx_read_device_status(cfg, ws)
    # Calls that merge the row statistics inside pass 2 launch no score_combine.
    launched = [s for s in SCORE_STAGES if s in per]
    score_ms = sum(per[s][0] for s in launched)
    score_label = "nexus_score (" + " + ".join(launched) + ")"
    roofline = roofline_obj(k_bytes / 1e9, "GB/s", HBM_PEAK_GBS, "hbm", score_ms,
                            per["score_probs"][1],
                            score_label, counter_traffic(launched))
    roofline["algorithmic_bytes"] = int(k_bytes)
    roofline["note"] = ("K bytes counted once over both sweeps: the second sweep over K is an "
                        "implementation cost, not algorithmic work")
    compact = roofline_obj(compact_bytes / 1e9, "GB/s", HBM_PEAK_GBS, "hbm", per["kv_compact"][0],
                           per["kv_compact"][1], "kv_compact", counter_traffic(("kv_compact",)))
    compact["algorithmic_bytes"] = int(compact_bytes)
    value = tokens / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_stream32 eviction event at N=32768 (32 layers x 8 KV "
                               "heads, GQA 32:8, head_dim 128, W=32, H=3, B=6554)",
                   "layers": wl.n_layers, "kv_heads": wl.h_kv, "n_tokens": wl.n_tokens,
                   "budget": wl.budget, "window": wl.window, "walk_iters": wl.walk_iters,
                   "n_avg": args.n_avg, "block": args.block, "heads": args.heads,
                   "budget_units": data["budget"]},
        "step_latency_ms": {"mean": round(ms_per_step, 4), "median": round(pct(step_ms, 50), 4),
                            "p10": round(pct(step_ms, 10), 4), "p90": round(pct(step_ms, 90), 4)},
        "kv_token_positions_per_s": round(value / wl.h_kv, 1),
        "stage_ms_per_launch": {k: round(v[0], 4) for k, v in per_launch.items()},
        "stage_ms_note": "per-stage times from a pass with events around every stage, "
                         "outside the timed region",
        "stage_gbs": {
            **{f"{s}_k_read": round(k_bytes / (per[s][0] * 1e-3) / 1e9, 1)
               for s in ("score_stats", "score_probs")},
            "kv_compact": round(compact_bytes / (per["kv_compact"][0] * 1e-3) / 1e9, 1),
            "step_algorithmic": round((k_bytes + compact_bytes) / (ms_per_step * 1e-3) / 1e9, 1),
        },
        "mfma_tflops_per_sweep": {s: round(qk_flops / (per[s][0] * 1e-3) / 1e12, 1)
                                  for s in ("score_stats", "score_probs")},
        "roofline": roofline,
        "roofline_kv_compact": compact,
        # The whole step against HBM: one K read plus the compaction's K/V traffic.
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": int(k_bytes + compact_bytes),
                          "ms_at_peak": round((k_bytes + compact_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
                          "frac": round((k_bytes + compact_bytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, data, args.cpu_seconds, args.n_avg, args.block)
    if args.n_avg == 1 and args.block == 1 and args.heads == "uniform" and not args.no_steady:
        # Context, not the metric: the same model's streaming steady state (every
        # later event of the streaming workload), N = B + A -> B kept + A appended.
        del data
        torch.cuda.empty_cache()
        st = {}
        for mode in ("copy", "inplace"):
            ms, stages, _ = steady_run(wl, mode, 10, 2)
            st[mode] = {"ms_per_event": round(ms, 4), "kv_compact_ms": stages.get("kv_compact")}
        out["streaming_steady_state"] = {
            "events": f"N={wl.budget + wl.stream_append} -> {wl.budget} kept + {wl.stream_append} "
                      f"appended per KV head, 32 layers x 8 KV heads, 10 timed events each",
            **st}
    print(json.dumps(out))


def layer_latency(args):
    """One (sequence, layer) eviction through nx_evict_step: the tiny fp32 head
    (N = 512) or one Llama-3-8B layer (N = 4096).  Latency-bound shapes, so the
    report is absolute microseconds: eager launches timed with events per step,
    and the same steps captured in a HIP graph and replayed.  Steps rotate over
    copies of the layer (about 256 MB in total for the 8B layer) so that no step
    finds its K in the caches from the previous one."""
    dev = "cuda"
    wl = WORKLOADS[args.workload]
    dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, wl.head_dim, wl.window, dtype)
    n, B, H, D = wl.n_tokens, wl.budget, wl.h_kv, wl.head_dim
    x = gen_layer(wl, device=dev)
    per_copy = 2 * x["k"].numel() * x["k"].element_size()
    copies = int(min(64, max(4, -(-(256 << 20) // per_copy))))
    ks = [x["k"].clone() for _ in range(copies)]
    vs = [x["v"].clone() for _ in range(copies)]
    keep = torch.empty(copies, H, B, dtype=torch.int32, device=dev)
    ok = torch.empty(copies, H, min(B, n), D, dtype=dtype, device=dev)
    ov = torch.empty_like(ok)
    ws = nx.new_workspace(cfg, n, 1, wl.walk_iters, device=dev)

    def step(i):
        c = i % copies
        nx.nx_evict_step(cfg, x["q"], ks[c], vs[c], n, B, wl.walk_iters, 0, workspace=ws,
                         step=i, out_k=ok[c], out_v=ov[c], keep=keep[c])

    for i in range(max(args.warmup, 5)):
        step(i)
    nx.nx_read_device_status(cfg, ws)
    reps = max(args.steps, 30)
    stages = stage_pass(step, reps)
    ms_mean, ev_ms, _ = timed_batch(step, reps, ())
    # Eager reference for the graph: the steps the graph captures, run once eagerly.
    for i in range(copies):
        step(i)
    torch.cuda.synchronize()
    eager_keep = keep.clone()
    eager_k = ok.clone()
    # The same `copies` steps captured once and replayed: launch costs leave the
    # measurement, kernel time and inter-kernel gaps stay.
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(copies):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    graph_same = bool(torch.equal(keep, eager_keep)) and bool(torch.equal(ok, eager_k))
    graph_ms = []
    for _ in range(max(reps // copies, 8)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        graph_ms.append(a.elapsed_time(b) / copies)
    nx.nx_read_device_status(cfg, ws)
    tokens = H * n
    k_bytes = tokens * D * x["k"].element_size()
    compact_bytes = H * min(B, n) * (4 * D * x["k"].element_size() + 4)
    med_eager, med_graph = pct(ev_ms, 50), pct(graph_ms, 50)
    print(json.dumps({
        "metric": f"eviction-step latency and KV tokens scored+sampled/sec, {args.workload}, 1 MI355X",
        "value": round(med_graph * 1e3, 2), "unit": "us per step (graph-replayed, median)",
        "n_gpus": 1, "steps": reps, "warmup": max(args.warmup, 5),
        "ms_per_step": round(ms_mean, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "kv_heads": H, "q_heads": wl.h_q,
                   "head_dim": D, "n_tokens": n, "budget": B, "window": wl.window,
                   "walk_iters": wl.walk_iters, "cache_copies_rotated": copies},
        "latency_us": {"eager": {"median": round(med_eager * 1e3, 2),
                                 "p10": round(pct(ev_ms, 10) * 1e3, 2),
                                 "p90": round(pct(ev_ms, 90) * 1e3, 2)},
                       "graph": {"median": round(med_graph * 1e3, 2),
                                 "p10": round(pct(graph_ms, 10) * 1e3, 2),
                                 "p90": round(pct(graph_ms, 90) * 1e3, 2)}},
        "graph_replay_matches_eager": graph_same,
        "stage_us_per_launch": {k: round(v[0] * 1e3, 2) for k, v in stages.items()},
        "stage_us_note": "eager, events around every stage (outside the timed loops)",
        "kv_tokens_per_s": {"eager": round(tokens / (med_eager * 1e-3), 1),
                            "graph": round(tokens / (med_graph * 1e-3), 1)},
        "roofline": {"bound": "latency", "algorithmic_bytes": int(k_bytes + compact_bytes),
                     "us_at_hbm_peak": round((k_bytes + compact_bytes) / (HBM_PEAK_GBS * 1e9) * 1e6, 3),
                     "frac_graph": round((k_bytes + compact_bytes) / (med_graph * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }))


def other_workload(args):
    """One eviction event of the ragged batch or of the 70B-shaped share, timed
    like the headline and reported against its own bound: HBM for the ragged
    batch (K bytes once over both sweeps), bf16 MFMA for the 70B share (the QK^T
    flops of one pass over both sweeps' time, G*W = 512 query rows per K byte).
    No CPU baseline."""
    from workloads import budget_for, gen_model, ragged_lengths
    dev = "cuda"
    wl = WORKLOADS[args.workload]
    D, Hk, L = wl.head_dim, wl.h_kv, wl.n_layers
    lens = ragged_lengths(wl) if args.workload == "ragged16_zipf" else [wl.n_tokens]
    items, keep_bufs = [], []
    tokens = kept_rows = 0
    for s, n in enumerate(lens):
        B = budget_for(n) if args.workload == "ragged16_zipf" else wl.budget
        q, k, v = gen_model(wl, device=dev, n_tokens=n, seq=s)
        keep = torch.empty(L, Hk, B, dtype=torch.int32, device=dev)
        ok = torch.empty(L, Hk, B, D, dtype=torch.bfloat16, device=dev)
        ov = torch.empty_like(ok)
        keep_bufs.append((q, k, v, keep, ok, ov))
        for l in range(L):
            items.append(dict(q=q[l], k=k[l], v=v[l], keep=keep[l], out_k=ok[l], out_v=ov[l],
                              kv_head_stride=n * D, out_head_stride=B * D, n_tokens=n,
                              budget=B, layer=l, seq_id=s))
        tokens += L * Hk * n
        kept_rows += L * Hk * min(B, n)
    n_max = max(lens)
    units = nx.make_units(items, device=dev)
    cfg = nx.NexusConfig(wl.h_q, wl.h_kv, D, wl.window, torch.bfloat16)
    ws = nx.new_workspace(cfg, n_max, len(items), wl.walk_iters, device=dev)
    b_max = max(it["budget"] for it in items)

    def step(i):
        nx.nx_evict_batch(cfg, units, len(items), n_max, wl.walk_iters, 0, workspace=ws, step=i,
                          max_out_rows=b_max)

    for i in range(args.warmup):
        step(i)
    nx.nx_read_device_status(cfg, ws)
    torch.cuda.synchronize()
    per_launch = stage_pass(lambda i: step(args.warmup + i), args.steps)
    e = 2
    k_bytes = tokens * D * e
    compact_bytes = kept_rows * (4 * D * e + 4)
    qk_flops = tokens * 2 * wl.group * wl.window * D       # one pass
    timed = SCORE_STAGES + ("kv_compact",)
    ms_per_step, step_ms, per = timed_batch(lambda i: step(args.warmup + args.steps + i),
                                            args.steps, timed)
    nx.nx_read_device_status(cfg, ws)
    # Calls that merge the row statistics inside pass 2 launch no score_combine.
    launched = [s for s in SCORE_STAGES if s in per]
    score_ms = sum(per[s][0] for s in launched)
    score_label = "nexus_score (" + " + ".join(launched) + ")"
    counters = os.path.join(ROOT, "profiles", f"{args.workload}_hbm_bytes.txt")
    if args.workload == "llama70b_share":
        roofline = roofline_obj(qk_flops / 1e12, "TFLOP/s", BF16_PEAK_TFLOPS, "mfma", score_ms,
                                per["score_probs"][1],
                                score_label, counter_traffic(launched, counters))
        roofline["algorithmic_flops"] = int(qk_flops)
        roofline["note"] = "QK^T flops of one pass over both sweeps' time"
    else:
        roofline = roofline_obj(k_bytes / 1e9, "GB/s", HBM_PEAK_GBS, "hbm", score_ms,
                                per["score_probs"][1],
                                score_label, counter_traffic(launched, counters))
        roofline["algorithmic_bytes"] = int(k_bytes)
        roofline["note"] = "K bytes counted once over both sweeps"
    compact = roofline_obj(compact_bytes / 1e9, "GB/s", HBM_PEAK_GBS, "hbm", per["kv_compact"][0],
                           per["kv_compact"][1], "kv_compact",
                           counter_traffic(("kv_compact",), counters))
    print(json.dumps({
        "metric": f"KV tokens scored+sampled/sec and eviction-step latency, {args.workload}, 1 MI355X",
        "value": round(tokens / (ms_per_step * 1e-3), 1), "unit": "KV tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "items": len(items), "layers": L, "kv_heads": Hk,
                   "group": wl.group, "window": wl.window, "walk_iters": wl.walk_iters,
                   "n_tokens_min": min(lens), "n_tokens_max": n_max, "kv_tokens": tokens,
                   "kept_rows": kept_rows},
        "step_latency_ms": {"mean": round(ms_per_step, 4), "median": round(pct(step_ms, 50), 4),
                            "p10": round(pct(step_ms, 10), 4), "p90": round(pct(step_ms, 90), 4)},
        "stage_ms_per_launch": {k: round(v[0], 4) for k, v in per_launch.items()},
        "mfma_tflops_per_sweep": {s: round(qk_flops / (per[s][0] * 1e-3) / 1e12, 1)
                                  for s in ("score_stats", "score_probs")},
        "stage_gbs": {f"{s}_k_read": round(k_bytes / (per[s][0] * 1e-3) / 1e9, 1)
                      for s in ("score_stats", "score_probs")},
        "roofline": roofline,
        "roofline_kv_compact": compact,
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": int(k_bytes + compact_bytes),
                          "ms_at_peak": round((k_bytes + compact_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
                          "frac": round((k_bytes + compact_bytes) / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }))


def read_ceiling(args):
    """What one read of a buffer costs on this GPU, through the library's read
    probe (nx_stream_read): the score sweeps' LDS ring and plain vector loads,
    over 2 GiB (each pass from HBM) and over 128 MB and 32 MB regions read
    again right after themselves (the 256 MB Infinity Cache and the 32 MB of L2).
    The first pass over a region is untimed; the following ones are timed."""
    dev = "cuda"
    lib = nx.load()
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    rows = []
    for mode, name in ((0, "lds_ring"), (1, "vector_loads")):
        for mb in (2048, 512, 256, 128, 64, 32):
            nbytes = mb << 20
            passes = 4 if mb >= 1024 else 16
            nx.check(lib.nx_stream_read(buf.data_ptr(), nbytes, mode, 1, sink.data_ptr(),
                                        stream.cuda_stream), "nx_stream_read")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            nx.check(lib.nx_stream_read(buf.data_ptr(), nbytes, mode, passes, sink.data_ptr(),
                                        stream.cuda_stream), "nx_stream_read")
            b.record(stream)
            b.synchronize()
            ms = a.elapsed_time(b) / passes
            rows.append({"mode": name, "region_mb": mb, "passes_timed": passes,
                         "us_per_pass": round(ms * 1e3, 2),
                         "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    print(json.dumps({"read_ceiling": rows, "hbm_peak_gbs": HBM_PEAK_GBS,
                      "note": "regions of 2 GiB stream from HBM on every pass; smaller ones are "
                              "read again right after themselves"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the headline part of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-steady", action="store_true",
                    help="leave out the streaming steady-state context of the headline line "
                         "(profiling runs of the headline event alone)")
    ap.add_argument("--steady", action="store_true",
                    help="time the streaming steady-state event (N = B + 256 -> B, 32 layers) "
                         "through StreamingCache instead of the N = 32768 event")
    ap.add_argument("--survival", action="store_true",
                    help="run the survival stream (400 events) under every selection policy")
    ap.add_argument("--heads", choices=["uniform", "alloc"], default="uniform",
                    help="per-head budgets: uniform B, or allocated over the heads of each "
                         "layer (floor B/5, capacity 2B)")
    ap.add_argument("--compact", choices=["copy", "inplace"], default="copy",
                    help="with --steady: copy kept rows to the other buffer, or fill holes in place")
    ap.add_argument("--block", type=int, default=1,
                    help="selection unit of Eq. 1: 1 = tokens, else blocks of that many tokens")
    ap.add_argument("--n-avg", type=int, default=1,
                    help="priority averaging count of Eq. 6 (1: A-Res key; -1: top-B by weight)")
    ap.add_argument("--workload", choices=["llama3_8b_stream32", "tiny_mha_f32", "llama3_8b_layer",
                                           "ragged16_zipf", "llama70b_share"],
                    default="llama3_8b_stream32",
                    help="the headline 32-layer event (default), single-layer latency of the "
                         "tiny head or of one Llama-3-8B layer, the ragged 16-sequence batch, or "
                         "the 8-layer 70B-shaped share at N = 131072")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only time the read probe (LDS ring and vector loads) over 2 GiB and "
                         "over regions read again right after themselves")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1-GiB device copy (3 times), the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the eviction path has no multi-GPU mode "
              "(head units are independent, so units would be split across GPUs with no "
              "exchange between them).", file=sys.stderr)
        sys.exit(2)

    dev = "cuda"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "repeats": 3}))
        return
    if args.read_ceiling:
        read_ceiling(args)
        return
    if args.workload in ("tiny_mha_f32", "llama3_8b_layer"):
        layer_latency(args)
        return
    if args.workload != "llama3_8b_stream32":
        other_workload(args)
        return
    wl = WORKLOADS["llama3_8b_stream32"]
    if args.survival:
        survival_bench(args)
        return
    if args.steady:
        steady(wl, args)
        return
    headline(args)


if __name__ == "__main__":
    main()
