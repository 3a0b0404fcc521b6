// Host side of the C ABI declared in include/nexus.h: argument validation,
// workspace carving and the launch sequence on the caller's stream.
//
// [Nexus] = "Forget Without Compromise: Nexus Sampling for Streaming KV-Cache
// Eviction Under Fixed Budgets" (academ.us article page).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "nx_internal.hpp"

using namespace nx;

namespace {

constexpr int32_t kMaxTokens = 1 << 24;
constexpr int32_t kMaxRowsPad = 512;    // 16 wavefronts x one 32-row tile

int32_t elem_size(int32_t dtype) { return dtype == NX_BF16 ? 2 : 4; }

// Shape checks shared by every entry point.
nx_status check_desc(const nx_desc* d) {
  if (d == nullptr) return NX_EINVAL;
  if (d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads || d->n_q_heads % d->n_kv_heads)
    return NX_EINVAL;
  if (d->window < 1 || d->n_sink < 0 || d->n_recent < 0) return NX_EINVAL;
  if (!std::isfinite(d->lambda) || !std::isfinite(d->eps_tie)) return NX_EINVAL;
  if (d->n_avg != NX_TOPK && (d->n_avg < 0 || d->n_avg > NX_MAX_AVG)) return NX_EINVAL;
  if (d->block < 0) return NX_EINVAL;
  if (d->compact != NX_COMPACT_COPY && d->compact != NX_COMPACT_INPLACE) return NX_EINVAL;
  if (d->head_alloc < NX_HEADS_UNIFORM || d->head_alloc > NX_HEADS_ALLOC || d->head_floor < 0)
    return NX_EINVAL;
  if (d->block > 1 && (d->block > 32 || (d->block & (d->block - 1)) != 0)) return NX_EUNSUPPORTED;
  if (d->dtype != NX_BF16 && d->dtype != NX_F32) return NX_EUNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return NX_EUNSUPPORTED;
  return NX_OK;
}

nx_status make_geometry(const nx_desc* d, int32_t max_tokens, int32_t n_items, int32_t walk,
                        Geometry* g) {
  *g = Geometry{};
  nx_status st = check_desc(d);
  if (st != NX_OK) return st;
  if (max_tokens < 1 || max_tokens > kMaxTokens || n_items < 1) return NX_EINVAL;
  // The per-head workspace rows (a, the walk rows, the keys) hold max_tokens
  // rounded up to a multiple of 4, so that every row starts 16-B aligned and
  // the token passes read them 16 bytes at a time whatever N the call has.
  g->max_n = max_tokens;
  max_tokens = (max_tokens + 3) & ~3;
  // One KV head's rows (and each per-head workspace array) stay below 2 GB so
  // 32-bit buffer offsets address them.
  if (walk < 0 || walk > d->window) return NX_EINVAL;
  if (int64_t(max_tokens) * d->head_dim * elem_size(d->dtype) > (int64_t(1) << 31) ||
      int64_t(max_tokens) * (walk > kMaxWalk ? walk : kMaxWalk) * 4 > (int64_t(1) << 31))
    return NX_EUNSUPPORTED;
  const int32_t group = d->n_q_heads / d->n_kv_heads;
  const int64_t rows = int64_t(group) * d->window;
  const int64_t rows_pad = (rows + 31) / 32 * 32;
  if (rows_pad > kMaxRowsPad) return NX_EUNSUPPORTED;
  // Deep walks take one row tile per G rows of a window slot (G <= 32).
  const bool deep = walk > kMaxWalk || int64_t(group) * walk > kMaxWalkRows;
  if (deep && (walk > kMaxWalkDeep || group > 32)) return NX_EUNSUPPORTED;
  const int64_t n_hu = int64_t(n_items) * d->n_kv_heads;
  if (n_hu > 65535) return NX_EUNSUPPORTED;     // grid y dimension of the token stages
  g->h_q = d->n_q_heads;
  g->h_kv = d->n_kv_heads;
  g->group = group;
  g->head_dim = d->head_dim;
  g->window = d->window;
  g->walk = walk;
  g->rows = int32_t(rows);
  g->rows_pad = int32_t(rows_pad);
  g->walk_rows = group * walk;
  g->block = d->block > 1 ? d->block : 1;
  g->inplace = d->compact == NX_COMPACT_INPLACE;
  g->head_alloc = d->head_alloc;
  // The allocation selects over all heads' units of an item at once.
  if (d->head_alloc == NX_HEADS_ALLOC &&
      (d->n_kv_heads > NX_MAX_ALLOC_HEADS || int64_t(d->n_kv_heads) * max_tokens >= (int64_t(1) << 31)))
    return NX_EUNSUPPORTED;
  g->dtype = d->dtype;
  g->n_hu = int32_t(n_hu);
  g->max_tokens = max_tokens;
  g->max_out_rows = max_tokens;
  g->n_t1 = (max_tokens + kMinTokPerBlock - 1) / kMinTokPerBlock;
  g->n_t2 = g->n_t1;
  // Tokens per score workgroup: first the tile count per head unit, the
  // fewest that give >= 2048 workgroups per pass (8 per CU) with tiles of at
  // most 2048 tokens; then equal tiles, rounded up to whole 32-token
  // sub-tiles and kept in [128, 2048].  Equal tiles keep the workgroups'
  // rounds on the chip full (N = 6810 at 256 head units: 8 tiles of 864
  // tokens, two full rounds, where halving powers of two gave 14 tiles of 512).
  const int64_t t_min = std::max<int64_t>((2048 + n_hu - 1) / n_hu,
                                          (int64_t(max_tokens) + kMaxTokPerBlock - 1) / kMaxTokPerBlock);
  const int64_t tpb64 = ((int64_t(max_tokens) + t_min - 1) / t_min + 31) / 32 * 32;
  const int32_t tpb = int32_t(std::min<int64_t>(std::max<int64_t>(tpb64, kMinTokPerBlock), kMaxTokPerBlock));
  g->tok_per_block = tpb;
  g->n_tmax = (max_tokens + tpb - 1) / tpb;
  g->n_kc = (max_tokens + kKeysPerBlock - 1) / kKeysPerBlock;
  g->deep = deep ? 1 : 0;
  g->packed = packed_rows(g->walk, g->group, g->block, deep) ? 1 : 0;
  g->n_gc = (max_tokens + kGramChunk - 1) / kGramChunk;
  return NX_OK;
}

nx_status bind_workspace(const nx_desc* d, const Geometry& g, Args* a) {
  const WsLayout L = ws_layout(g);
  if (d->workspace == nullptr || d->workspace_bytes < L.total) return NX_EWORKSPACE;
  char* base = static_cast<char*>(d->workspace);
  a->status = reinterpret_cast<uint32_t*>(base + L.status);
  a->part1 = reinterpret_cast<float*>(base + L.part1);
  a->beta = reinterpret_cast<float*>(base + L.beta);
  a->a = reinterpret_cast<float*>(base + L.a);
  a->p = reinterpret_cast<float*>(base + L.p);
  a->gram = reinterpret_cast<float*>(base + L.gram);
  a->coef = reinterpret_cast<float*>(base + L.coef);
  a->keys = reinterpret_cast<uint64_t*>(base + L.keys);
  a->selp = reinterpret_cast<uint64_t*>(base + L.selp);
  a->ahist = reinterpret_cast<uint32_t*>(base + L.ahist);
  a->acand = reinterpret_cast<uint32_t*>(base + L.acand);
  a->acnt = reinterpret_cast<int32_t*>(base + L.acnt);
  return NX_OK;
}

Args base_args(const nx_desc* d, const Geometry& g, uint64_t seed) {
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.g = g;
  // K streams of more than twice the 256 MB Infinity Cache bypass the caches
  // (faster sweeps); smaller ones stay cached in the second sweep, where the
  // copy compaction that follows finds part of the kept rows.  In-place
  // compaction reads only the moved rows, so there the second sweep bypasses
  // the caches above the cache's own size, and the first sweep always does
  // (the second re-reads K from its start, so whatever the first left cached
  // is gone by then).
  const int64_t k_bytes = int64_t(g.n_hu) * g.max_tokens * g.head_dim * elem_size(g.dtype);
  a.k_stream_nt = k_bytes > (int64_t(g.inplace ? 256 : 512) << 20);
  a.k_stream_nt1 = k_bytes > (int64_t(256) << 20);
  a.lambda = d->lambda;
  a.eps_tie = d->eps_tie;
  a.c_log2 = float(1.4426950408889634 / std::sqrt(double(d->head_dim)));
  a.n_sink = d->n_sink;
  a.n_recent = d->n_recent;
  a.step = d->step;
  a.seed = seed;
  a.n_avg = d->n_avg == 0 ? 1 : d->n_avg;
  a.head_floor = d->head_floor;
  return a;
}

struct Range {
  uintptr_t lo, hi;
};
Range span(const void* p, int64_t heads, int64_t stride_elems, int64_t last_elems, int32_t esz) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + uintptr_t(((heads - 1) * stride_elems + last_elems) * esz)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// ---- profiling (process-wide) ----
struct Profiler {
  std::mutex mu;
  uint32_t mask = 0;   // bit i: record events around stage i
  struct Rec { int stage; hipEvent_t e0, e1; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler& prof() { static Profiler p; return p; }

template <typename F>
hipError_t run_stage(int stage, hipStream_t s, F&& launch, bool profile = true) {
  Profiler& p = prof();
  if (!profile || !((p.mask >> stage) & 1u)) return launch();
  std::lock_guard<std::mutex> lock(p.mu);
  hipEvent_t e0 = p.get(), e1 = p.get();
  if (e0) (void)hipEventRecord(e0, s);
  const hipError_t err = launch();
  if (e1) (void)hipEventRecord(e1, s);
  if (e0 && e1) p.recs.push_back({stage, e0, e1});
  return err;
}

// NX_DEBUG (environment, read at every call): a non-empty value other than
// "0" makes each call synchronous -- after every stage the stream is
// synchronised, the HIP error state and the device status word are checked,
// and the first failure is returned by the entry point itself (the stage is
// named on stderr).  Skipped while the stream is being captured into a graph.
bool debug_mode() {
  const char* e = std::getenv("NX_DEBUG");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

nx_status debug_check(const Args& a, hipStream_t s, int stage) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return NX_EHIP;
  if (cap != hipStreamCaptureStatusNone) return NX_OK;
  const char* name = nx_stage_name(stage);
  hipError_t err = hipStreamSynchronize(s);
  if (err == hipSuccess) err = hipGetLastError();
  if (err != hipSuccess) {
    std::fprintf(stderr, "nexus debug: stage %s: %s\n", name, hipGetErrorString(err));
    return NX_EHIP;
  }
  uint32_t word = 0;
  if (a.status != nullptr &&
      hipMemcpy(&word, a.status, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return NX_EHIP;
  const nx_status st = (word & kStatusNonFinite) ? NX_ENONFINITE
                       : (word & kStatusBadItem) ? NX_EINVAL
                                                 : NX_OK;
  if (st != NX_OK) std::fprintf(stderr, "nexus debug: stage %s: %s\n", name, nx_status_str(st));
  return st;
}

// Enqueue stages [first, last] in order.
// Items of up to kWideMaxTokens units select on estimate codes (estimate_keys
// + sample_select; held in the select kernel's registers up to
// kFusedMaxTokens) when the call goes on to selection (not the weights-only
// export): n >= 1 draws per token, or the top-B-by-weight limit.
// profile = false keeps the HIP-event profiler (which creates events) out of the call.
nx_status enqueue(const Args& a, hipStream_t s, int first, int last, bool profile = true) {
  hipError_t err = hipSuccess;
  const bool debug = debug_mode();
  auto run_stage = [profile](int stage, hipStream_t st, auto&& launch) {
    return ::run_stage(stage, st, launch, profile);
  };
  const int max_units = (a.g.max_tokens + a.g.block - 1) / a.g.block;
  const bool fused = max_units <= kWideMaxTokens && !a.stop_after_weights &&
                     first <= kStageReservoirKeys && last >= kStageTopbSelect;
  // Calls of at most 4096 estimate_keys workgroups form the walk coefficients
  // inside estimate_keys (one launch fewer: on the single-layer shapes the
  // walk_coef launch cost ~9 us on its own; on the 32-layer event the fold
  // broke even).  Deep walks keep their Gram pass.
  const bool coef_in_keys = fused && !a.g.deep && a.w_in == nullptr && first <= kStageWalkCoef &&
                            int64_t(a.g.n_hu) * a.g.n_kc <= 4096;
  // Calls of at most 4096 second-sweep workgroups, each merging at most 4096
  // (tile, row) pairs, merge the row statistics in every second-sweep
  // workgroup instead of a score_combine launch (the 32-layer event: 16 x 128
  // pairs per workgroup; the 70B-shaped share, 64 x 512, keeps the launch).
  const bool beta_in_probs = first <= kStageScoreCombine && last >= kStageScoreProbs &&
                             int64_t(a.g.n_hu) * a.g.n_tmax <= 4096 &&
                             int64_t(a.g.n_tmax) * a.g.rows_pad <= 4096;
  Args sa = a;
  sa.beta_in_probs = beta_in_probs ? 1 : 0;
  // The stages from the keys on read the per-head budgets of this call.
  Args live = a;
  live.heads_live = 1;
  live.coef_in_keys = coef_in_keys ? 1 : 0;
  for (int st = first; st <= last && err == hipSuccess; ++st) {
    switch (st) {
      case kStageScoreStats: err = run_stage(st, s, [&] { return launch_score_stats(a, s); }); break;
      case kStageScoreCombine:
        if (!beta_in_probs) err = run_stage(st, s, [&] { return launch_score_combine(a, s); });
        break;
      case kStageScoreProbs: err = run_stage(st, s, [&] { return launch_score_probs(sa, s); }); break;
      case kStageWalkCoef:
        if (!coef_in_keys) err = run_stage(st, s, [&] { return launch_walk_coef(a, s); });
        break;
      case kStageReservoirKeys: {
        // Per-head budgets are settled before any stage that reads them.  On
        // the fused path with allocated budgets the estimate pass runs first
        // (it does not read the budgets) and also writes the weight codes.
        const bool heads = a.g.head_alloc != NX_HEADS_UNIFORM && !a.stop_after_weights;
        const bool est_first = heads && fused && a.g.head_alloc == NX_HEADS_ALLOC;
        Args pre = a;
        pre.coef_in_keys = coef_in_keys ? 1 : 0;
        pre.est_wcodes = est_first ? 1 : 0;
        pre.wcode_off = est_first ? a.g.max_tokens : 0;
        if (est_first) {
          err = run_stage(kStageEstimateKeys, s, [&] { return launch_estimate_keys(pre, s); });
          if (err != hipSuccess) break;
        }
        if (heads) {
          err = run_stage(kStageHeadBudget, s, [&] { return launch_head_budget(pre, s); });
          if (err != hipSuccess) break;
        }
        if (est_first) break;
        if (fused)
          err = run_stage(kStageEstimateKeys, s, [&] { return launch_estimate_keys(live, s); });
        else
          err = run_stage(st, s, [&] { return launch_reservoir_keys(live, s); });
        break;
      }
      case kStageTopbSelect:
        if (fused)
          err = run_stage(kStageSampleSelect, s, [&] { return launch_sample_select(live, s); });
        else
          err = run_stage(st, s, [&] { return launch_topb_select(live, s); });
        break;
      case kStageKvCompact: err = run_stage(st, s, [&] { return launch_kv_compact(live, s); }); break;
      case kStageHeadBudget: err = run_stage(st, s, [&] { return launch_head_budget(a, s); }); break;
      default: break;
    }
    if (err == hipSuccess && debug) {
      const nx_status dst = debug_check(a, s, st);
      if (dst != NX_OK) return dst;
    }
  }
  return err == hipSuccess ? NX_OK : NX_EHIP;
}

nx_unit single_unit(const nx_desc* d, const void* q, const void* k, const void* v, int32_t* keep,
                    void* out_k, void* out_v, int32_t n, int32_t budget) {
  nx_unit u;
  std::memset(&u, 0, sizeof(u));
  u.q = q;
  u.k = k;
  u.v = v;
  u.keep = keep;
  u.out_k = out_k;
  u.out_v = out_v;
  u.kv_head_stride = d->kv_head_stride ? d->kv_head_stride : int64_t(n) * d->head_dim;
  u.out_head_stride = d->out_head_stride ? d->out_head_stride
                                         : int64_t(budget) * (d->block > 1 ? d->block : 1) * d->head_dim;
  u.n_tokens = n;
  u.budget = budget;
  u.layer = d->layer;
  u.seq_id = d->seq_id;
  return u;
}

// ---- the no-allocation variant of nx_evict_step ----
// Its workspace is this file-scope device array, one copy per GPU that the
// library runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current, and
// only that address is ever handed to kernels or copies.
constexpr size_t kScratchBytes = size_t(NX_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

__global__ __launch_bounds__(64) void zero_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

// Device address of this device's scratch array (nullptr on a HIP error).  The
// first call on a device looks it up and clears the status word with a fill
// kernel on `s`; every later call returns the cached address.
void* scratch_ptr(hipStream_t s) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, s, static_cast<uint32_t*>(p), 64);
    if (hipGetLastError() != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

size_t nx_evict_workspace_bytes(const nx_desc* desc, int32_t max_tokens, int32_t max_units,
                                int32_t walk_iters) {
  Geometry g{};
  if (make_geometry(desc, max_tokens, max_units, walk_iters, &g) != NX_OK) return 0;
  return ws_layout(g).total;
}

static nx_status evict_step_impl(const nx_desc* desc, const void* q_window, const void* k_cache,
                                 const void* v_cache, int32_t n_tokens, int32_t budget,
                                 int32_t walk_iters, uint64_t seed, int32_t* out_keep_idx,
                                 void* out_k, void* out_v, bool profile) {
  Geometry g{};
  nx_status st = make_geometry(desc, n_tokens, 1, walk_iters, &g);
  if (st != NX_OK) return st;
  if (desc->head_alloc != NX_HEADS_UNIFORM) return NX_EINVAL;   // batch calls only
  const bool inplace = desc->compact == NX_COMPACT_INPLACE;
  if (!q_window || !k_cache || !v_cache || !out_keep_idx) return NX_EINVAL;
  if (inplace ? (out_k || out_v) : (!out_k || !out_v)) return NX_EINVAL;
  if (budget < 1 || desc->n_sink + desc->n_recent > budget) return NX_EINVAL;
  nx_unit u = single_unit(desc, q_window, k_cache, v_cache, out_keep_idx, out_k, out_v,
                          n_tokens, budget);
  u.out_w = desc->out_w;
  const int64_t d = desc->head_dim, hk = desc->n_kv_heads;
  const int32_t blk = desc->block > 1 ? desc->block : 1;
  const int32_t units = (n_tokens + blk - 1) / blk;
  const int32_t kept_units = budget < units ? budget : units;
  const int32_t kept = int32_t(std::min<int64_t>(int64_t(kept_units) * blk, n_tokens));   // rows
  if (u.kv_head_stride < n_tokens * d || u.out_head_stride < kept * d) return NX_EINVAL;
  const int32_t esz = elem_size(desc->dtype);
  const Range rk = span(k_cache, hk, u.kv_head_stride, n_tokens * d, esz);
  const Range rv = span(v_cache, hk, u.kv_head_stride, n_tokens * d, esz);
  const Range rq = span(q_window, 1, 0, int64_t(desc->n_q_heads) * desc->window * d, esz);
  const Range rkeep = span(out_keep_idx, 1, 0, hk * budget, 4);
  if (desc->out_w != nullptr) {
    // The weight export must not overlap anything else the call reads or writes.
    const Range rw = span(desc->out_w, 1, 0, hk * units, 4);
    for (Range i : {rk, rv, rq, rkeep})
      if (overlap(rw, i)) return NX_EALIAS;
    if (!inplace) {
      if (overlap(rw, span(out_k, hk, u.out_head_stride, kept * d, esz)) ||
          overlap(rw, span(out_v, hk, u.out_head_stride, kept * d, esz)))
        return NX_EALIAS;
    }
  }
  if (inplace) {
    // k and v are compacted in place: only the keep array must stay apart.
    for (Range i : {rk, rv, rq})
      if (overlap(rkeep, i)) return NX_EALIAS;
    if (overlap(rk, rv)) return NX_EALIAS;
  } else {
    const Range rok = span(out_k, hk, u.out_head_stride, kept * d, esz);
    const Range rov = span(out_v, hk, u.out_head_stride, kept * d, esz);
    for (Range o : {rok, rov, rkeep})
      for (Range i : {rk, rv, rq})
        if (overlap(o, i)) return NX_EALIAS;
    if (overlap(rok, rov) || overlap(rok, rkeep) || overlap(rov, rkeep)) return NX_EALIAS;
  }
  g.max_out_rows = kept;
  Args a = base_args(desc, g, seed);
  if ((st = bind_workspace(desc, g, &a)) != NX_OK) return st;
  a.single = u;
  return enqueue(a, static_cast<hipStream_t>(desc->stream), kStageScoreStats, kStageKvCompact,
                 profile);
}

nx_status nx_evict_step(const nx_desc* desc, const void* q_window, const void* k_cache,
                        const void* v_cache, int32_t n_tokens, int32_t budget, int32_t walk_iters,
                        uint64_t seed, int32_t* out_keep_idx, void* out_k, void* out_v) {
  return evict_step_impl(desc, q_window, k_cache, v_cache, n_tokens, budget, walk_iters, seed,
                         out_keep_idx, out_k, out_v, true);
}

nx_status nx_evict_step_noalloc(const nx_desc* desc, const void* q_window, const void* k_cache,
                                const void* v_cache, int32_t n_tokens, int32_t budget,
                                int32_t walk_iters, uint64_t seed, int32_t* out_keep_idx,
                                void* out_k, void* out_v) {
  if (desc == nullptr) return NX_EINVAL;
  void* ws = scratch_ptr(static_cast<hipStream_t>(desc->stream));
  if (ws == nullptr) return NX_EHIP;
  nx_desc d = *desc;
  d.workspace = ws;
  d.workspace_bytes = kScratchBytes;
  // The shape's workspace must fit the static scratch: NX_EWORKSPACE otherwise
  // (bind_workspace), before anything is enqueued.
  return evict_step_impl(&d, q_window, k_cache, v_cache, n_tokens, budget, walk_iters, seed,
                         out_keep_idx, out_k, out_v, false);
}

nx_status nx_evict_batch(const nx_desc* desc, const nx_unit* units_dev, int32_t n_units,
                         int32_t max_tokens, int32_t walk_iters, uint64_t seed) {
  Geometry g{};
  nx_status st = make_geometry(desc, max_tokens, n_units, walk_iters, &g);
  if (st != NX_OK) return st;
  if (units_dev == nullptr) return NX_EINVAL;
  if (desc->max_out_rows < 0) return NX_EINVAL;
  g.max_out_rows = desc->max_out_rows > 0 ? desc->max_out_rows : max_tokens;
  Args a = base_args(desc, g, seed);
  if ((st = bind_workspace(desc, g, &a)) != NX_OK) return st;
  a.units = units_dev;
  return enqueue(a, static_cast<hipStream_t>(desc->stream), kStageScoreStats, kStageKvCompact);
}

nx_status nx_nexus_weights(const nx_desc* desc, const void* q_window, const void* k_cache,
                           int32_t n_tokens, int32_t walk_iters, float* out_w) {
  Geometry g{};
  nx_status st = make_geometry(desc, n_tokens, 1, walk_iters, &g);
  if (st != NX_OK) return st;
  g.head_alloc = NX_HEADS_UNIFORM;   // weights do not depend on the budgets
  if (!q_window || !k_cache || !out_w) return NX_EINVAL;
  nx_unit u = single_unit(desc, q_window, k_cache, nullptr, nullptr, nullptr, nullptr, n_tokens,
                          n_tokens);
  if (u.kv_head_stride < int64_t(n_tokens) * desc->head_dim) return NX_EINVAL;
  if (desc->n_sink + desc->n_recent > n_tokens) return NX_EINVAL;
  u.out_w = out_w;
  Args a = base_args(desc, g, 0);
  if ((st = bind_workspace(desc, g, &a)) != NX_OK) return st;
  a.single = u;
  a.stop_after_weights = 1;
  return enqueue(a, static_cast<hipStream_t>(desc->stream), kStageScoreStats, kStageReservoirKeys);
}

nx_status nx_reservoir_select(const nx_desc* desc, const float* w, int32_t n_tokens,
                              int32_t budget, uint64_t seed, int32_t* out_keep_idx,
                              double* out_keys) {
  Geometry g{};
  nx_status st = make_geometry(desc, n_tokens, 1, 0, &g);
  if (st != NX_OK) return st;
  if (desc->head_alloc != NX_HEADS_UNIFORM) return NX_EINVAL;   // batch calls only
  g.block = 1;   // the given weights are the selection units
  if (!w || !out_keep_idx) return NX_EINVAL;
  if (budget < 1 || desc->n_sink + desc->n_recent > budget) return NX_EINVAL;
  // The scoring inputs are not used; q and k only need to be non-null.
  nx_unit u = single_unit(desc, w, w, nullptr, out_keep_idx, nullptr, nullptr, n_tokens, budget);
  u.kv_head_stride = int64_t(n_tokens) * desc->head_dim;
  Args a = base_args(desc, g, seed);
  if ((st = bind_workspace(desc, g, &a)) != NX_OK) return st;
  a.single = u;
  a.w_in = w;
  a.keys_out = out_keys;
  return enqueue(a, static_cast<hipStream_t>(desc->stream), kStageReservoirKeys, kStageTopbSelect);
}

nx_status nx_head_budgets(const nx_desc* desc, const float* w, int32_t n_tokens, int32_t budget,
                          int32_t head_cap, int32_t* out_head_budget) {
  Geometry g{};
  nx_status st = make_geometry(desc, n_tokens, 1, 0, &g);
  if (st != NX_OK) return st;
  g.block = 1;   // the given weights are the selection units
  if (desc->head_alloc != NX_HEADS_ALLOC) return NX_EINVAL;
  if (!w || !out_head_budget || budget < 1 || head_cap < 0) return NX_EINVAL;
  if (desc->n_sink + desc->n_recent > (head_cap > 0 ? head_cap : budget)) return NX_EINVAL;
  // The scoring inputs are not used; q and k only need to be non-null.
  nx_unit u = single_unit(desc, w, w, nullptr, nullptr, nullptr, nullptr, n_tokens, budget);
  u.kv_head_stride = int64_t(n_tokens) * desc->head_dim;
  u.head_cap = head_cap;
  u.head_budget = out_head_budget;
  Args a = base_args(desc, g, 0);
  if ((st = bind_workspace(desc, g, &a)) != NX_OK) return st;
  a.single = u;
  a.w_in = w;
  return enqueue(a, static_cast<hipStream_t>(desc->stream), kStageHeadBudget, kStageHeadBudget);
}

nx_status nx_kv_compact(const nx_desc* desc, const void* k_cache, const void* v_cache,
                        const int32_t* keep_idx, int32_t n_tokens, int32_t budget, void* out_k,
                        void* out_v) {
  Geometry g{};
  nx_status st = make_geometry(desc, n_tokens, 1, 0, &g);
  if (st != NX_OK) return st;
  if (desc->head_alloc != NX_HEADS_UNIFORM) return NX_EINVAL;   // batch calls only
  const bool inplace = desc->compact == NX_COMPACT_INPLACE;
  if (!k_cache || !v_cache || !keep_idx) return NX_EINVAL;
  if (inplace ? (out_k || out_v) : (!out_k || !out_v)) return NX_EINVAL;
  if (budget < 1) return NX_EINVAL;
  const nx_unit u = single_unit(desc, k_cache, k_cache, v_cache, const_cast<int32_t*>(keep_idx),
                                out_k, out_v, n_tokens, budget);
  const int64_t d = desc->head_dim, hk = desc->n_kv_heads;
  const int32_t blk = desc->block > 1 ? desc->block : 1;
  const int32_t units = (n_tokens + blk - 1) / blk;
  const int32_t kept_units = budget < units ? budget : units;
  const int32_t kept = int32_t(std::min<int64_t>(int64_t(kept_units) * blk, n_tokens));   // rows
  if (u.kv_head_stride < n_tokens * d || u.out_head_stride < kept * d) return NX_EINVAL;
  const int32_t esz = elem_size(desc->dtype);
  const Range rk = span(k_cache, hk, u.kv_head_stride, n_tokens * d, esz);
  const Range rv = span(v_cache, hk, u.kv_head_stride, n_tokens * d, esz);
  if (inplace) {
    if (overlap(rk, rv)) return NX_EALIAS;
  } else {
    const Range rok = span(out_k, hk, u.out_head_stride, kept * d, esz);
    const Range rov = span(out_v, hk, u.out_head_stride, kept * d, esz);
    for (Range o : {rok, rov})
      for (Range i : {rk, rv})
        if (overlap(o, i)) return NX_EALIAS;
    if (overlap(rok, rov)) return NX_EALIAS;
  }
  if (desc->workspace == nullptr || desc->workspace_bytes < 256) return NX_EWORKSPACE;
  g.max_out_rows = kept;
  Args a = base_args(desc, g, 0);
  a.status = static_cast<uint32_t*>(desc->workspace);   // the status word is the only scratch used
  a.single = u;
  return enqueue(a, static_cast<hipStream_t>(desc->stream), kStageKvCompact, kStageKvCompact);
}

nx_status nx_read_device_status(const nx_desc* desc) {
  if (desc == nullptr) return NX_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(desc->stream);
  void* ws = desc->workspace;
  if (ws == nullptr) {
    ws = scratch_ptr(s);   // the status of nx_evict_step_noalloc calls on this device
    if (ws == nullptr) return NX_EHIP;
  } else if (desc->workspace_bytes < 256) {
    return NX_EINVAL;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return NX_EHIP;
  uint32_t word = 0;
  if (hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return NX_EHIP;
  if (word != 0) {
    const uint32_t zero = 0;
    if (hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return NX_EHIP;
  }
  if (word & kStatusNonFinite) return NX_ENONFINITE;
  if (word & kStatusBadItem) return NX_EINVAL;
  return NX_OK;
}

const char* nx_status_str(nx_status s) {
  switch (s) {
    case NX_OK: return "NX_OK";
    case NX_EINVAL: return "NX_EINVAL: invalid argument";
    case NX_EALIAS: return "NX_EALIAS: output overlaps an input";
    case NX_EWORKSPACE: return "NX_EWORKSPACE: workspace missing or too small";
    case NX_EUNSUPPORTED: return "NX_EUNSUPPORTED: shape or dtype outside the built kernels";
    case NX_ENONFINITE: return "NX_ENONFINITE: non-finite Nexus weight";
    case NX_EHIP: return "NX_EHIP: HIP runtime error";
    default: return "unknown nx_status";
  }
}

nx_status nx_stream_read(const void* src, size_t bytes, int32_t mode, int32_t passes, void* sink,
                         void* stream) {
  if (src == nullptr || sink == nullptr || passes < 1 || (mode != 0 && mode != 1)) return NX_EINVAL;
  if (bytes == 0 || bytes % 256 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0) return NX_EINVAL;
  const int64_t rows = int64_t(bytes / 256);
  if (rows > (int64_t(1) << 22) * 65535) return NX_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t p = 0; p < passes; ++p)
    if (launch_stream_read(src, rows, mode, static_cast<uint32_t*>(sink), s) != hipSuccess) return NX_EHIP;
  return NX_OK;
}

nx_status nx_profile_enable(int32_t stage_mask) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  if (stage_mask) {
    for (auto& r : p.recs) { p.pool.push_back(r.e0); p.pool.push_back(r.e1); }
    p.recs.clear();
  }
  p.mask = uint32_t(stage_mask);
  return NX_OK;
}

int32_t nx_profile_read(float* stage_ms, int32_t* stage_launches, int32_t max_stages) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  const int n = max_stages < kNumStages ? max_stages : kNumStages;
  for (int i = 0; i < n; ++i) {
    if (stage_ms) stage_ms[i] = 0.f;
    if (stage_launches) stage_launches[i] = 0;
  }
  for (auto& r : p.recs) {
    if (r.stage >= n) continue;
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) == hipSuccess && hipEventElapsedTime(&ms, r.e0, r.e1) == hipSuccess) {
      if (stage_ms) stage_ms[r.stage] += ms;
      if (stage_launches) stage_launches[r.stage] += 1;
    }
  }
  return kNumStages;
}

const char* nx_stage_name(int32_t stage) {
  static const char* names[kNumStages] = {"score_stats", "score_combine",  "score_probs",
                                          "walk_coef",   "reservoir_keys", "topb_select",
                                          "kv_compact",  "sample_select", "estimate_keys",
                                          "head_budget"};
  return stage >= 0 && stage < kNumStages ? names[stage] : "unknown";
}

}  // extern "C"
