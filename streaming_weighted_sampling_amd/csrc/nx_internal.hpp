// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
//
// One eviction event runs these kernel stages over "head units" (one head
// unit = one KV head of one (sequence, layer) item):
//   score_stats    window logits Q K^T / sqrt(D) with bf16/fp32 MFMA; per tile
//                  and window row the max and the sum of exponentials
//   score_combine  merge the tile statistics of every window row
//   score_probs    logits again, probabilities averaged over the GQA group:
//                  direct score a, the H walk rows, and their Gram partials
//   walk_coef      reduce the Gram partials, run the walk recurrence, store
//                  the per-row coefficients gamma_t / ||C||_1
//   estimate_keys + sample_select (head units of up to kWideMaxTokens units,
//                  one draw per token): fp32 estimates of the keys, radix
//                  select (codes in registers up to kFusedMaxTokens units,
//                  else re-read per pass), exact fp64 keys near the boundary
//   reservoir_keys + topb_select (otherwise): Nexus weight, Philox uniform,
//                  fp64 key; radix select of the budget largest keys
//   kv_compact     gather of the kept K/V rows (+ optional appended rows), or
//                  kv_fill_holes + kv_append for in-place compaction
// and, with per-head budgets, head_budget (before the keys).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "../../include/nexus.h"

namespace nx {

constexpr int kMaxWalk = 8;          // walk depth H of the register-held walk forms
constexpr int kMaxWalkRows = 64;     // G * H window rows feeding those forms
// Deeper walks (H > kMaxWalk or G * H > kMaxWalkRows, up to kMaxWalkDeep with
// G <= 32): the second sweep writes every walk row P_t, a separate pass forms
// their Gram matrix, and the recurrence runs in LDS.
constexpr int kMaxWalkDeep = 64;
constexpr int kMaxCoef = kMaxWalkDeep;   // walk coefficient slots per head unit
constexpr int kGramChunk = 2048;     // units per Gram workgroup of the deep walk
constexpr int kMaxRows = 1024;       // G * W rows per head unit
constexpr int kMinTokPerBlock = 128;   // smallest token range of a score workgroup
constexpr int kMaxTokPerBlock = 2048;  // largest (chosen per call, power of two)
constexpr int kKeysPerBlock = 1024;  // tokens per reservoir_keys workgroup
constexpr int kCompactRows = 64;     // kept rows per kv_compact workgroup
constexpr int kFusedPer = 32;        // tokens per lane of the fused keys + select kernel
constexpr int kFusedMaxTokens = 1024 * kFusedPer;   // largest n it handles in registers
constexpr int kWideMaxTokens = 8 * kFusedMaxTokens;  // largest n of the estimate-code select
constexpr int kAllocBins = 4096;     // per-item histogram of bits 30..19 of the weight codes
constexpr int kAllocShift = 19;
constexpr int kAllocCand = 8192;     // boundary-bin codes held per item (and per head unit)

enum Stage {
  kStageScoreStats = 0,
  kStageScoreCombine,
  kStageScoreProbs,
  kStageWalkCoef,
  kStageReservoirKeys,
  kStageTopbSelect,
  kStageKvCompact,
  kStageSampleSelect,   // select on estimate codes (n <= kWideMaxTokens)
  kStageEstimateKeys,   // estimate codes of the keys (n <= kWideMaxTokens)
  kStageHeadBudget,     // per-head budgets (before the keys; NX_HEADS_GIVEN / _ALLOC)
  kNumStages
};

// Geometry of one call: everything the host derives from the descriptor.
struct Geometry {
  int32_t h_q, h_kv, group, head_dim, window, walk, rows, rows_pad, walk_rows;
  int32_t dtype;
  int32_t n_hu;          // head units = n_items * h_kv
  int32_t max_tokens;    // workspace row length: the call's max_tokens rounded up to 4
  int32_t max_n;         // the call's max_tokens (bound on every item's n_tokens)
  int32_t max_out_rows;  // compaction grid rows per head unit
  int32_t tok_per_block; // tokens per score workgroup for this call
  int32_t n_tmax;        // score tiles per head unit at tok_per_block (for max_tokens)
  int32_t n_t1, n_t2;    // workspace tile slots per head unit (sized for kMinTokPerBlock)
  int32_t n_kc;          // reservoir_keys chunks per head unit
  int32_t block;         // tokens per selection unit (1, or a block size up to 32)
  int32_t inplace;       // 1: compaction rearranges k / v in place (hole filling)
  int32_t head_alloc;    // NX_HEADS_UNIFORM / _GIVEN / _ALLOC
  int32_t deep;          // 1: deep walk (walk rows stored whole, Gram in its own pass)
  int32_t n_gc;          // Gram chunks per head unit (deep walk)
  int32_t packed;        // 1: a_j and the walk rows as one 16-B record per token (packed_rows)
};

// Walks of exactly three rows at token granularity with G = 4 or 8 (the
// second sweep's exact-depth kernels): the second sweep writes a_j, P_1[j],
// P_2[j], P_3[j] as one 16-byte record per token instead of four planar rows.
inline bool packed_rows(int walk, int group, int block, bool deep) {
  return walk == 3 && (group == 4 || group == 8) && block <= 1 && !deep;
}

// Workspace carving (byte offsets from the workspace base, 256-B aligned).
struct WsLayout {
  size_t status, part1, beta, a, p, gram, coef, keys, selp, ahist, acand, acnt, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(const Geometry& g) {
  WsLayout L{};
  size_t off = 0;
  const size_t hu = size_t(g.n_hu), nm = size_t(g.max_tokens);
  L.status = off; off = align256(off + 256);
  L.part1 = off;  off = align256(off + hu * g.n_t1 * g.rows_pad * 2 * sizeof(float));
  L.beta = off;   off = align256(off + hu * g.rows_pad * sizeof(float));
  if (g.packed) {   // records [n_hu][max_tokens][4]
    L.a = off;    off = align256(off + hu * nm * 4 * sizeof(float));
    L.p = L.a;
  } else {
    L.a = off;    off = align256(off + hu * nm * sizeof(float));
    L.p = off;    off = align256(off + hu * size_t(g.walk) * nm * sizeof(float));   // none for H = 0
  }
  // Gram partials: per score tile [kMaxWalk][kMaxWalk]; deep walk: per Gram
  // chunk [H][H].
  const size_t gram_floats = g.deep ? size_t(g.n_gc) * g.walk * g.walk
                                    : size_t(g.n_t2) * kMaxWalk * kMaxWalk;
  L.gram = off;   off = align256(off + hu * gram_floats * sizeof(float));
  L.coef = off;   off = align256(off + hu * kMaxCoef * sizeof(float));
  L.keys = off;   off = align256(off + hu * nm * sizeof(uint64_t));
  L.selp = off;   off = align256(off + hu * g.n_kc * 2 * sizeof(uint64_t));
  // per-item histogram of the per-head allocation (cleared by each call that builds it)
  L.ahist = off;
  if (g.head_alloc == NX_HEADS_ALLOC) off = align256(off + (hu / g.h_kv) * kAllocBins * sizeof(uint32_t));
  // per head unit: its boundary-bin codes and (count above, candidate count)
  L.acand = off;
  if (g.head_alloc == NX_HEADS_ALLOC) off = align256(off + hu * kAllocCand * sizeof(uint32_t));
  L.acnt = off;
  if (g.head_alloc == NX_HEADS_ALLOC) off = align256(off + hu * 2 * sizeof(int32_t));
  L.total = off;
  return L;
}

// Device status bits (OR-ed into the workspace status word).
constexpr uint32_t kStatusNonFinite = 1u;
constexpr uint32_t kStatusBadItem = 2u;

// Kernel argument block, passed by value to every stage.
struct Args {
  const nx_unit* units;   // device array of items, or nullptr: use `single`
  nx_unit single;
  Geometry g;
  float lambda, eps_tie, c_log2;   // c_log2 = log2(e) / sqrt(D)
  int32_t n_sink, n_recent;
  uint32_t step;
  int32_t n_avg;   // 1, 2 .. NX_MAX_AVG draws, or NX_TOPK
  int32_t k_stream_nt;   // 1: the second score sweep copies K with the non-temporal hint
  int32_t k_stream_nt1;  // 1: the first score sweep does
  uint64_t seed;
  // workspace
  uint32_t* status;
  float* part1;    // [n_hu][n_t1][rows_pad][2]: (max, sum) in log2 units
  float* beta;     // [n_hu][rows_pad]
  float* a;        // [n_hu][max_tokens]: direct score (packed: [n_hu][max_tokens][4] records)
  float* p;        // [n_hu][walk][max_tokens] (packed: unused)
  float* gram;     // [n_hu][n_t2][kMaxWalk * kMaxWalk]
  float* coef;     // [n_hu][kMaxWalk]: gamma_t / ||C||_1
  uint64_t* keys;  // [n_hu][max_tokens], order-preserving bits of the fp64 key
  uint64_t* selp;  // [n_hu][n_kc][2]: OR and AND of the chunk's keys
  uint32_t* ahist; // [n_items][kAllocBins]: allocation histogram (zero between calls)
  uint32_t* acand; // [n_hu][kAllocCand]: boundary-bin codes of each head unit
  int32_t* acnt;   // [n_hu][2]: codes above the boundary bin, codes in it
  // stage-only extras
  const float* w_in;    // reservoir-only mode: weights [h_kv][n] (row stride n)
  double* keys_out;     // optional key export [h_kv][n]
  int32_t stop_after_weights;  // 1: reservoir_keys writes the weight export and stops
  int32_t head_floor;   // NX_HEADS_ALLOC floor
  int32_t heads_live;   // 1: the items' head_budget arrays hold this call's budgets
  int32_t est_wcodes;   // 1: estimate_keys also writes the allocation's weight codes
  int32_t coef_in_keys; // 1: estimate_keys forms the walk coefficients (no walk_coef launch)
  int32_t beta_in_probs; // 1: score_probs merges the row statistics itself (no score_combine launch)
  int32_t wcode_off;    // uint32 offset of the weight codes in a head unit's key array
};

hipError_t launch_score_stats(const Args& a, hipStream_t s);
hipError_t launch_score_combine(const Args& a, hipStream_t s);
hipError_t launch_score_probs(const Args& a, hipStream_t s);
hipError_t launch_walk_coef(const Args& a, hipStream_t s);
hipError_t launch_reservoir_keys(const Args& a, hipStream_t s);
hipError_t launch_topb_select(const Args& a, hipStream_t s);
hipError_t launch_sample_select(const Args& a, hipStream_t s);
hipError_t launch_estimate_keys(const Args& a, hipStream_t s);
hipError_t launch_kv_compact(const Args& a, hipStream_t s);
hipError_t launch_head_budget(const Args& a, hipStream_t s);
// Read-ceiling probe: rows of 256 B at src, mode 0 (LDS ring) or 1 (vector loads).
hipError_t launch_stream_read(const void* src, int64_t rows, int mode, uint32_t* sink,
                              hipStream_t s);

}  // namespace nx
