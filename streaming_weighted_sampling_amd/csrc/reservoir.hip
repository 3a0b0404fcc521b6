// Weighted reservoir selection on gfx950.
//
// [Nexus] = "Forget Without Compromise: Nexus Sampling for Streaming KV-Cache
// Eviction Under Fixed Budgets" (academ.us article page).
//
// walk_coef       (one wavefront per head unit)
//   * walk coefficients of section 2.2 Eq. (4) from the Gram partials of the
//     walk rows P_t: gamma_1 = 1, gamma_t = 1 + sum_{t'<t} gamma_t' <P_t, P_t'>,
//     so that c~_j = sum_t gamma_t P_t[j] / ||C||_1, ||C||_1 = sum_t gamma_t |P_t|_1
//     (the rank-1 form of the recurrence, appendix 8.6; no N-vector is carried)
// reservoir_keys  (many workgroups per head unit, 1024 tokens each)
//   * Nexus weight w_j = a_j + lambda c~_j + eps j/(N-1) (Eqs. 2 and 5)
//   * Philox4x32-10 uniform u_j, counter (j, unit, layer, step), key = seed
//   * A-Res key ln(u_j)/w_j in fp64 (section 2.3 Eq. 6 with n = 1), -inf for
//     w <= 0, +inf for the forced sink / recency slots, stored as an
//     order-preserving uint64 code, plus the chunk's OR and AND of the codes
// topb_select  (one 1024-thread workgroup per head unit)
//   * skips the common prefix of all codes, then MSD radix select with
//     8-bit digits: LDS histogram of the candidates (each bin in 8 words, one
//     per lane residue), boundary bin by a wavefront suffix scan, until the
//     boundary bin holds exactly the missing count or all 64 bits are fixed
//     (true ties: larger index wins)
//   * writes the kept indices in ascending order with per-lane keep masks,
//     ballots and one scan per 32 rounds of 1024 tokens.
// estimate_keys + sample_select (the default path, head units of up to
// 262144 units): an fp32 order code of every key (n = 1, n >= 2 averaged
// draws, or the top-B limit), the same radix select on the codes (held in
// registers up to 32768 units, re-read from memory above), and exact fp64
// keys only for the tokens within +-2^-9 of the boundary estimate.
#include <algorithm>
#include <type_traits>

#include "nx_device.hpp"

namespace nx {
namespace {

constexpr int kKeysThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
static_assert(kFusedMaxTokens == kSelThreads * kFusedPer, "fused select covers 1024 lanes");

// One wavefront per head unit: fixed-order reduction of the per-tile Gram
// partials (lane-strided sums, then a butterfly), then the walk recurrence
// of section 2.2 Eq. (4) in its rank-1 form: gamma_1 = 1,
// gamma_t = 1 + sum_{t'<t} gamma_t' <P_t, P_t'>, ||C||_1 = sum_t gamma_t |P_t|_1.
// Lane 0 writes the coefficients gamma_t / ||C||_1 for t < kMaxWalk (zero past
// the walk) to `out`.
__device__ inline void walk_coef_unit(const Args& a, const HeadUnit& u, int hu, int lane, float* out) {
  const Geometry& g = a.g;
  const int n_tiles = (u.n + g.tok_per_block - 1) / g.tok_per_block;
  const float* gp = a.gram + size_t(hu) * g.n_t2 * (kMaxWalk * kMaxWalk);
  float gm[kMaxWalk][kMaxWalk];
#pragma unroll
  for (int t = 0; t < kMaxWalk; ++t)
#pragma unroll
    for (int t2 = 0; t2 < kMaxWalk; ++t2) gm[t][t2] = 0.f;
  for (int tl = lane; tl < n_tiles; tl += 64) {
#pragma unroll
    for (int t = 0; t < kMaxWalk; ++t)
#pragma unroll
      for (int t2 = 0; t2 <= t; ++t2)
        if (t < g.walk) gm[t][t2] += gp[size_t(tl) * (kMaxWalk * kMaxWalk) + t * kMaxWalk + t2];
  }
#pragma unroll
  for (int t = 0; t < kMaxWalk; ++t)
#pragma unroll
    for (int t2 = 0; t2 <= t; ++t2)
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) gm[t][t2] += __shfl_xor(gm[t][t2], m, 64);
  if (lane == 0) {
    float gam[kMaxWalk];
    float norm = 0.f;
#pragma unroll
    for (int t = 0; t < kMaxWalk; ++t) {
      float x = 1.f;
#pragma unroll
      for (int t2 = 0; t2 < t; ++t2) x = fmaf(gam[t2], gm[t][t2], x);
      gam[t] = x;
      if (t < g.walk) norm = fmaf(x, gm[t][t], norm);
    }
#pragma unroll
    for (int t = 0; t < kMaxWalk; ++t) out[t] = (t < g.walk) ? gam[t] / norm : 0.f;
  }
}

__global__ __launch_bounds__(64) void walk_coef_kernel(const Args a) {
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  walk_coef_unit(a, u, hu, threadIdx.x, a.coef + size_t(hu) * kMaxCoef);
}

// ---- deep walks (H > kMaxWalk or G * H > kMaxWalkRows) --------------------
//
// Gram partials of the stored walk rows: one workgroup per (chunk of
// kGramChunk units, head unit) sums P_t[j] P_t'[j] (t' < t) and, on the
// diagonal, P_t[j] (the row's L1 norm: the rows are non-negative) over its
// units in ascending order, as the second sweep's own partials hold them; 64
// units at a time staged in LDS (row stride 65 floats: the lanes of a
// wavefront, on different rows t, read different banks).
constexpr int kGramStage = 64;
__global__ __launch_bounds__(256) void gram_deep_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.y, chunk = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int j0 = chunk * kGramChunk;
  if (j0 >= u.nu) return;
  const int j1 = min(j0 + kGramChunk, u.nu);
  const int H = g.walk, n_pairs = H * (H + 1) / 2;
  constexpr int kPairs = (kMaxWalkDeep * (kMaxWalkDeep + 1) / 2 + 255) / 256;
  __shared__ float s_p[kMaxWalkDeep][kGramStage + 1];
  const float* p_in = a.p + size_t(hu) * g.walk * g.max_tokens;
  int pt[kPairs], pt2[kPairs];
  float acc[kPairs];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int p = threadIdx.x + 256 * k;
    int t = 0;
    while ((t + 1) * (t + 2) / 2 <= p) ++t;
    pt[k] = t;
    pt2[k] = p - t * (t + 1) / 2;
    acc[k] = 0.f;
  }
  for (int c0 = j0; c0 < j1; c0 += kGramStage) {
    const int cn = min(kGramStage, j1 - c0);
    __syncthreads();
    for (int i = threadIdx.x; i < H * kGramStage; i += 256) {
      const int t = i / kGramStage, jj = i - t * kGramStage;
      s_p[t][jj] = jj < cn ? p_in[size_t(t) * g.max_tokens + c0 + jj] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      if (threadIdx.x + 256 * k < n_pairs) {
        const float* x = s_p[pt[k]];
        const float* y = s_p[pt2[k]];
        float s0 = acc[k];
        if (pt[k] == pt2[k]) {
          for (int jj = 0; jj < cn; ++jj) s0 += x[jj];
        } else {
          for (int jj = 0; jj < cn; ++jj) s0 = fmaf(x[jj], y[jj], s0);
        }
        acc[k] = s0;
      }
    }
  }
  float* out = a.gram + (size_t(hu) * g.n_gc + chunk) * H * H;
#pragma unroll
  for (int k = 0; k < kPairs; ++k)
    if (threadIdx.x + 256 * k < n_pairs) out[pt[k] * H + pt2[k]] = acc[k];
}

// Walk coefficients of a deep walk, one workgroup per head unit: the chunk
// partials summed in chunk order (one thread per Gram entry), then the walk
// recurrence of section 2.2 Eq. (4) in its rank-1 form by one thread, with
// the same fused multiply-adds as walk_coef_kernel.
__global__ __launch_bounds__(256) void walk_coef_deep_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int H = g.walk, n_pairs = H * (H + 1) / 2;
  const int n_chunks = (u.nu + kGramChunk - 1) / kGramChunk;
  __shared__ float s_gm[kMaxWalkDeep][kMaxWalkDeep + 1];
  const float* gp = a.gram + size_t(hu) * g.n_gc * H * H;
  for (int p = threadIdx.x; p < n_pairs; p += 256) {
    int t = 0;
    while ((t + 1) * (t + 2) / 2 <= p) ++t;
    const int t2 = p - t * (t + 1) / 2;
    float sum = 0.f;
    for (int c = 0; c < n_chunks; ++c) sum += gp[size_t(c) * H * H + t * H + t2];
    s_gm[t][t2] = sum;
  }
  __syncthreads();
  __shared__ float s_gam[kMaxWalkDeep];
  __shared__ float s_norm;
  if (threadIdx.x == 0) {
    float norm = 0.f;
    for (int t = 0; t < H; ++t) {
      float x = 1.f;
      for (int t2 = 0; t2 < t; ++t2) x = fmaf(s_gam[t2], s_gm[t][t2], x);
      s_gam[t] = x;
      norm = fmaf(x, s_gm[t][t], norm);
    }
    s_norm = norm;
  }
  __syncthreads();
  if (threadIdx.x < kMaxCoef)
    a.coef[size_t(hu) * kMaxCoef + threadIdx.x] = int(threadIdx.x) < H ? s_gam[threadIdx.x] / s_norm : 0.f;
}

// w_j = a_j + lambda c~_j + eps r_j (section 2.2 Eqs. 2 and 5) with
// c~_j = sum_t coef_t P_t[j] and r_j = j ramp, ramp = 1/(N-1).  Every fused
// multiply-add is written out, so each kernel that forms a token's weight gets
// the same bits (a weight export equals the weight the keys were drawn on).
// kW >= 0: the walk depth, fixed at compile time (the same multiply-adds).
template <int kW = -1>
__device__ __attribute__((always_inline)) inline float combine_weight(
    const Args& a, const float* s_coef, float aj, const float (&pv)[kMaxWalk], int j, float ramp) {
  const int walk = kW >= 0 ? kW : a.g.walk;
  float cj = 0.f;
#pragma unroll
  for (int t = 0; t < kMaxWalk; ++t)
    if (t < walk) cj = fmaf(s_coef[t], pv[t], cj);
  const float r = float(j) * ramp;
  return fmaf(a.eps_tie, r, fmaf(a.lambda, cj, aj));
}

// The same weight for walks deeper than kMaxWalk: the walk rows are read
// eight at a time, and the multiply-adds run in the same order.
__device__ inline float deep_weight(const Args& a, const float* s_coef, const float* a_in,
                                    const float* p_in, float ramp, int j) {
  float cj = 0.f;
  for (int t0 = 0; t0 < a.g.walk; t0 += 8) {
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pv[i] = t0 + i < a.g.walk ? p_in[size_t(t0 + i) * a.g.max_tokens + j] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (t0 + i < a.g.walk) cj = fmaf(s_coef[t0 + i], pv[i], cj);
  }
  const float r = float(j) * ramp;
  return fmaf(a.eps_tie, r, fmaf(a.lambda, cj, a_in[j]));
}

// The fp64 key of token j with weight w (section 2.3 Eq. 6).  n = 1: ln(u)/w
// (A-Res).  n >= 2: ln(pi), pi = (1/n) sum_i u_i^(1/w), by an online
// log-sum-exp of t_i = ln(u_i)/w (u^(1/w) underflows for small w); draws 2c
// and 2c + 1 come from Philox block c, the token's counter under key
// (seed lo, seed hi + c), words (x, y) and (z, w).  NX_TOPK: the key is w
// itself (the n -> infinity limit ranks by w/(w+1), appendix 8.2).  w <= 0
// gives -inf, a forced slot +inf.
__device__ inline double token_key(const Args& a, const HeadUnit& u, int j, float w, uint32_t k0,
                                   uint32_t k1) {
  double key;
  if (!(w > 0.f)) {
    key = -INFINITY;
  } else if (a.n_avg == NX_TOPK) {
    key = double(w);
  } else if (a.n_avg <= 1) {
    const uint4 x = philox4x32_10(make_uint4(uint32_t(j), u.unit_id, u.layer, a.step), k0, k1);
    key = log(philox_uniform53(x.x, x.y)) / double(w);
  } else {
    const double rw = 1.0 / double(w);
    double m = -INFINITY, sum = 0.0;
    for (int c = 0; 2 * c < a.n_avg; ++c) {
      const uint4 x = philox4x32_10(make_uint4(uint32_t(j), u.unit_id, u.layer, a.step), k0,
                                    k1 + uint32_t(c));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (2 * c + h < a.n_avg) {
          const double t = log(h == 0 ? philox_uniform53(x.x, x.y) : philox_uniform53(x.z, x.w)) * rw;
          if (t > m) {
            sum = sum * exp(m - t) + 1.0;
            m = t;
          } else {
            sum += exp(t - m);
          }
        }
      }
    }
    key = m + log(sum) - log(double(a.n_avg));
  }
  if (j < a.n_sink || j >= u.nu - a.n_recent) key = INFINITY;
  return key;
}

__global__ __launch_bounds__(kKeysThreads) void reservoir_keys_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.y, chunk = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int j0 = chunk * kKeysPerBlock;
  if (j0 >= u.nu) return;
  __shared__ float s_coef[kMaxCoef];
  __shared__ uint64_t s_or[kKeysThreads / 64], s_and[kKeysThreads / 64];

  if (threadIdx.x < kMaxCoef)
    s_coef[threadIdx.x] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxCoef + threadIdx.x] : 0.f;
  __syncthreads();

  const ScoreRows sr = score_rows(a, hu);
  uint64_t* keys = a.keys + size_t(hu) * g.max_tokens;
  const size_t ext = size_t(u.h) * u.nu;   // row of head h in [h_kv, n] exports
  const float ramp = u.nu > 1 ? 1.f / float(u.nu - 1) : 0.f;
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  uint64_t v_or = 0, v_and = ~0ull;
  bool nonfinite = false;
  // Each lane owns kPer tokens j0 + lane + 256 i: every input load of the
  // lane is issued before the first Philox / log, so one memory latency
  // covers all of them.
  constexpr int kPer = kKeysPerBlock / kKeysThreads;
  float w[kPer];
  bool in[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + threadIdx.x + kKeysThreads * i;
    in[i] = j < u.nu;
    const int jc = in[i] ? j : j0;   // a valid token for the lanes past the end
    if (a.w_in != nullptr) {
      w[i] = a.w_in[ext + jc];
    } else if (g.walk > kMaxWalk) {
      w[i] = deep_weight(a, s_coef, sr.a, sr.p, ramp, jc);
    } else {
      // The same arithmetic as token_weight, loads first.
      float pv[kMaxWalk];
#pragma unroll
      for (int t = 0; t < kMaxWalk; ++t) pv[t] = t < g.walk ? sr.p[t * sr.rs + size_t(jc) * sr.ts] : 0.f;
      w[i] = combine_weight(a, s_coef, sr.a[size_t(jc) * sr.ts], pv, jc, ramp);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (!in[i]) continue;
    const int j = j0 + threadIdx.x + kKeysThreads * i;
    nonfinite |= !isfinite(w[i]);
    if (u.w_out != nullptr) u.w_out[j] = w[i];
    if (a.stop_after_weights) continue;
    const double key = token_key(a, u, j, w[i], k0, k1);
    if (a.keys_out != nullptr) a.keys_out[ext + j] = key;
    const uint64_t code = key_code(key);
    keys[j] = code;
    v_or |= code;
    v_and &= code;
  }
  if (__syncthreads_or(nonfinite) && threadIdx.x == 0) raise_status(a, kStatusNonFinite);
  if (a.stop_after_weights) return;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    v_or |= __shfl_xor(v_or, m, 64);
    v_and &= __shfl_xor(v_and, m, 64);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_or[wave] = v_or; s_and[wave] = v_and; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t o = 0, n = ~0ull;
    for (int w = 0; w < kKeysThreads / 64; ++w) { o |= s_or[w]; n &= s_and[w]; }
    uint64_t* sp = a.selp + (size_t(hu) * g.n_kc + chunk) * 2;
    sp[0] = o;
    sp[1] = n;
  }
}

// Exclusive prefix count of `flag` over the block (ascending thread order);
// returns the block total in *total.  Uses s_cnt[kSelWaves].
template <int kThr = kSelThreads>
__device__ inline int block_rank(bool flag, int* s_cnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_cnt[wave] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < (kThr / 64); ++w) {
    const int c = s_cnt[w];
    off += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + below;
}

// Kept indices in ascending order: keep_at(j) decides token j; tokens are
// taken in groups of kFusedPer rounds of kSelThreads (thread tid holds tokens
// (r0 + r) * kSelThreads + tid), with per-lane keep masks, per (round,
// wavefront) counts and one exclusive scan per group.  round_cnt holds
// kFusedPer * kSelWaves ints; every thread of the block calls this.
template <int kThr = kSelThreads, typename KeepAt>
__device__ inline void write_ascending(int n, int budget, int32_t* keep, int* round_cnt,
                                       int* group_total, KeepAt&& keep_at) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below_lane = (1ull << lane) - 1ull;
  const int slots = (n + kThr - 1) / kThr;
  int base = 0;
  for (int r0 = 0; r0 < slots; r0 += kFusedPer) {
    uint32_t kmask = 0;
#pragma unroll
    for (int r = 0; r < kFusedPer; ++r) {
      const int j = (r0 + r) * kThr + tid;
      if (j < n && keep_at(j)) kmask |= 1u << r;
    }
#pragma unroll
    for (int r = 0; r < kFusedPer; ++r) {
      const uint64_t bal = __ballot((kmask >> r) & 1u);
      if (lane == 0) round_cnt[r * (kThr / 64) + wave] = __popcll(bal);
    }
    __syncthreads();
    if (tid < 64) {
      constexpr int kPerLane = kFusedPer * (kThr / 64) / 64;
      int loc[kPerLane], sum = 0;
#pragma unroll
      for (int q = 0; q < kPerLane; ++q) { loc[q] = sum; sum += round_cnt[lane * kPerLane + q]; }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      const int excl = incl - sum;
#pragma unroll
      for (int q = 0; q < kPerLane; ++q) round_cnt[lane * kPerLane + q] = excl + loc[q];
      if (lane == 63) *group_total = incl;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kFusedPer; ++r) {
      const uint64_t bal = __ballot((kmask >> r) & 1u);
      if ((kmask >> r) & 1u) {
        const int pos = base + round_cnt[r * (kThr / 64) + wave] + __popcll(bal & below_lane);
        if (pos < budget) keep[pos] = (r0 + r) * kThr + tid;
      }
    }
    base += *group_total;
    __syncthreads();   // round_cnt and group_total are rewritten by the next group
  }
}

// The same ascending write over codes in memory, four consecutive tokens per
// lane: round r of a group covers kSelThreads * 4 tokens, lane tid the four at
// 4 ((g0 + r) kSelThreads + tid), read with one 16-byte load (the code array
// holds at least ceil(n / 4) * 4 codes); eight rounds (eight loads per lane
// in flight) per group and one scan per group.  A lane's offset inside its
// wavefront is the sum of the kept counts (0..4) of the lanes below it, taken
// from three ballots over the counts' bits.  keep_at(j, code) decides token j;
// round_cnt holds at least 8 * kSelWaves ints.
template <typename KeepAt>
__device__ inline void write_ascending4(const uint32_t* codes, int n, int budget, int32_t* keep,
                                        int* round_cnt, int* group_total, KeepAt&& keep_at) {
  constexpr int kR = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below_lane = (1ull << lane) - 1ull;
  const uint4* c4 = reinterpret_cast<const uint4*>(codes);
  const int n4 = (n + 3) >> 2;
  int base = 0;
  for (int g0 = 0; g0 * kSelThreads < n4; g0 += kR) {
    uint4 c[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int q = (g0 + r) * kSelThreads + tid;
      c[r] = q < n4 ? c4[q] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t m[kR];   // keep mask of the lane's four tokens
    int pre[kR];      // kept tokens of the lanes below, in this wavefront
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int j = 4 * ((g0 + r) * kSelThreads + tid);
      m[r] = 0u;
      if (j < n && keep_at(j, c[r].x)) m[r] |= 1u;
      if (j + 1 < n && keep_at(j + 1, c[r].y)) m[r] |= 2u;
      if (j + 2 < n && keep_at(j + 2, c[r].z)) m[r] |= 4u;
      if (j + 3 < n && keep_at(j + 3, c[r].w)) m[r] |= 8u;
      const uint32_t cnt = uint32_t(__popc(m[r]));
      const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u);
      pre[r] = __popcll(b0 & below_lane) + 2 * __popcll(b1 & below_lane) + 4 * __popcll(b2 & below_lane);
      if (lane == 0) round_cnt[r * kSelWaves + wave] = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    }
    __syncthreads();
    if (tid < 64) {
      constexpr int kPerLane = kR * kSelWaves / 64;
      int loc[kPerLane], sum = 0;
#pragma unroll
      for (int q = 0; q < kPerLane; ++q) { loc[q] = sum; sum += round_cnt[lane * kPerLane + q]; }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      const int excl = incl - sum;
#pragma unroll
      for (int q = 0; q < kPerLane; ++q) round_cnt[lane * kPerLane + q] = excl + loc[q];
      if (lane == 63) *group_total = incl;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      if (m[r] != 0u) {
        int pos = base + round_cnt[r * kSelWaves + wave] + pre[r];
        const int j = 4 * ((g0 + r) * kSelThreads + tid);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((m[r] >> e) & 1u) {
            if (pos < budget) keep[pos] = j + e;
            ++pos;
          }
        }
      }
    }
    base += *group_total;
    __syncthreads();   // round_cnt and group_total are rewritten by the next group
  }
}

// Shared state of one radix selection.  After the passes: keys whose bits
// under `mask` exceed `prefix` are kept; of the `eq` keys equal to it under
// the mask, `need` are kept (all of them when eq == need, else the ones with
// the largest indices: true ties, every bit fixed).
// Each digit bin is counted in kHistCopies words, one per lane residue mod
// kHistCopies: lanes that share a bin then hit at most 64 / kHistCopies the
// same LDS word (same-address atomics of a wavefront serialise; the estimate
// codes' first digit puts most of a wavefront in a few bins).
constexpr int kHistCopies = 8;

struct SelCore {
  uint32_t hist[256 * kHistCopies];   // [bin][copy]
  uint64_t prefix, mask;
  int need, eq, done, start, cut;
  int cnt[kSelWaves];
  uint64_t red_or[kSelWaves], red_and[kSelWaves];
  int round_cnt[kFusedPer * kSelWaves];   // write_ascending
  int group_total;
};

// Thread 0: the state before the passes, from the OR and AND of all codes
// (the bits above the highest differing one are common to every code).
__device__ inline void sel_init(SelCore& sh, uint64_t o, uint64_t an, int n, int budget) {
  const uint64_t diff = o ^ an;
  sh.need = budget;
  sh.eq = n;
  if (diff == 0) {                       // every code equal: pure ties
    sh.prefix = an;
    sh.mask = ~0ull;
    sh.done = 1;
  } else {
    const int top = 63 - __clzll(diff);  // highest bit that differs
    const uint64_t above = top == 63 ? 0ull : (~0ull << (top + 1));
    sh.prefix = an & above;
    sh.mask = above;
    sh.done = 0;
    sh.start = top;
  }
}

// Wave 0 after a histogram pass: lane l owns bins 4l..4l+3; suffix sums over
// the lanes find the bin that holds the need-th largest candidate.
__device__ inline void sel_pick_bin(SelCore& sh, int shift, uint32_t dmask) {
  const int lane = threadIdx.x & 63;
  // (copy 0 of each bin holds the bin's total; see sel_passes)
  const uint32_t h0 = sh.hist[(4 * lane) * kHistCopies], h1 = sh.hist[(4 * lane + 1) * kHistCopies],
                 h2 = sh.hist[(4 * lane + 2) * kHistCopies], h3 = sh.hist[(4 * lane + 3) * kHistCopies];
  const uint32_t own = h0 + h1 + h2 + h3;
  uint32_t suf = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += v;
  }
  const uint32_t higher = suf - own;   // candidates in bins above this lane's
  const uint32_t need = uint32_t(sh.need);
  if (higher < need && need <= suf) {
    const uint32_t c3 = higher + h3, c2 = c3 + h2, c1 = c2 + h1;
    const int b = need <= c3 ? 3 : need <= c2 ? 2 : need <= c1 ? 1 : 0;
    const uint32_t acc = b == 3 ? higher : b == 2 ? c3 : b == 1 ? c2 : c1;
    const uint32_t hb = b == 3 ? h3 : b == 2 ? h2 : b == 1 ? h1 : h0;
    sh.need = int(need - acc);
    sh.eq = int(hb);
    sh.prefix = sh.prefix | (uint64_t(4 * lane + b) << shift);
    sh.mask = sh.mask | (uint64_t(dmask) << shift);
    sh.done = (hb == need - acc) || shift == 0;
  }
}

// MSD radix passes with 8-bit digits over the unresolved bits, highest first,
// until the boundary bin holds exactly the missing count or every bit is
// fixed; at most 64 bits, so at most 8 passes.  Each pass clears the digit
// histogram (sel_pass_begin), counts the candidates under the current prefix
// (one atomic per code) and picks the boundary bin (sel_pass_end).
__device__ inline void sel_pass_begin(SelCore& sh, int start, int* shift, uint32_t* dmask) {
  *shift = start >= 7 ? start - 7 : 0;
  *dmask = (1u << (start - *shift + 1)) - 1u;
  for (int b = threadIdx.x; b < 256 * kHistCopies; b += blockDim.x) sh.hist[b] = 0;
  __syncthreads();
}
__device__ inline void sel_pass_end(SelCore& sh, int shift, uint32_t dmask) {
  __syncthreads();
  if (threadIdx.x < 256) {   // fold bin threadIdx.x's copies into copy 0
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) t += sh.hist[threadIdx.x * kHistCopies + c];
    sh.hist[threadIdx.x * kHistCopies] = t;
  }
  __syncthreads();
  if (threadIdx.x < 64) sel_pick_bin(sh, shift, dmask);
  __syncthreads();
}

// The passes over slots: code_at(i) gives the code of the i-th candidate slot
// of this thread (slot count `slots`, valid(i)).  kBatch slots at a time: for
// codes read from memory (kBatch 8) their loads are all issued before the
// first is used, one round trip per batch; codes in registers or LDS take
// kBatch 1.
template <int kBatch = 1, typename CodeAt, typename Valid>
__device__ inline void sel_passes(SelCore& sh, int slots, CodeAt&& code_at, Valid&& valid) {
  int start = sh.start;
  while (!sh.done && start >= 0) {
    int shift;
    uint32_t dmask;
    sel_pass_begin(sh, start, &shift, &dmask);
    const uint64_t prefix = sh.prefix, mask = sh.mask;
    const uint32_t copy = threadIdx.x & (kHistCopies - 1);
    for (int i0 = 0; i0 < slots; i0 += kBatch) {
      uint64_t c[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        ok[k] = i0 + k < slots && valid(i0 + k);
        c[k] = ok[k] ? code_at(i0 + k) : 0ull;
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (ok[k] && (c[k] & mask) == prefix)
          atomicAdd(&sh.hist[((uint32_t(c[k] >> shift) & dmask) * kHistCopies) | copy], 1u);
    }
    sel_pass_end(sh, shift, dmask);
    start = shift - 1;
  }
}

// The same passes with visit(count) calling count(c) once for every candidate
// code c of this thread (codes streamed from memory by the caller's loads).
template <typename Visit>
__device__ inline void sel_passes_visit(SelCore& sh, Visit&& visit) {
  int start = sh.start;
  while (!sh.done && start >= 0) {
    int shift;
    uint32_t dmask;
    sel_pass_begin(sh, start, &shift, &dmask);
    const uint64_t prefix = sh.prefix, mask = sh.mask;
    const uint32_t copy = threadIdx.x & (kHistCopies - 1);
    visit([&](uint64_t c) {
      if ((c & mask) == prefix)
        atomicAdd(&sh.hist[((uint32_t(c >> shift) & dmask) * kHistCopies) | copy], 1u);
    });
    sel_pass_end(sh, shift, dmask);
    start = shift - 1;
  }
}

// Selection over codes in global memory (keys[j], j < n): the common prefix
// from (o, an), the radix passes, then the kept indices in ascending order.
template <int kThr = kSelThreads>
__device__ inline void select_global(const Args& a, const HeadUnit& u, const uint64_t* keys,
                                     uint64_t o, uint64_t an, SelCore& sh) {
  const int n = u.nu, tid = threadIdx.x;
  if (tid == 0) sel_init(sh, o, an, n, u.budget);
  __syncthreads();
  const int slots = (n + kThr - 1) / kThr;
  sel_passes<8>(sh, slots, [&](int i) { return keys[tid + kThr * i]; },
             [&](int i) { return tid + kThr * i < n; });
  if (!sh.done) {
    // Unreachable with consistent inputs; report and keep the oldest tokens.
    if (tid == 0) raise_status(a, kStatusBadItem);
    for (int j = tid; j < u.budget; j += kThr) u.keep[j] = j;
    return;
  }
  const uint64_t prefix = sh.prefix, mask = sh.mask;
  const int need = sh.need;
  const bool ties = sh.eq != need;   // only possible with all 64 bits fixed
  if (tid == 0) sh.cut = 0;
  __syncthreads();
  if (ties) {
    // Among codes equal to the threshold keep the `need` largest indices:
    // scan rounds from the end and find the index where the count reaches need.
    int seen = 0;
    for (int r = slots - 1; r >= 0; --r) {
      const int j = r * kThr + tid;
      const bool eq = j < n && (keys[j] & mask) == prefix;
      int tot;
      const int below = block_rank<kThr>(eq, sh.cnt, &tot);
      const int above = tot - below - (eq ? 1 : 0);   // ties at larger j in this round
      if (eq && seen + above + 1 == need) sh.cut = j;
      seen += tot;
      if (seen >= need) break;
    }
    __syncthreads();
  }
  const int cut = sh.cut;
  write_ascending<kThr>(n, u.budget, u.keep, sh.round_cnt, &sh.group_total, [&](int j) {
    const uint64_t top = keys[j] & mask;
    return top > prefix || (top == prefix && (!ties || j >= cut));
  });
}

__global__ __launch_bounds__(kSelThreads) void topb_select_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid || u.keep == nullptr) return;
  const int n = u.nu;
  if (u.budget >= n) {
    for (int j = threadIdx.x; j < n; j += kSelThreads) u.keep[j] = j;
    return;
  }
  __shared__ SelCore sh;
  uint64_t o = 0, an = ~0ull;
  if (threadIdx.x == 0) {
    const int n_chunks = (n + kKeysPerBlock - 1) / kKeysPerBlock;
    const uint64_t* sp = a.selp + size_t(hu) * g.n_kc * 2;
    for (int c = 0; c < n_chunks; ++c) { o |= sp[2 * c]; an &= sp[2 * c + 1]; }
  }
  select_global(a, u, a.keys + size_t(hu) * g.max_tokens, o, an, sh);
}

// Keys and selection in one workgroup per head unit, for n <= kFusedMaxTokens.
// Lane l owns tokens l + 1024 i (i < kFusedPer).
//
// The order of the keys ln(u)/w equals the reverse order of
// s = log2(-ln u) - log2(w), which fp32 estimates within 1e-4 (estimate_code).
// A radix select on 32-bit codes of -s, held in registers, finds the B-th
// largest estimate; tokens whose estimate lies more than kBand from it are
// provably on their side of the exact threshold (kBand >= 2 x the estimate
// error, strictly, so no tie crosses it), and only the tokens inside the band
// get the exact fp64 key of reservoir_keys, which decides among them.  The
// result equals selecting on the exact keys.  The -inf class (w <= 0) and the
// +inf class (forced slots) are exact in both.  Fallback (key export
// requested, or more than kBandCap band tokens): exact keys of every token
// into the workspace and the global-memory selection of topb_select.
constexpr int kBandCap = 2048;
constexpr float kBand = 0x1p-9f;
constexpr float kLn2f = 0.693147180559945309f;

struct SelShared {
  SelCore core;
  float coef[kMaxCoef];
  int n_band, n_above;
  uint32_t cb;
  uint32_t band_idx[kBandCap];
  uint64_t band_code[kBandCap];
  uint32_t chosen[kFusedMaxTokens / 32];
  int round_cnt[kFusedPer * kSelWaves];
};

// (All loads are issued before the first use, so one memory round trip
// serves the direct score and every walk row.)
__device__ __attribute__((always_inline)) inline float token_weight(
    const Args& a, const float* s_coef, const ScoreRows& sr, float ramp, int j) {
  if (a.g.walk > kMaxWalk) return deep_weight(a, s_coef, sr.a, sr.p, ramp, j);
  float pv[kMaxWalk];
#pragma unroll
  for (int t = 0; t < kMaxWalk; ++t) pv[t] = t < a.g.walk ? sr.p[t * sr.rs + size_t(j) * sr.ts] : 0.f;
  return combine_weight(a, s_coef, sr.a[size_t(j) * sr.ts], pv, j, ramp);
}

// Weight of token j of this head unit (given weights, or a + lambda c~ + ramp).
struct WeightSrc {
  const float* w_in;   // [h_kv, n] row of this head, or nullptr
  ScoreRows sr;
  float ramp;
  __device__ __attribute__((always_inline)) float operator()(const Args& a, const float* s_coef,
                                                             int j) const {
    return w_in != nullptr ? w_in[j] : token_weight(a, s_coef, sr, ramp, j);
  }
};

// Order-preserving 32-bit code of a float (-0 folded into +0).
__device__ inline uint32_t f32_code(float x) {
  const uint32_t b = __float_as_uint(x + 0.f);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}
__device__ inline float f32_decode(uint32_t c) {
  return __uint_as_float((c >> 31) ? (c & 0x7FFFFFFFu) : ~c);
}

// Estimate code of the key ln(u)/w: 0 for w <= 0 (key -inf), ~0 for a forced
// slot (+inf), else the code of -s.  With u = m 2^-53 (m = k53 + 1) and
// x = 1 - u = (2^53 - m) 2^-53 (both exact in 53 bits), E = -ln u is taken in
// the form E = x * ln(uf) / (uf - 1) with uf = u rounded to fp32 (Goldberg's
// log1p identity: ln(w)/(w - 1) varies slowly, so the rounding of uf costs a
// relative 2^-24 at most, for every u).  uf - 1 is exact for uf >= 1/2 and
// within an ulp below; v_log_f32 is within one ulp of its output (measured on
// gfx950 down to inputs 2^-24 below 1), so E carries a relative error of a few
// 2^-24.  uf = 1 (x < 2^-25) gives E = x, whose neglected x^2/2 is below 2^-26
// relative.  Then s = (eE - ew) + log2(mE / mw) from the exact binary
// exponents and mantissas of E and w (subnormal w included).  |error of s| <
// 5e-5, twenty times inside kBand.  One formula for every u keeps the
// wavefront on one path.
// E = -ln u of the uniform from words (x0, x1), as above; exactly 0 for u = 1.
__device__ inline float neg_log_u(uint32_t x0, uint32_t x1) {
  const uint64_t m = (((uint64_t(x0) << 32) | uint64_t(x1)) >> 11) + 1;
  const uint64_t d = (1ull << 53) - m;
  const float uf = (float(uint32_t(m >> 21)) * 0x1p21f + float(uint32_t(m) & 0x1FFFFFu)) * 0x1p-53f;
  const float x = (float(uint32_t(d >> 21)) * 0x1p21f + float(uint32_t(d) & 0x1FFFFFu)) * 0x1p-53f;
  const float r = -__builtin_amdgcn_logf(uf) * kLn2f * __builtin_amdgcn_rcpf(1.f - uf);
  return (uf == 1.f || x == 0.f) ? x : x * r;   // u = 1: m = 2^53 does not fit uf's formula
}

// Code of -s, s = log2(X) - log2(w) for a key -X/w (X > 0; X = 0, key 0, is
// the largest finite key).
__device__ inline uint32_t order_code(float x, float w) {
  if (!(x > 0.f)) return f32_code(INFINITY);
  int ee, ew;
  const float me = __builtin_frexpf(x, &ee);
  const float mw = __builtin_frexpf(w, &ew);
  const float sv = float(ee - ew) + __builtin_amdgcn_logf(me * __builtin_amdgcn_rcpf(mw));
  return min(max(f32_code(-sv), 1u), 0xFFFFFFFEu);
}

__device__ inline uint32_t estimate_code(uint32_t x0, uint32_t x1, float w, bool forced) {
  if (forced) return 0xFFFFFFFFu;
  if (!(w > 0.f)) return 0u;
  return order_code(neg_log_u(x0, x1), w);
}

// n >= 2 draws (section 2.3 Eq. 6): with E_i = -ln u_i (draws 2c, 2c + 1 from
// Philox block c, key word 1 bumped by c, as token_key takes them) the key is
// ln pi = -E_min / w + L, L = ln(sum_i exp(-(E_i - E_min) / w)) - ln n in
// [-ln n, 0], so -key = (E_min + |L| w) / w with no cancellation: the fp32
// estimate of log2(E_min + |L| w) - log2(w) carries the error of E_min
// (above) plus a few ulp of the sum and log, well inside kBand.
__device__ inline uint32_t estimate_code_avg(const Args& a, const HeadUnit& u, int j, float w,
                                             bool forced, uint32_t k0, uint32_t k1) {
  if (forced) return 0xFFFFFFFFu;
  if (!(w > 0.f)) return 0u;
  const float c2 = 1.4426950408889634f / w;   // log2(e) / w
  float emin = INFINITY, sum = 0.f;
  for (int c = 0; 2 * c < a.n_avg; ++c) {
    const uint4 x = philox4x32_10(make_uint4(uint32_t(j), u.unit_id, u.layer, a.step), k0,
                                  k1 + uint32_t(c));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (2 * c + h < a.n_avg) {
        const float e = h == 0 ? neg_log_u(x.x, x.y) : neg_log_u(x.z, x.w);
        if (e < emin) {
          sum = emin == INFINITY ? 1.f : sum * __builtin_amdgcn_exp2f((e - emin) * c2) + 1.f;
          emin = e;
        } else {
          sum += __builtin_amdgcn_exp2f((emin - e) * c2);
        }
      }
    }
  }
  const float abs_l = __builtin_amdgcn_logf(float(a.n_avg) * __builtin_amdgcn_rcpf(sum)) * kLn2f;
  return order_code(emin + fmaxf(abs_l, 0.f) * w, w);
}

// Exact fp64 key of token j (reservoir_keys' definition).
__device__ __attribute__((always_inline)) inline double exact_key(const Args& a, const HeadUnit& u,
                                                                  int j, float w, uint32_t k0,
                                                                  uint32_t k1) {
  return token_key(a, u, j, w, k0, k1);
}

// f(integral_constant<int, i>) for i = B .. E-1, expanded at compile time, so
// that register arrays indexed by i stay in registers where the body is too
// large for the loop unroller.
template <int B, int E, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Whether a head unit's selection runs on estimate codes (no key export, a
// keep array, and something to drop).
// (With allocated per-head budgets the estimate pass runs before the budgets
// exist, so every head unit gets its codes.)
__device__ inline bool uses_estimate(const Args& a, const HeadUnit& u) {
  return a.keys_out == nullptr && u.keep != nullptr &&
         (u.budget < u.nu || a.g.head_alloc == NX_HEADS_ALLOC);
}

// Estimate codes of kKeysPerBlock tokens of one head unit (many workgroups
// per head unit, like reservoir_keys), stored as uint32 at the start of the
// head unit's key array; also the non-finite check and the weight export.
// kW >= 0: the call's walk depth at compile time (weights computed in rows of
// a multiple of 4 floats).
template <int kW>
__global__ __launch_bounds__(kKeysThreads) void estimate_keys_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.y, chunk = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int j0 = chunk * kKeysPerBlock;
  if (j0 >= u.nu) return;
  __shared__ float s_coef[kMaxCoef];
  if (a.coef_in_keys) {
    // Small calls: the walk coefficients are formed here (no walk_coef
    // launch), and chunk 0 leaves them for the select kernel.
    if (threadIdx.x < 64) walk_coef_unit(a, u, hu, threadIdx.x, s_coef);
    __syncthreads();
    if (chunk == 0 && threadIdx.x < kMaxWalk) a.coef[size_t(hu) * kMaxCoef + threadIdx.x] = s_coef[threadIdx.x];
  } else {
    if (threadIdx.x < kMaxCoef)
      s_coef[threadIdx.x] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxCoef + threadIdx.x] : 0.f;
    __syncthreads();
  }
  const int n = u.nu;
  const size_t ext = size_t(u.h) * n;
  const WeightSrc ws{a.w_in != nullptr ? a.w_in + ext : nullptr, score_rows(a, hu),
                     n > 1 ? 1.f / float(n - 1) : 0.f};
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  const bool estimate = uses_estimate(a, u);
  uint32_t* codes = reinterpret_cast<uint32_t*>(a.keys + size_t(hu) * g.max_tokens);
  constexpr int kPer = kKeysPerBlock / kKeysThreads;
  static_assert(kPer == 4, "one 16-byte vector per array and thread");
  // Computed weights in planar rows of a multiple of 4 floats: thread t takes
  // tokens j0 + 4t .. +3 with one 16-byte load per row (and one 16-byte code
  // store); otherwise tokens j0 + t + kKeysThreads i: one float at a time, or
  // for packed rows one 16-byte record (a, P_1, P_2, P_3) per token, so that
  // each load instruction reads 1 KB in one piece.
  const bool packed = kW == 3 && g.packed;
  const bool vec = !packed && (kW >= 0 || (a.w_in == nullptr && g.walk <= kMaxWalk &&
                                           (g.max_tokens & 3) == 0));
  auto tok = [&](int i) {
    return vec ? j0 + 4 * int(threadIdx.x) + i : j0 + int(threadIdx.x) + kKeysThreads * i;
  };
  float w[kPer];
  if (packed) {
    const float4* rec = reinterpret_cast<const float4*>(ws.sr.a);
    float4 r[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tok(i);
      r[i] = rec[j < n ? j : j0];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tok(i);
      float pe[kMaxWalk] = {r[i].y, r[i].z, r[i].w};
      w[i] = combine_weight<kW>(a, s_coef, r[i].x, pe, j < n ? j : j0, ws.ramp);
    }
  } else if (vec) {
    const int jv = j0 + 4 * int(threadIdx.x);
    const int jl = jv < n ? jv : j0;   // rows hold max_tokens >= n rounded up to 4 floats
    const float4 av = *reinterpret_cast<const float4*>(ws.sr.a + jl);
    const int walk = kW >= 0 ? kW : g.walk;
    float4 pv[kMaxWalk];
#pragma unroll
    for (int t = 0; t < kMaxWalk; ++t)
      pv[t] = t < walk ? *reinterpret_cast<const float4*>(ws.sr.p + t * ws.sr.rs + jl)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    const float ae[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe[kMaxWalk];
#pragma unroll
      for (int t = 0; t < kMaxWalk; ++t)
        pe[t] = e == 0 ? pv[t].x : e == 1 ? pv[t].y : e == 2 ? pv[t].z : pv[t].w;
      w[e] = combine_weight<kW>(a, s_coef, ae[e], pe, jl + e, ws.ramp);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tok(i);
      w[i] = ws(a, s_coef, j < n ? j : j0);
    }
  }
  bool nonfinite = false;
  uint32_t cv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tok(i);
    cv[i] = 0u;
    if (j < n) {
      nonfinite |= !isfinite(w[i]);
      if (u.w_out != nullptr) u.w_out[j] = w[i];
      if (estimate) {
        const bool forced = j < a.n_sink || j >= n - a.n_recent;
        if (a.n_avg == NX_TOPK) {
          // The key is w itself (appendix 8.2 limit): code of log2(w), same
          // order, within an ulp of the log, and exact keys (w) in the band.
          cv[i] = forced ? 0xFFFFFFFFu
                  : !(w[i] > 0.f) ? 0u
                  : min(max(f32_code(__builtin_amdgcn_logf(w[i])), 1u), 0xFFFFFFFEu);
        } else if (a.n_avg <= 1) {
          const uint4 x = philox4x32_10(make_uint4(uint32_t(j), u.unit_id, u.layer, a.step), k0, k1);
          cv[i] = estimate_code(x.x, x.y, w[i], forced);
        } else {
          cv[i] = estimate_code_avg(a, u, j, w[i], forced, k0, k1);
        }
      }
    }
  }
  if (estimate) {
    if (vec && tok(kPer - 1) < n) {
      *reinterpret_cast<uint4*>(codes + tok(0)) = make_uint4(cv[0], cv[1], cv[2], cv[3]);
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (tok(i) < n) codes[tok(i)] = cv[i];
    }
  }
  if (a.est_wcodes) {
    // Allocated per-head budgets: the weight codes (after the estimate codes)
    // and the item's histogram, as in head_codes_kernel.
    __shared__ uint32_t s_hist[kAllocBins];
    for (int b = threadIdx.x; b < kAllocBins; b += kKeysThreads) s_hist[b] = 0u;
    __syncthreads();
    uint32_t* wc = codes + a.wcode_off;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tok(i);
      if (j < n) {
        const uint32_t c = (w[i] > 0.f && w[i] < INFINITY) ? __float_as_uint(w[i]) : 0u;
        wc[j] = c;
        atomicAdd(&s_hist[c >> kAllocShift], 1u);
      }
    }
    __syncthreads();
    uint32_t* gh = a.ahist + size_t(hu / g.h_kv) * kAllocBins;
    for (int b = threadIdx.x; b < kAllocBins; b += kKeysThreads)
      if (s_hist[b] != 0u) atomicAdd(&gh[b], s_hist[b]);
  }
  if (__syncthreads_or(nonfinite) && threadIdx.x == 0) raise_status(a, kStatusNonFinite);
}

// kPer codes per lane on kThr lanes (kThr kPer >= the call's units): small
// head units take fewer register slots, and every per-slot loop and the write
// scan shrink; 512 lanes let two workgroups share a CU.
template <int kPer, int kThr = kSelThreads>
__global__ __launch_bounds__(kThr) __attribute__((amdgpu_waves_per_eu(4)))
void sample_select_kernel(const Args a) {
  static_assert(kPer >= 4 && kPer <= kFusedPer && kThr >= 256 && kThr <= kSelThreads &&
                    (kPer * (kThr / 64)) % 64 == 0,
                "slot count");
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int n = u.nu;
  __shared__ SelShared sh;
  SelCore& core = sh.core;
  const int tid = threadIdx.x;

  if (tid < kMaxCoef) sh.coef[tid] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxCoef + tid] : 0.f;
  __syncthreads();

  const size_t ext = size_t(u.h) * u.nu;   // row of head h in [h_kv, n] exports
  const WeightSrc ws{a.w_in != nullptr ? a.w_in + ext : nullptr, score_rows(a, hu),
                     n > 1 ? 1.f / float(n - 1) : 0.f};
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  const bool estimate = uses_estimate(a, u);
  if (u.keep != nullptr && u.budget >= n && a.keys_out == nullptr) {
    for (int j = tid; j < n; j += kThr) u.keep[j] = j;
    return;
  }
  // This lane's estimate codes (written by estimate_keys_kernel).
  uint32_t code[kPer];
  if (estimate) {
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(a.keys + size_t(hu) * g.max_tokens);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tid + kThr * i;
      code[i] = j < n ? codes[j] : 0u;
    }
  }

  bool fallback = !estimate;
  uint32_t lo = 0, hi = 0;
  int need2 = 0, m = 0;
  if (estimate) {
    // Radix select on the estimate codes.
    uint32_t v_or = 0, v_and = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (tid + kThr * i < n) { v_or |= code[i]; v_and &= code[i]; }
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) {
      v_or |= uint32_t(__shfl_xor(int(v_or), mm, 64));
      v_and &= uint32_t(__shfl_xor(int(v_and), mm, 64));
    }
    if ((tid & 63) == 0) { core.red_or[tid >> 6] = v_or; core.red_and[tid >> 6] = v_and; }
    __syncthreads();
    if (tid == 0) {
      uint64_t o = 0, an = 0xFFFFFFFFull;
      for (int w = 0; w < (kThr / 64); ++w) { o |= core.red_or[w]; an &= core.red_and[w]; }
      // The codes enter the 64-bit passes with their upper 32 bits set.
      sel_init(core, o | 0xFFFFFFFF00000000ull, an | 0xFFFFFFFF00000000ull, n, u.budget);
      sh.n_band = 0;
      sh.n_above = 0;
      sh.cb = 0xFFFFFFFFu;
    }
    __syncthreads();
    sel_passes(core, kPer, [&](int i) { return uint64_t(code[i]) | 0xFFFFFFFF00000000ull; },
               [&](int i) { return tid + kThr * i < n; });
    if (!core.done) {
      if (tid == 0) raise_status(a, kStatusBadItem);
      for (int j = tid; j < u.budget; j += kThr) u.keep[j] = j;
      return;
    }
    // The B-th largest estimate is the smallest code of the boundary bin
    // (prefix under mask): the bin is either taken whole or fully resolved.
    {
      uint32_t mn = 0xFFFFFFFFu;
      const uint64_t prefix = core.prefix, mask = core.mask;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (tid + kThr * i < n && ((uint64_t(code[i]) | 0xFFFFFFFF00000000ull) & mask) == prefix)
          mn = min(mn, code[i]);
#pragma unroll
      for (int mm = 32; mm >= 1; mm >>= 1) mn = min(mn, uint32_t(__shfl_xor(int(mn), mm, 64)));
      if ((tid & 63) == 0) atomicMin(&sh.cb, mn);
    }
    __syncthreads();
    const uint32_t cb = sh.cb;
    if (cb == 0u || cb == 0xFFFFFFFFu) {
      // Boundary in the -inf or +inf class: the estimate codes are exact
      // there, so the band is just the boundary class, decided by index.
      lo = hi = cb;
    } else {
      const float v = f32_decode(cb);   // -s of the B-th largest estimate
      lo = min(max(f32_code(v - kBand), 1u), 0xFFFFFFFEu);
      hi = min(max(f32_code(v + kBand), 1u), 0xFFFFFFFEu);
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tid + kThr * i;
      if (j < n) {
        if (code[i] > hi) {
          ++above;
        } else if (code[i] >= lo) {
          const int pos = atomicAdd(&sh.n_band, 1);
          if (pos < kBandCap) sh.band_idx[pos] = uint32_t(j);
        }
      }
    }
    for (int c = tid; c < kPer * kThr / 32; c += kThr) sh.chosen[c] = 0;
    atomicAdd(&sh.n_above, above);
    __syncthreads();
    m = sh.n_band;
    need2 = u.budget - sh.n_above;
    fallback = m > kBandCap || need2 < 1 || need2 > m;
  }

  if (fallback) {
    // Exact keys of every token into the workspace, then the global selection.
    uint64_t* keys = a.keys + size_t(hu) * g.max_tokens;
    uint64_t o = 0, an = ~0ull;
    for (int j = tid; j < n; j += kThr) {
      const double key = exact_key(a, u, j, ws(a, sh.coef, j), k0, k1);
      if (a.keys_out != nullptr) a.keys_out[ext + j] = key;
      const uint64_t c = key_code(key);
      keys[j] = c;
      o |= c;
      an &= c;
    }
    if (u.keep == nullptr) return;
    if (u.budget >= n) {
      for (int j = tid; j < n; j += kThr) u.keep[j] = j;
      return;
    }
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) {
      o |= __shfl_xor(o, mm, 64);
      an &= __shfl_xor(an, mm, 64);
    }
    if ((tid & 63) == 0) { core.red_or[tid >> 6] = o; core.red_and[tid >> 6] = an; }
    __syncthreads();
    uint64_t ob = 0, anb = ~0ull;
    for (int w = 0; w < (kThr / 64); ++w) { ob |= core.red_or[w]; anb &= core.red_and[w]; }
    __syncthreads();
    select_global<kThr>(a, u, keys, ob, anb, core);
    return;
  }

  // Exact keys of the band, one list entry per lane, then the exact order
  // inside the band ((code, index) descending): the first need2 win.
  for (int t = tid; t < m; t += kThr) {
    const int j = int(sh.band_idx[t]);
    sh.band_code[t] = key_code(exact_key(a, u, j, ws(a, sh.coef, j), k0, k1));
  }
  __syncthreads();
  for (int t = tid; t < m; t += kThr) {
    const uint64_t ct = sh.band_code[t];
    const uint32_t it = sh.band_idx[t];
    int rank = 0;
    for (int q = 0; q < m; ++q) {
      const uint64_t cq = sh.band_code[q];
      rank += (cq > ct || (cq == ct && sh.band_idx[q] > it)) ? 1 : 0;
    }
    if (rank < need2) atomicOr(&sh.chosen[it >> 5], 1u << (it & 31));
  }
  __syncthreads();
  // Ascending write in one pass: bit r of kmask keeps token r * 1024 + tid;
  // per (round, wave) counts, one exclusive scan over them in token order.
  uint32_t kmask = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int j = r * kThr + tid;
    if (j < n && (code[r] > hi || ((sh.chosen[j >> 5] >> (j & 31)) & 1u))) kmask |= 1u << r;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below_lane = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const uint64_t bal = __ballot((kmask >> r) & 1u);
    if (lane == 0) sh.round_cnt[r * (kThr / 64) + wave] = __popcll(bal);
  }
  __syncthreads();
  if (tid < 64) {
    // 512 counts in (round, wave) order, eight per lane: exclusive scan.
    constexpr int kPerLane = kPer * (kThr / 64) / 64;
    int loc[kPerLane], sum = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) { loc[q] = sum; sum += sh.round_cnt[lane * kPerLane + q]; }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    const int excl = incl - sum;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) sh.round_cnt[lane * kPerLane + q] = excl + loc[q];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const uint64_t bal = __ballot((kmask >> r) & 1u);
    if ((kmask >> r) & 1u) {
      const int pos = sh.round_cnt[r * (kThr / 64) + wave] + __popcll(bal & below_lane);
      if (pos < u.budget) u.keep[pos] = r * kThr + tid;
    }
  }
}

// Selection on estimate codes for head units of more than kFusedMaxTokens
// units (up to kWideMaxTokens): the radix select, band and exact keys of
// sample_select_kernel, with the 32-bit codes read from the head unit's key
// array on every pass instead of held in registers.  The band argument does
// not depend on n, so the kept set again equals the selection on exact keys.
// f(j, code) for every token j < n of this thread: four consecutive codes per
// 16-byte load (the key array is 16-byte aligned and holds at least
// ceil(n / 4) * 4 codes), eight loads (32 codes per lane, 128 KB per
// workgroup) in flight before the first use.
template <typename F>
__device__ __forceinline__ void for_codes(const uint32_t* codes, int n, F&& f) {
  constexpr int kLoads = 8;
  const uint4* c4 = reinterpret_cast<const uint4*>(codes);
  const int n4 = (n + 3) >> 2;
  for (int q0 = int(threadIdx.x); q0 < n4; q0 += kSelThreads * kLoads) {
    uint4 c[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int q = q0 + kSelThreads * k;
      c[k] = q < n4 ? c4[q] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int j = 4 * (q0 + kSelThreads * k);
      if (j < n) f(j, c[k].x);
      if (j + 1 < n) f(j + 1, c[k].y);
      if (j + 2 < n) f(j + 2, c[k].z);
      if (j + 3 < n) f(j + 3, c[k].w);
    }
  }
}

struct WideShared {
  SelCore core;
  float coef[kMaxCoef];
  int n_band, n_above;
  uint32_t cb;
  uint32_t band_idx[kBandCap];
  uint64_t band_code[kBandCap];
  uint32_t chosen[kWideMaxTokens / 32];
};

__global__ __launch_bounds__(kSelThreads) void sample_select_wide_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int n = u.nu;
  __shared__ WideShared sh;
  SelCore& core = sh.core;
  const int tid = threadIdx.x;
  if (tid < kMaxCoef) sh.coef[tid] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxCoef + tid] : 0.f;
  __syncthreads();
  const size_t ext = size_t(u.h) * u.nu;
  const WeightSrc ws{a.w_in != nullptr ? a.w_in + ext : nullptr, score_rows(a, hu),
                     n > 1 ? 1.f / float(n - 1) : 0.f};
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  if (u.keep != nullptr && u.budget >= n && a.keys_out == nullptr) {
    for (int j = tid; j < n; j += kSelThreads) u.keep[j] = j;
    return;
  }
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(a.keys + size_t(hu) * g.max_tokens);
  bool fallback = !uses_estimate(a, u) || n > kWideMaxTokens;
  uint32_t hi = 0;
  int need2 = 0, m = 0;
  if (!fallback) {
    uint32_t v_or = 0, v_and = 0xFFFFFFFFu;
    for_codes(codes, n, [&](int, uint32_t c) { v_or |= c; v_and &= c; });
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) {
      v_or |= uint32_t(__shfl_xor(int(v_or), mm, 64));
      v_and &= uint32_t(__shfl_xor(int(v_and), mm, 64));
    }
    if ((tid & 63) == 0) { core.red_or[tid >> 6] = v_or; core.red_and[tid >> 6] = v_and; }
    __syncthreads();
    if (tid == 0) {
      uint64_t o = 0, an = 0xFFFFFFFFull;
      for (int w = 0; w < kSelWaves; ++w) { o |= core.red_or[w]; an &= core.red_and[w]; }
      sel_init(core, o | 0xFFFFFFFF00000000ull, an | 0xFFFFFFFF00000000ull, n, u.budget);
      sh.n_band = 0;
      sh.n_above = 0;
      sh.cb = 0xFFFFFFFFu;
    }
    __syncthreads();
    sel_passes_visit(core, [&](auto&& count) {
      for_codes(codes, n, [&](int, uint32_t c) { count(uint64_t(c) | 0xFFFFFFFF00000000ull); });
    });
    if (!core.done) {
      if (tid == 0) raise_status(a, kStatusBadItem);
      for (int j = tid; j < u.budget; j += kSelThreads) u.keep[j] = j;
      return;
    }
    // The B-th largest estimate: the smallest code of the boundary bin.
    {
      uint32_t mn = 0xFFFFFFFFu;
      const uint64_t prefix = core.prefix, mask = core.mask;
      for_codes(codes, n, [&](int, uint32_t c) {
        if (((uint64_t(c) | 0xFFFFFFFF00000000ull) & mask) == prefix) mn = min(mn, c);
      });
#pragma unroll
      for (int mm = 32; mm >= 1; mm >>= 1) mn = min(mn, uint32_t(__shfl_xor(int(mn), mm, 64)));
      if ((tid & 63) == 0) atomicMin(&sh.cb, mn);
    }
    __syncthreads();
    const uint32_t cb = sh.cb;
    uint32_t lo;
    if (cb == 0u || cb == 0xFFFFFFFFu) {
      lo = hi = cb;   // boundary in the -inf or +inf class: exact there, decided by index
    } else {
      const float v = f32_decode(cb);
      lo = min(max(f32_code(v - kBand), 1u), 0xFFFFFFFEu);
      hi = min(max(f32_code(v + kBand), 1u), 0xFFFFFFFEu);
    }
    int above = 0;
    for_codes(codes, n, [&](int j, uint32_t c) {
      if (c > hi) {
        ++above;
      } else if (c >= lo) {
        const int pos = atomicAdd(&sh.n_band, 1);
        if (pos < kBandCap) sh.band_idx[pos] = uint32_t(j);
      }
    });
    for (int c = tid; c < (n + 31) / 32; c += kSelThreads) sh.chosen[c] = 0;
    atomicAdd(&sh.n_above, above);
    __syncthreads();
    m = sh.n_band;
    need2 = u.budget - sh.n_above;
    fallback = m > kBandCap || need2 < 1 || need2 > m;
  }

  if (fallback) {
    // Exact keys of every token (over the codes, all read by now), then the
    // global-memory selection.
    __syncthreads();
    uint64_t* keys = a.keys + size_t(hu) * g.max_tokens;
    uint64_t o = 0, an = ~0ull;
    for (int j = tid; j < n; j += kSelThreads) {
      const double key = exact_key(a, u, j, ws(a, sh.coef, j), k0, k1);
      if (a.keys_out != nullptr) a.keys_out[ext + j] = key;
      const uint64_t c = key_code(key);
      keys[j] = c;
      o |= c;
      an &= c;
    }
    if (u.keep == nullptr) return;
    if (u.budget >= n) {
      for (int j = tid; j < n; j += kSelThreads) u.keep[j] = j;
      return;
    }
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) {
      o |= __shfl_xor(o, mm, 64);
      an &= __shfl_xor(an, mm, 64);
    }
    if ((tid & 63) == 0) { core.red_or[tid >> 6] = o; core.red_and[tid >> 6] = an; }
    __syncthreads();
    uint64_t ob = 0, anb = ~0ull;
    for (int w = 0; w < kSelWaves; ++w) { ob |= core.red_or[w]; anb &= core.red_and[w]; }
    __syncthreads();
    select_global(a, u, keys, ob, anb, core);
    return;
  }

  // Exact keys of the band; the first need2 in ((code, index) descending) win.
  for (int t = tid; t < m; t += kSelThreads) {
    const int j = int(sh.band_idx[t]);
    sh.band_code[t] = key_code(exact_key(a, u, j, ws(a, sh.coef, j), k0, k1));
  }
  __syncthreads();
  for (int t = tid; t < m; t += kSelThreads) {
    const uint64_t ct = sh.band_code[t];
    const uint32_t it = sh.band_idx[t];
    int rank = 0;
    for (int q = 0; q < m; ++q) {
      const uint64_t cq = sh.band_code[q];
      rank += (cq > ct || (cq == ct && sh.band_idx[q] > it)) ? 1 : 0;
    }
    if (rank < need2) atomicOr(&sh.chosen[it >> 5], 1u << (it & 31));
  }
  __syncthreads();
  // Ascending write (four tokens per lane, eight rounds per group).
  write_ascending4(codes, n, u.budget, u.keep, core.round_cnt, &core.group_total,
                   [&](int j, uint32_t c) { return c > hi || ((sh.chosen[j >> 5] >> (j & 31)) & 1u); });
}

}  // namespace

hipError_t launch_walk_coef(const Args& a, hipStream_t s) {
  if (a.g.deep) {
    hipLaunchKernelGGL(gram_deep_kernel, dim3(a.g.n_gc, a.g.n_hu), dim3(256), 0, s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(walk_coef_deep_kernel, dim3(a.g.n_hu), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(walk_coef_kernel, dim3(a.g.n_hu), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_reservoir_keys(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(reservoir_keys_kernel, dim3(a.g.n_kc, a.g.n_hu), dim3(kKeysThreads), 0, s, a);
  return hipGetLastError();
}

// ---- per-head budgets ([Nexus] appendix 10) ----------------------------
//
// NX_HEADS_ALLOC: an item's heads share the layer budget H * Bbar; each head
// keeps f + c_h units, c_h = its share of the H * (Bbar - f) largest weights
// over all heads of the item (the head-adaptive allocation of the cited
// Ada-KV), capped by the capacity and the head's units.

// Weight codes of one head unit's units for the allocation: the bits of w
// for finite w > 0 (positive floats order as their bit patterns), else 0;
// uint32 at the start of the head unit's key array (this call's keys are
// written there only afterwards).  Each workgroup also adds its codes to the
// item's histogram of code bits 30..19 (LDS first, then one global atomic
// per non-empty bin).
__global__ __launch_bounds__(kKeysThreads) void head_codes_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.y, chunk = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int j0 = chunk * kKeysPerBlock;
  if (j0 >= u.nu) return;
  __shared__ float s_coef[kMaxCoef];
  __shared__ uint32_t s_hist[kAllocBins];
  for (int b = threadIdx.x; b < kAllocBins; b += kKeysThreads) s_hist[b] = 0u;
  if (threadIdx.x < kMaxCoef)
    s_coef[threadIdx.x] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxCoef + threadIdx.x] : 0.f;
  __syncthreads();
  const int n = u.nu;
  const WeightSrc ws{a.w_in != nullptr ? a.w_in + size_t(u.h) * n : nullptr,
                     score_rows(a, hu), n > 1 ? 1.f / float(n - 1) : 0.f};
  uint32_t* codes = reinterpret_cast<uint32_t*>(a.keys + size_t(hu) * g.max_tokens);
  constexpr int kPer = kKeysPerBlock / kKeysThreads;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + threadIdx.x + kKeysThreads * i;
    if (j < n) {
      const float w = ws(a, s_coef, j);
      const uint32_t c = (w > 0.f && w < INFINITY) ? __float_as_uint(w) : 0u;
      codes[j] = c;
      atomicAdd(&s_hist[c >> kAllocShift], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = a.ahist + size_t(hu / g.h_kv) * kAllocBins;
  for (int b = threadIdx.x; b < kAllocBins; b += kKeysThreads)
    if (s_hist[b] != 0u) atomicAdd(&gh[b], s_hist[b]);
}

// Selection units of head h of an item (its resident count, per head when
// the item carries head_tokens; clamped into [0, n_tokens] so that indexing
// stays inside the item's arrays even for a bad count, which head_unit
// rejects).
__device__ inline int alloc_head_units(const Args& a, const nx_unit& it, int h) {
  int n = it.head_tokens != nullptr ? it.head_tokens[h] : it.n_tokens;
  n = min(max(n, 0), it.n_tokens);
  return (n + a.g.block - 1) / a.g.block;
}

// Allocation sizes of one item: Bbar = min(budget, units of its largest
// head), f = min(floor, Bbar), k = H (Bbar - f) codes to take out of all the
// heads' total units.
struct AllocSizes {
  int f, k, total;
};
__device__ inline AllocSizes alloc_sizes(const Args& a, const nx_unit& it) {
  int numax = 0, total = 0;
  for (int h = 0; h < a.g.h_kv; ++h) {
    const int nu = alloc_head_units(a, it, h);
    numax = max(numax, nu);
    total += nu;   // < 2^31: H * n_tokens is checked on the host
  }
  const int bbar = min(it.budget, numax);
  const int f = min(a.head_floor, bbar);
  return {f, a.g.h_kv * (bbar - f), total};
}

// The bin of the item's histogram (in LDS) that holds the k-th largest code.
// Thread t owns bins 4t .. 4t+3; suffix sums over the threads, highest bins
// first.  Sets *s_bstar (-1 if the histogram holds fewer than k codes),
// *s_krem (codes still needed from that bin) and *s_above (codes above it).
__device__ inline void alloc_boundary(const uint32_t* s_hist, int k, uint32_t* s_wsum,
                                      int* s_bstar, int* s_krem, int* s_above) {
  static_assert(kAllocBins == 4 * kSelThreads, "bin split");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) *s_bstar = -1;
  const uint32_t h0 = s_hist[4 * tid], h1 = s_hist[4 * tid + 1], h2 = s_hist[4 * tid + 2],
                 h3 = s_hist[4 * tid + 3];
  const uint32_t own = h0 + h1 + h2 + h3;
  uint32_t suf = own;   // inclusive suffix sum inside the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += v;
  }
  if (lane == 0) s_wsum[wave] = suf;
  __syncthreads();
  uint32_t higher = suf - own;
  for (int w = wave + 1; w < kSelWaves; ++w) higher += s_wsum[w];
  const uint32_t kk = uint32_t(k);
  if (higher < kk && kk <= higher + own) {
    const uint32_t c3 = higher + h3, c2 = c3 + h2, c1 = c2 + h1;
    const int b = kk <= c3 ? 3 : kk <= c2 ? 2 : kk <= c1 ? 1 : 0;
    const uint32_t acc = b == 3 ? higher : b == 2 ? c3 : b == 1 ? c2 : c1;
    *s_bstar = 4 * tid + b;
    *s_krem = int(kk - acc);
    *s_above = int(acc);
  }
  __syncthreads();
}

// One workgroup per head unit (NX_HEADS_ALLOC): from the item's histogram,
// the boundary bin b*; then one pass over this head's codes counts those
// above b* and copies those in b* (low 19 bits and the head) to the head
// unit's candidate area.  Writes (count above, candidate count); a count over
// kAllocCand means the candidates did not fit.
__global__ __launch_bounds__(kSelThreads) void head_count_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x, H = g.h_kv, tid = threadIdx.x, lane = tid & 63;
  const int item = hu / H, h = hu - item * H;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const nx_unit it = load_item(a, item);
  const int nu = u.nu;
  const AllocSizes z = alloc_sizes(a, it);
  if (!(z.k > 0 && z.k < z.total)) return;
  __shared__ uint32_t s_hist[kAllocBins];
  __shared__ uint32_t s_wsum[kSelWaves];
  __shared__ int s_bstar, s_krem, s_above, s_n, s_gt;
  const uint32_t* gh = a.ahist + size_t(item) * kAllocBins;
  for (int b = tid; b < kAllocBins; b += kSelThreads) s_hist[b] = gh[b];
  if (tid == 0) {
    s_n = 0;
    s_gt = 0;
  }
  __syncthreads();
  alloc_boundary(s_hist, z.k, s_wsum, &s_bstar, &s_krem, &s_above);
  const int bstar = s_bstar;
  int* cnt = a.acnt + 2 * size_t(hu);
  if (bstar < 0) {   // the histogram does not hold the item's codes
    if (tid == 0) {
      cnt[0] = -1;
      cnt[1] = -1;
    }
    return;
  }
  const uint32_t* ch = reinterpret_cast<const uint32_t*>(a.keys + size_t(hu) * g.max_tokens) + a.wcode_off;
  uint32_t* cand = a.acand + size_t(hu) * kAllocCand;
  // Codes are read as pairs (8-byte loads, 16 in flight per thread) when
  // they start on an 8-byte boundary (wcode_off even; the key array then
  // holds the pair that ends past the last code), else one by one.
  constexpr int kLoads = 16;
  const bool pairs = (a.wcode_off & 1) == 0;
  const int n2 = pairs ? (nu + 1) / 2 : nu;
  const uint2* ch2 = reinterpret_cast<const uint2*>(ch);
  int gt = 0;
  auto consider = [&](uint32_t c) {
    const int bin = int(c >> kAllocShift);
    gt += bin > bstar;
    if (bin == bstar) {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < kAllocCand) cand[slot] = (uint32_t(h) << kAllocShift) | (c & ((1u << kAllocShift) - 1u));
    }
  };
  for (int p0 = tid; p0 < n2; p0 += kSelThreads * kLoads) {
    uint2 v[kLoads];
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int pr = p0 + r * kSelThreads;
      v[r] = pr >= n2 ? make_uint2(0u, 0u) : pairs ? ch2[pr] : make_uint2(ch[pr], 0u);
    }
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int pr = p0 + r * kSelThreads;
      if (pr < n2) {
        consider(v[r].x);
        if (pairs && 2 * pr + 1 < nu) consider(v[r].y);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) gt += __shfl_xor(gt, off, 64);
  if (lane == 0 && gt != 0) atomicAdd(&s_gt, gt);
  __syncthreads();
  if (tid == 0) {
    cnt[0] = s_gt;
    cnt[1] = s_n;
  }
}

// One workgroup per item: sets the heads' keep rows to -1 (the selection
// then writes the kept entries) and, for NX_HEADS_ALLOC, turns the heads'
// counts into budgets: the boundary bin again from the histogram (cleared
// here for the next call), the heads' candidates gathered into LDS, the
// radix passes of SelCore among them, the threshold class's remaining places
// to the heads in ascending order.  If the candidates overflow or the counts
// disagree with the histogram (one left over from an interrupted call), the
// radix passes run over all codes of the item instead.
__global__ __launch_bounds__(kSelThreads) void head_alloc_kernel(const Args a) {
  const Geometry& g = a.g;
  const int item = blockIdx.x, H = g.h_kv, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const nx_unit it = load_item(a, item);
  const HeadUnit u0 = head_unit(a, item * H);
  if (!u0.valid) return;
  const int cap = u0.cap;
  if (it.keep != nullptr)
    for (int64_t i = tid; i < int64_t(H) * cap; i += kSelThreads) it.keep[i] = -1;
  if (g.head_alloc != NX_HEADS_ALLOC) return;
  __shared__ SelCore sh;
  __shared__ int s_gt[NX_MAX_ALLOC_HEADS], s_eq[NX_MAX_ALLOC_HEADS], s_off[NX_MAX_ALLOC_HEADS];
  // Units of every head and their exclusive prefix (the flat code index of
  // head h starts at s_pre[h]).
  __shared__ int s_nu[NX_MAX_ALLOC_HEADS], s_pre[NX_MAX_ALLOC_HEADS + 1];
  if (tid == 0) {
    int acc = 0;
    for (int h = 0; h < H; ++h) {
      s_nu[h] = alloc_head_units(a, it, h);
      s_pre[h] = acc;
      acc += s_nu[h];
    }
    s_pre[H] = acc;
  }
  __syncthreads();
  __shared__ uint32_t s_hist[kAllocBins];
  __shared__ uint32_t s_cand[kAllocCand];
  __shared__ uint32_t s_wsum[kSelWaves];
  __shared__ int s_bstar, s_krem, s_above, s_ncand, s_fallback;
  const AllocSizes z = alloc_sizes(a, it);
  const int f = z.f, k = z.k, total = z.total;
  const uint32_t* base =
      reinterpret_cast<const uint32_t*>(a.keys + size_t(item) * H * g.max_tokens) + a.wcode_off;
  const size_t hstride = 2 * size_t(g.max_tokens);   // uint32 per head unit's key array
  const uint32_t* gh = a.ahist + size_t(item) * kAllocBins;
  for (int h = tid; h < H; h += kSelThreads) {
    s_gt[h] = 0;
    s_eq[h] = 0;
  }
  for (int b = tid; b < kAllocBins; b += kSelThreads) s_hist[b] = gh[b];
  __syncthreads();
  bool all = true;   // every code of the threshold class is taken
  int need = 0;
  if (k > 0 && k < total) {
    alloc_boundary(s_hist, k, s_wsum, &s_bstar, &s_krem, &s_above);
    if (tid == 0) {
      // The heads' counts, checked against the histogram.
      int fb = s_bstar < 0, above = 0, nc = 0;
      for (int h = 0; h < H && !fb; ++h) {
        const int* cnt = a.acnt + 2 * (size_t(item) * H + h);
        if (cnt[0] < 0 || cnt[1] < 0 || cnt[1] > kAllocCand) {
          fb = 1;
          break;
        }
        s_gt[h] = cnt[0];
        s_off[h] = nc;
        above += cnt[0];
        nc += cnt[1];
      }
      if (!fb && (nc > kAllocCand || uint32_t(nc) != s_hist[s_bstar] || above != s_above)) fb = 1;
      s_fallback = fb;
      s_ncand = fb ? 0 : nc;
    }
    __syncthreads();
    const bool fallback = s_fallback != 0;
    if (!fallback) {
      // Gather the candidates, then the s_krem-th largest low part among them.
      const int ncand = s_ncand;
      for (int h = 0; h < H; ++h) {
        const int nh = a.acnt[2 * (size_t(item) * H + h) + 1];
        const uint32_t* src = a.acand + (size_t(item) * H + h) * kAllocCand;
        for (int i = tid; i < nh; i += kSelThreads) s_cand[s_off[h] + i] = src[i];
      }
      __syncthreads();
      constexpr uint64_t kHigh = ~uint64_t((1u << kAllocShift) - 1u);
      constexpr uint32_t kLow = (1u << kAllocShift) - 1u;
      uint32_t o = 0u, an = ~0u;
      for (int i = tid; i < ncand; i += kSelThreads) {
        o |= s_cand[i] & kLow;
        an &= s_cand[i] & kLow;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        o |= __shfl_xor(o, off, 64);
        an &= __shfl_xor(an, off, 64);
      }
      if (lane == 0) {
        sh.red_or[wave] = o;
        sh.red_and[wave] = an;
      }
      __syncthreads();
      if (tid == 0) {
        uint64_t oo = 0, aa = ~0ull;
        for (int w = 0; w < kSelWaves; ++w) {
          oo |= sh.red_or[w];
          aa &= sh.red_and[w];
        }
        sel_init(sh, oo | kHigh, (aa & kLow) | kHigh, ncand, s_krem);
      }
      __syncthreads();
      const int slots = (ncand + kSelThreads - 1) / kSelThreads;
      sel_passes(sh, slots, [&](int i) { return uint64_t(s_cand[tid + kSelThreads * i] & kLow) | kHigh; },
                 [&](int i) { return tid + kSelThreads * i < ncand; });
      const uint64_t prefix = sh.prefix, mask = sh.mask;
      for (int i = tid; i < ncand; i += kSelThreads) {
        const uint64_t c = (uint64_t(s_cand[i] & kLow) | kHigh) & mask;
        const int h = int(s_cand[i] >> kAllocShift);
        if (c > prefix) atomicAdd(&s_gt[h], 1);
        else if (c == prefix) atomicAdd(&s_eq[h], 1);
      }
      __syncthreads();
      need = sh.need;
      all = sh.eq == sh.need;
    } else {
      // Radix passes over all codes of the item.
      for (int h = tid; h < H; h += kSelThreads) {
        s_gt[h] = 0;
        s_eq[h] = 0;
      }
      // Head of flat code index idx: the last h with s_pre[h] <= idx.
      auto head_of = [&](int idx) {
        int lo = 0, hi = H - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_pre[mid] <= idx) lo = mid; else hi = mid - 1;
        }
        return lo;
      };
      auto code_at = [&](int idx) -> uint64_t {
        const int h = head_of(idx);
        return uint64_t(base[size_t(h) * hstride + (idx - s_pre[h])]) | 0xFFFFFFFF00000000ull;
      };
      uint32_t o = 0u, an = ~0u;
      for (int idx = tid; idx < total; idx += kSelThreads) {
        const uint32_t c = uint32_t(code_at(idx));
        o |= c;
        an &= c;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        o |= __shfl_xor(o, off, 64);
        an &= __shfl_xor(an, off, 64);
      }
      if (lane == 0) {
        sh.red_or[wave] = o;
        sh.red_and[wave] = an;
      }
      __syncthreads();
      if (tid == 0) {
        uint64_t oo = 0, aa = ~0ull;
        for (int w = 0; w < kSelWaves; ++w) {
          oo |= sh.red_or[w];
          aa &= sh.red_and[w];
        }
        sel_init(sh, oo | 0xFFFFFFFF00000000ull, aa | 0xFFFFFFFF00000000ull, total, k);
      }
      __syncthreads();
      const int slots = (total + kSelThreads - 1) / kSelThreads;
      sel_passes<8>(sh, slots, [&](int i) { return code_at(tid + kSelThreads * i); },
                 [&](int i) { return tid + kSelThreads * i < total; });
      const uint64_t prefix = sh.prefix, mask = sh.mask;
      int cur = -1, gt = 0, eq = 0;
      for (int idx = tid; idx < total; idx += kSelThreads) {
        const int h = head_of(idx);
        if (h != cur) {
          if (cur >= 0) {
            atomicAdd(&s_gt[cur], gt);
            atomicAdd(&s_eq[cur], eq);
          }
          cur = h;
          gt = eq = 0;
        }
        const uint64_t c = code_at(idx) & mask;
        gt += c > prefix;
        eq += c == prefix;
      }
      if (cur >= 0) {
        atomicAdd(&s_gt[cur], gt);
        atomicAdd(&s_eq[cur], eq);
      }
      __syncthreads();
      need = sh.need;
      all = sh.eq == sh.need;
    }
    if (!sh.done) {   // unreachable with consistent inputs
      if (tid == 0) raise_status(a, kStatusBadItem);
      return;
    }
  }
  // Budgets.
  if (tid == 0) {
    for (int h = 0; h < H; ++h) {
      int ch;
      if (k == 0) {
        ch = 0;
      } else if (k >= total) {
        ch = s_nu[h];
      } else {
        const int take = all ? s_eq[h] : min(s_eq[h], need);
        if (!all) need -= take;
        ch = s_gt[h] + take;
      }
      const int bh = min(min(f + ch, cap), s_nu[h]);
      it.head_budget[h] = bh;
      // A budget that cannot hold the forced slots makes the head invalid for
      // the stages that follow: report it.
      if (bh < a.n_sink + a.n_recent && bh < s_nu[h]) raise_status(a, kStatusBadItem);
    }
  }
}

// Clears the per-item histograms of the allocation before a call builds them
// (their place in the workspace moves with the call's shape, so a clear left
// by an earlier call cannot be relied on).  A fill kernel, not a memset, so
// that the call stays capturable into a graph.
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = 0u;
}

hipError_t launch_clear_alloc_hist(const Args& a, hipStream_t s) {
  const int64_t n = int64_t(a.g.n_hu / a.g.h_kv) * kAllocBins;
  const int blocks = int(std::min<int64_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(clear_words_kernel, dim3(blocks), dim3(256), 0, s, a.ahist, n);
  return hipGetLastError();
}

hipError_t launch_head_budget(const Args& a, hipStream_t s) {
  if (a.g.head_alloc == NX_HEADS_ALLOC && !a.est_wcodes) {
    const hipError_t cerr = launch_clear_alloc_hist(a, s);
    if (cerr != hipSuccess) return cerr;
    hipLaunchKernelGGL(head_codes_kernel, dim3(a.g.n_kc, a.g.n_hu), dim3(kKeysThreads), 0, s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.g.head_alloc == NX_HEADS_ALLOC) {
    hipLaunchKernelGGL(head_count_kernel, dim3(a.g.n_hu), dim3(kSelThreads), 0, s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(head_alloc_kernel, dim3(a.g.n_hu / a.g.h_kv), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_estimate_keys(const Args& a, hipStream_t s) {
  if (a.est_wcodes) {   // this pass also builds the allocation histograms
    const hipError_t cerr = launch_clear_alloc_hist(a, s);
    if (cerr != hipSuccess) return cerr;
  }
  const dim3 grid(a.g.n_kc, a.g.n_hu), block(kKeysThreads);
  const bool vec = a.w_in == nullptr && a.g.walk <= kMaxWalk && (a.g.max_tokens & 3) == 0;
  switch (vec ? a.g.walk : -1) {
    case 0: hipLaunchKernelGGL(estimate_keys_kernel<0>, grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL(estimate_keys_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(estimate_keys_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(estimate_keys_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(estimate_keys_kernel<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(estimate_keys_kernel<5>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(estimate_keys_kernel<-1>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_sample_select(const Args& a, hipStream_t s) {
  const int max_units = (a.g.max_tokens + a.g.block - 1) / a.g.block;
  // Units of up to 16384 tokens: 512-lane workgroups (8, 16 or 32 codes per
  // lane), two to a CU, so that a batch of many head units overlaps their
  // latencies; up to 32768 the 1024-lane kernel holds 32 codes per lane; above
  // that the codes stay in memory.
  constexpr int kHalf = kSelThreads / 2;
  if (max_units <= 8 * kHalf)
    hipLaunchKernelGGL((sample_select_kernel<8, kHalf>), dim3(a.g.n_hu), dim3(kHalf), 0, s, a);
  else if (max_units <= 16 * kHalf)
    hipLaunchKernelGGL((sample_select_kernel<16, kHalf>), dim3(a.g.n_hu), dim3(kHalf), 0, s, a);
  else if (max_units <= kFusedPer * kHalf)
    hipLaunchKernelGGL((sample_select_kernel<kFusedPer, kHalf>), dim3(a.g.n_hu), dim3(kHalf), 0, s, a);
  else if (max_units <= kFusedMaxTokens)
    hipLaunchKernelGGL((sample_select_kernel<kFusedPer>), dim3(a.g.n_hu), dim3(kSelThreads), 0, s, a);
  else
    hipLaunchKernelGGL(sample_select_wide_kernel, dim3(a.g.n_hu), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topb_select(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(topb_select_kernel, dim3(a.g.n_hu), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace nx
