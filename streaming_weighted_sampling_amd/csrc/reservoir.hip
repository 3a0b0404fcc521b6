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
//     8-bit digits: LDS histogram of the candidates, boundary bin by a
//     wavefront suffix scan, until the boundary bin holds exactly the missing
//     count or all 64 bits are fixed (true ties: larger index wins)
//   * writes the kept indices in ascending order with ballot / popcount
//     prefix sums, 1024 tokens per round.
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
__global__ __launch_bounds__(64) void walk_coef_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int lane = threadIdx.x;
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
    for (int t = 0; t < kMaxWalk; ++t)
      a.coef[size_t(hu) * kMaxWalk + t] = (t < g.walk) ? gam[t] / norm : 0.f;
  }
}

__global__ __launch_bounds__(kKeysThreads) void reservoir_keys_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.y, chunk = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int j0 = chunk * kKeysPerBlock;
  if (j0 >= u.n) return;
  __shared__ float s_coef[kMaxWalk];
  __shared__ uint64_t s_or[kKeysThreads / 64], s_and[kKeysThreads / 64];

  if (threadIdx.x < kMaxWalk)
    s_coef[threadIdx.x] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxWalk + threadIdx.x] : 0.f;
  __syncthreads();

  const float* a_in = a.a + size_t(hu) * g.max_tokens;
  const float* p_in = a.p + size_t(hu) * g.walk * g.max_tokens;
  uint64_t* keys = a.keys + size_t(hu) * g.max_tokens;
  const size_t ext = size_t(u.h) * u.n;   // row of head h in [h_kv, n] exports
  const float ramp = u.n > 1 ? 1.f / float(u.n - 1) : 0.f;
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
    in[i] = j < u.n;
    const int jc = in[i] ? j : j0;   // a valid token for the lanes past the end
    if (a.w_in != nullptr) {
      w[i] = a.w_in[ext + jc];
    } else {
      float cj = 0.f;
#pragma unroll
      for (int t = 0; t < kMaxWalk; ++t)
        if (t < g.walk) cj = fmaf(s_coef[t], p_in[size_t(t) * g.max_tokens + jc], cj);
      w[i] = a_in[jc] + a.lambda * cj + a.eps_tie * (float(jc) * ramp);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (!in[i]) continue;
    const int j = j0 + threadIdx.x + kKeysThreads * i;
    nonfinite |= !isfinite(w[i]);
    if (a.w_out != nullptr) a.w_out[ext + j] = w[i];
    if (a.stop_after_weights) continue;
    const uint4 x = philox4x32_10(make_uint4(uint32_t(j), u.unit_id, u.layer, a.step), k0, k1);
    const double uj = philox_uniform53(x.x, x.y);
    double key = w[i] > 0.f ? log(uj) / double(w[i]) : -INFINITY;
    if (j < a.n_sink || j >= u.n - a.n_recent) key = INFINITY;
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
__device__ inline int block_rank(bool flag, int* s_cnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) s_cnt[wave] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = s_cnt[w];
    off += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + below;
}

__global__ __launch_bounds__(kSelThreads) void topb_select_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid || u.keep == nullptr) return;
  const int n = u.n;
  if (u.budget >= n) {
    for (int j = threadIdx.x; j < n; j += kSelThreads) u.keep[j] = j;
    return;
  }
  const uint64_t* keys = a.keys + size_t(hu) * g.max_tokens;
  __shared__ uint32_t s_hist[256];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ int s_need, s_eq, s_done, s_start;
  __shared__ int s_cnt[kSelWaves];
  __shared__ int s_cut;

  if (threadIdx.x == 0) {
    const int n_chunks = (n + kKeysPerBlock - 1) / kKeysPerBlock;
    const uint64_t* sp = a.selp + size_t(hu) * g.n_kc * 2;
    uint64_t o = 0, an = ~0ull;
    for (int c = 0; c < n_chunks; ++c) { o |= sp[2 * c]; an &= sp[2 * c + 1]; }
    const uint64_t diff = o ^ an;
    s_need = u.budget;
    if (diff == 0) {                       // every code equal: pure ties
      s_prefix = an;
      s_mask = ~0ull;
      s_eq = n;
      s_done = 1;
    } else {
      const int top = 63 - __clzll(diff);  // highest bit that differs
      const uint64_t above = top == 63 ? 0ull : (~0ull << (top + 1));
      s_prefix = an & above;
      s_mask = above;
      s_eq = n;
      s_done = 0;
      s_start = top;
    }
  }
  __syncthreads();

  // MSD radix passes over the unresolved bits, highest first.  At most 64
  // bits are resolved, so the loop ends after at most 8 passes even if the
  // codes were inconsistent with the OR/AND summary.
  int start = s_start;
  while (!s_done && start >= 0) {
    const int shift = start >= 7 ? start - 7 : 0;
    const int width = start - shift + 1;
    const uint32_t dmask = (1u << width) - 1u;
    for (int b = threadIdx.x; b < 256; b += kSelThreads) s_hist[b] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix, mask = s_mask;
    for (int j = threadIdx.x; j < n; j += kSelThreads) {
      const uint64_t c = keys[j];
      if ((c & mask) == prefix) atomicAdd(&s_hist[uint32_t(c >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // Lane l owns bins 4l..4l+3; suffix sums over lanes find the bin that
      // holds the need-th largest candidate.
      const int l = threadIdx.x;
      const uint32_t h0 = s_hist[4 * l], h1 = s_hist[4 * l + 1], h2 = s_hist[4 * l + 2],
                     h3 = s_hist[4 * l + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t suf = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off, 64);
        if (l + off < 64) suf += v;
      }
      const uint32_t higher = suf - own;   // candidates in bins above this lane's
      const uint32_t need = uint32_t(s_need);
      if (higher < need && need <= suf) {
        const uint32_t c3 = higher + h3, c2 = c3 + h2, c1 = c2 + h1;
        const int b = need <= c3 ? 3 : need <= c2 ? 2 : need <= c1 ? 1 : 0;
        const uint32_t acc = b == 3 ? higher : b == 2 ? c3 : b == 1 ? c2 : c1;
        const uint32_t hb = b == 3 ? h3 : b == 2 ? h2 : b == 1 ? h1 : h0;
        s_need = int(need - acc);
        s_eq = int(hb);
        s_prefix = prefix | (uint64_t(4 * l + b) << shift);
        s_mask = mask | (uint64_t(dmask) << shift);
        s_done = (hb == need - acc) || shift == 0;
      }
    }
    __syncthreads();
    start = shift - 1;
  }

  if (!s_done) {
    // Unreachable with consistent inputs; report and keep the oldest tokens.
    if (threadIdx.x == 0) raise_status(a, kStatusBadItem);
    for (int j = threadIdx.x; j < u.budget; j += kSelThreads) u.keep[j] = j;
    return;
  }
  const uint64_t prefix = s_prefix, mask = s_mask;
  const int need = s_need;
  const bool ties = s_eq != need;   // only possible with all 64 bits fixed
  if (threadIdx.x == 0) s_cut = 0;
  __syncthreads();
  if (ties) {
    // Among codes equal to the threshold keep the `need` largest indices:
    // scan rounds from the end and find the index where the count reaches need.
    int seen = 0;
    const int n_rounds = (n + kSelThreads - 1) / kSelThreads;
    for (int r = n_rounds - 1; r >= 0; --r) {
      const int j = r * kSelThreads + threadIdx.x;
      const bool eq = j < n && (keys[j] & mask) == prefix;
      int tot;
      const int below = block_rank(eq, s_cnt, &tot);
      const int above = tot - below - (eq ? 1 : 0);   // ties at larger j in this round
      if (eq && seen + above + 1 == need) s_cut = j;
      seen += tot;
      if (seen >= need) break;
    }
    __syncthreads();
  }
  const int cut = s_cut;
  int base = 0;
  const int n_rounds = (n + kSelThreads - 1) / kSelThreads;
  for (int r = 0; r < n_rounds; ++r) {
    const int j = r * kSelThreads + threadIdx.x;
    bool keep = false;
    if (j < n) {
      const uint64_t top = keys[j] & mask;
      keep = top > prefix || (top == prefix && (!ties || j >= cut));
    }
    int tot;
    const int pos = block_rank(keep, s_cnt, &tot);
    if (keep && base + pos < u.budget) u.keep[base + pos] = j;
    base += tot;
  }
}

// Keys and selection in one workgroup per head unit, for n <= kFusedMaxTokens:
// lane l computes the codes of tokens l + 1024 i (i < kFusedPer) into
// registers exactly as reservoir_keys does, and the MSD radix passes of
// topb_select then run over those registers, so the codes never go through
// memory.  Same keys, same selection rule, same output as the two kernels.
__device__ inline float token_weight(const Args& a, const float* s_coef, const float* a_in,
                                     const float* p_in, float ramp, int j) {
  float cj = 0.f;
#pragma unroll
  for (int t = 0; t < kMaxWalk; ++t)
    if (t < a.g.walk) cj = fmaf(s_coef[t], p_in[size_t(t) * a.g.max_tokens + j], cj);
  return a_in[j] + a.lambda * cj + a.eps_tie * (float(j) * ramp);
}

__global__ __launch_bounds__(kSelThreads) void sample_select_kernel(const Args a) {
  const Geometry& g = a.g;
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int n = u.n;
  __shared__ float s_coef[kMaxWalk];
  __shared__ uint32_t s_hist[256];
  __shared__ uint64_t s_prefix, s_mask;
  __shared__ int s_need, s_eq, s_done, s_start;
  __shared__ int s_cnt[kSelWaves];
  __shared__ int s_cut;
  __shared__ uint64_t s_or[kSelWaves], s_and[kSelWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (tid < kMaxWalk)
    s_coef[tid] = a.w_in == nullptr ? a.coef[size_t(hu) * kMaxWalk + tid] : 0.f;
  __syncthreads();

  const float* a_in = a.a + size_t(hu) * g.max_tokens;
  const float* p_in = a.p + size_t(hu) * g.walk * g.max_tokens;
  const size_t ext = size_t(u.h) * u.n;   // row of head h in [h_kv, n] exports
  const float ramp = n > 1 ? 1.f / float(n - 1) : 0.f;
  const uint32_t k0 = uint32_t(a.seed), k1 = uint32_t(a.seed >> 32);
  uint64_t code[kFusedPer];
  uint64_t v_or = 0, v_and = ~0ull;
  bool nonfinite = false;
  constexpr int kBatch = 4;   // tokens whose inputs are loaded together
  // One batch at compile-time offset b; the eight batches are spelled out so
  // that every index into code[] is a constant (a loop over all 32 tokens is
  // too large for the unroller, and a runtime index would put code[] in
  // scratch memory).
  auto batch = [&](auto b_const) {
    constexpr int b = decltype(b_const)::value;
    float w[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = tid + kSelThreads * (b + i);
      const int jc = j < n ? j : 0;
      w[i] = a.w_in != nullptr ? a.w_in[ext + jc] : token_weight(a, s_coef, a_in, p_in, ramp, jc);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = tid + kSelThreads * (b + i);
      code[b + i] = 0;
      if (j < n) {
        nonfinite |= !isfinite(w[i]);
        if (a.w_out != nullptr) a.w_out[ext + j] = w[i];
        const uint4 x = philox4x32_10(make_uint4(uint32_t(j), u.unit_id, u.layer, a.step), k0, k1);
        const double uj = philox_uniform53(x.x, x.y);
        double key = w[i] > 0.f ? log(uj) / double(w[i]) : -INFINITY;
        if (j < a.n_sink || j >= n - a.n_recent) key = INFINITY;
        if (a.keys_out != nullptr) a.keys_out[ext + j] = key;
        code[b + i] = key_code(key);
        v_or |= code[b + i];
        v_and &= code[b + i];
      }
    }
  };
  static_assert(kFusedPer == 8 * kBatch, "eight batches");
  batch(std::integral_constant<int, 0>{});
  batch(std::integral_constant<int, kBatch>{});
  batch(std::integral_constant<int, 2 * kBatch>{});
  batch(std::integral_constant<int, 3 * kBatch>{});
  batch(std::integral_constant<int, 4 * kBatch>{});
  batch(std::integral_constant<int, 5 * kBatch>{});
  batch(std::integral_constant<int, 6 * kBatch>{});
  batch(std::integral_constant<int, 7 * kBatch>{});
  if (__syncthreads_or(nonfinite) && tid == 0) raise_status(a, kStatusNonFinite);
  if (u.keep == nullptr) return;
  if (u.budget >= n) {
    for (int j = tid; j < n; j += kSelThreads) u.keep[j] = j;
    return;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    v_or |= __shfl_xor(v_or, m, 64);
    v_and &= __shfl_xor(v_and, m, 64);
  }
  if (lane == 0) { s_or[wave] = v_or; s_and[wave] = v_and; }
  __syncthreads();
  if (tid == 0) {
    uint64_t o = 0, an = ~0ull;
    for (int w = 0; w < kSelWaves; ++w) { o |= s_or[w]; an &= s_and[w]; }
    const uint64_t diff = o ^ an;
    s_need = u.budget;
    s_eq = n;
    if (diff == 0) {                       // every code equal: pure ties
      s_prefix = an;
      s_mask = ~0ull;
      s_done = 1;
    } else {
      const int top = 63 - __clzll(diff);  // highest bit that differs
      const uint64_t above = top == 63 ? 0ull : (~0ull << (top + 1));
      s_prefix = an & above;
      s_mask = above;
      s_done = 0;
      s_start = top;
    }
  }
  __syncthreads();

  // MSD radix passes over the unresolved bits (at most 8, see topb_select).
  int start = s_start;
  while (!s_done && start >= 0) {
    const int shift = start >= 7 ? start - 7 : 0;
    const int width = start - shift + 1;
    const uint32_t dmask = (1u << width) - 1u;
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();
    const uint64_t prefix = s_prefix, mask = s_mask;
#pragma unroll
    for (int i = 0; i < kFusedPer; ++i) {
      const int j = tid + kSelThreads * i;
      if (j < n && (code[i] & mask) == prefix)
        atomicAdd(&s_hist[uint32_t(code[i] >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t h0 = s_hist[4 * lane], h1 = s_hist[4 * lane + 1], h2 = s_hist[4 * lane + 2],
                     h3 = s_hist[4 * lane + 3];
      const uint32_t own = h0 + h1 + h2 + h3;
      uint32_t suf = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off, 64);
        if (lane + off < 64) suf += v;
      }
      const uint32_t higher = suf - own;
      const uint32_t need = uint32_t(s_need);
      if (higher < need && need <= suf) {
        const uint32_t c3 = higher + h3, c2 = c3 + h2, c1 = c2 + h1;
        const int bb = need <= c3 ? 3 : need <= c2 ? 2 : need <= c1 ? 1 : 0;
        const uint32_t acc = bb == 3 ? higher : bb == 2 ? c3 : bb == 1 ? c2 : c1;
        const uint32_t hb = bb == 3 ? h3 : bb == 2 ? h2 : bb == 1 ? h1 : h0;
        s_need = int(need - acc);
        s_eq = int(hb);
        s_prefix = prefix | (uint64_t(4 * lane + bb) << shift);
        s_mask = mask | (uint64_t(dmask) << shift);
        s_done = (hb == need - acc) || shift == 0;
      }
    }
    __syncthreads();
    start = shift - 1;
  }

  if (!s_done) {
    if (tid == 0) raise_status(a, kStatusBadItem);
    for (int j = tid; j < u.budget; j += kSelThreads) u.keep[j] = j;
    return;
  }
  const uint64_t prefix = s_prefix, mask = s_mask;
  const int need = s_need;
  const bool ties = s_eq != need;
  if (tid == 0) s_cut = 0;
  __syncthreads();
  const int n_rounds = (n + kSelThreads - 1) / kSelThreads;
  if (ties) {
    int seen = 0;
#pragma unroll
    for (int r = kFusedPer - 1; r >= 0; --r) {
      if (r < n_rounds && seen < need) {
        const int j = r * kSelThreads + tid;
        const bool eq = j < n && (code[r] & mask) == prefix;
        int tot;
        const int below = block_rank(eq, s_cnt, &tot);
        const int above = tot - below - (eq ? 1 : 0);
        if (eq && seen + above + 1 == need) s_cut = j;
        seen += tot;
      }
    }
    __syncthreads();
  }
  const int cut = s_cut;
  int base = 0;
#pragma unroll
  for (int r = 0; r < kFusedPer; ++r) {
    if (r < n_rounds) {
      const int j = r * kSelThreads + tid;
      bool keep = false;
      if (j < n) {
        const uint64_t top = code[r] & mask;
        keep = top > prefix || (top == prefix && (!ties || j >= cut));
      }
      int tot;
      const int pos = block_rank(keep, s_cnt, &tot);
      if (keep && base + pos < u.budget) u.keep[base + pos] = j;
      base += tot;
    }
  }
}

}  // namespace

hipError_t launch_walk_coef(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(walk_coef_kernel, dim3(a.g.n_hu), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reservoir_keys(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(reservoir_keys_kernel, dim3(a.g.n_kc, a.g.n_hu), dim3(kKeysThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sample_select(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(sample_select_kernel, dim3(a.g.n_hu), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topb_select(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(topb_select_kernel, dim3(a.g.n_hu), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace nx
