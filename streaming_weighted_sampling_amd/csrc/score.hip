// Nexus scoring on gfx950: window attention over the resident cache with MFMA.
//
// [Nexus] = "Forget Without Compromise: Nexus Sampling for Streaming KV-Cache
// Eviction Under Fixed Budgets" (academ.us article page).
//
// For one head unit (KV head h of one item) the G query heads h*G .. h*G+G-1
// each contribute W window rows, R = G*W rows in total.  Section 2.1 Eq. (1)
// needs, for every row, softmax over all N resident tokens of Q K^T / sqrt(D);
// "head-averaged" is read as the mean of the G heads' probability rows.  Two
// sweeps over K give exact normalisation without materialising R x N logits:
//
//   score_stats    logits of a 256-token tile for all R rows (one K tile in
//                  LDS serves every query head of the group); per row the
//                  max and the sum of 2^(y - max), y = logit * log2(e)/sqrt(D)
//   score_combine  merges the tile pairs of each row in tile order and stores
//                  beta_r = max_r + log2(Z_r) + log2(G*W)
//   score_probs    logits again; e = 2^(y - beta_r) = p_r / (G*W), so the
//                  direct score of section 2.2 Eq. (3) is a_j = sum_r e_rj, and
//                  each walk row of Eq. (4) is P_t = W * sum_i e_(i,t) j.  It
//                  stores a, the H walk rows and per-tile partials of their
//                  Gram matrix (diagonal: row sums), so that the walk needs no
//                  N x N object and no second pass over the rows.
//
// Row order inside a head unit: the G*H walk rows first, t-major (row t*G+i is
// query head i at window position W-H+t), then the other rows.  MFMA layout
// (v_mfma_f32_32x32x16_bf16, or _32x32x2f32 for fp32 inputs): A = 32 query
// rows, B = 32 tokens, contraction over head_dim.  Lane l holds row / token
// l % 32; its half l / 32 supplies the contraction slots of head dims
// [half*D/2, half*D/2 + D/2), the same dims for A and B, so every lane reads
// one contiguous half-row of 16-B chunks.  Output register v of lane l is
// C[8*(v/4) + 4*(l/32) + v%4][l % 32].
#include "nx_device.hpp"

namespace nx {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

template <typename T, int D>
struct Geo {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kRowBytes = D * int(sizeof(T));
  static constexpr int kHalfBytes = kRowBytes / 2;
  static constexpr int kChunks = kHalfBytes / 16;              // 16-B chunks per lane
  static constexpr int kPitch = kRowBytes + 16;                // LDS row pitch, bytes
  static constexpr int kTileBytes = 32 * kPitch;
  static constexpr int kLoads = (32 * kRowBytes / 16) / kThreads;
  static_assert(kLoads >= 1, "tile smaller than one 16-B load per thread");
};

__device__ inline int out_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

// Window row rho of a head unit -> (query head within the group, window slot).
__device__ inline bool row_source(const Geometry& g, int rho, int& qh, int& wpos) {
  if (rho >= g.rows) return false;
  if (rho < g.walk_rows) {
    const int t = rho / g.group;
    qh = rho - t * g.group;
    wpos = g.window - g.walk + t;
  } else {
    const int r = rho - g.walk_rows;
    const int wn = g.window - g.walk;
    qh = r / wn;
    wpos = r - qh * wn;
  }
  return true;
}

template <typename T, int D, int MPW>
__device__ inline void load_q(const Args& a, const HeadUnit& u, int wave, int nn, int hh,
                              uint4 (&qf)[MPW][Geo<T, D>::kChunks]) {
  using GE = Geo<T, D>;
  const int n_mt = a.g.rows_pad / 32;
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int mt = wave + kWaves * i;
    int qh = 0, wpos = 0;
    const bool ok = mt < n_mt && row_source(a.g, mt * 32 + nn, qh, wpos);
    const char* src = u.q + (int64_t(qh) * a.g.window + wpos) * GE::kRowBytes + hh * GE::kHalfBytes;
#pragma unroll
    for (int c = 0; c < GE::kChunks; ++c)
      qf[i][c] = ok ? *reinterpret_cast<const uint4*>(src + 16 * c) : make_uint4(0, 0, 0, 0);
  }
}

template <typename T, int D>
__device__ inline void load_tile_regs(const char* kbase, int tok0, int n,
                                      uint4 (&r)[Geo<T, D>::kLoads]) {
  using GE = Geo<T, D>;
  constexpr int kPerRow = GE::kRowBytes / 16;
#pragma unroll
  for (int i = 0; i < GE::kLoads; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / kPerRow, col = c - row * kPerRow;
    const int tok = tok0 + row;
    r[i] = tok < n ? *reinterpret_cast<const uint4*>(kbase + int64_t(tok) * GE::kRowBytes + 16 * col)
                   : make_uint4(0, 0, 0, 0);
  }
}

template <typename T, int D>
__device__ inline void store_tile_lds(char* lds, const uint4 (&r)[Geo<T, D>::kLoads]) {
  using GE = Geo<T, D>;
  constexpr int kPerRow = GE::kRowBytes / 16;
#pragma unroll
  for (int i = 0; i < GE::kLoads; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / kPerRow, col = c - row * kPerRow;
    *reinterpret_cast<uint4*>(lds + row * GE::kPitch + 16 * col) = r[i];
  }
}

template <typename T, int D>
__device__ inline void read_frag(const char* lds, int nn, int hh, uint4 (&kf)[Geo<T, D>::kChunks]) {
  using GE = Geo<T, D>;
  const char* p = lds + nn * GE::kPitch + hh * GE::kHalfBytes;
#pragma unroll
  for (int c = 0; c < GE::kChunks; ++c) kf[c] = *reinterpret_cast<const uint4*>(p + 16 * c);
}

// Raw dot products of 32 query rows with 32 tokens (no scaling).
template <typename T, int D>
__device__ inline floatx16_t mfma_tile(const uint4 (&qf)[Geo<T, D>::kChunks],
                                       const uint4 (&kf)[Geo<T, D>::kChunks]) {
  using GE = Geo<T, D>;
  floatx16_t acc = {};
#pragma unroll
  for (int c = 0; c < GE::kChunks; ++c) {
    if constexpr (GE::kBf16) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qf[c]),
                                                    __builtin_bit_cast(bf16x8_t, kf[c]), acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(qf[c].x), __uint_as_float(kf[c].x), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(qf[c].y), __uint_as_float(kf[c].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(qf[c].z), __uint_as_float(kf[c].z), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(qf[c].w), __uint_as_float(kf[c].w), acc, 0, 0, 0);
    }
  }
  return acc;
}

// One sweep of pass 1 over the block's tokens.  kExact = false keeps one
// shift per row (the row max of the first 32 tokens) and adds 2^(y - shift);
// kExact = true keeps a per-lane running max (two exponentials per logit) and
// is only used when the cheap sweep overflowed.
template <typename T, int D, int MPW, bool kExact>
__device__ inline void stats_sweep(const Args& a, const HeadUnit& u, int t0, int n_sub,
                                   const uint4 (&qf)[MPW][Geo<T, D>::kChunks],
                                   float (&my)[MPW][16], float (&z)[MPW][16], char* lds0, char* lds1) {
  using GE = Geo<T, D>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nn = lane & 31, hh = lane >> 5;
  const int n_mt = a.g.rows_pad / 32;
  const float c = a.c_log2;
  uint4 pre[GE::kLoads];
  load_tile_regs<T, D>(u.k, t0, u.n, pre);
  store_tile_lds<T, D>(lds0, pre);
  __syncthreads();
  for (int st = 0; st < n_sub; ++st) {
    char* cur = (st & 1) ? lds1 : lds0;
    char* nxt = (st & 1) ? lds0 : lds1;
    if (st + 1 < n_sub) load_tile_regs<T, D>(u.k, t0 + 32 * (st + 1), u.n, pre);
    uint4 kf[GE::kChunks];
    read_frag<T, D>(cur, nn, hh, kf);
    const bool valid = t0 + 32 * st + nn < u.n;
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      if (wave + kWaves * i < n_mt) {
        const floatx16_t acc = mfma_tile<T, D>(qf[i], kf);
        if constexpr (!kExact) {
          if (st == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              my[i][v] = half_max(valid ? acc[v] * c : -INFINITY);
              z[i][v] = 0.f;
            }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float e = __builtin_amdgcn_exp2f(fmaf(acc[v], c, -my[i][v]));
            z[i][v] += valid ? e : 0.f;
          }
        } else {
          if (st == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) { my[i][v] = -INFINITY; z[i][v] = 0.f; }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float y = acc[v] * c;
            if (valid) {
              const float m2 = fmaxf(my[i][v], y);
              z[i][v] = z[i][v] * __builtin_amdgcn_exp2f(my[i][v] - m2) + __builtin_amdgcn_exp2f(y - m2);
              my[i][v] = m2;
            }
          }
        }
      }
    }
    if (st + 1 < n_sub) store_tile_lds<T, D>(nxt, pre);
    __syncthreads();
  }
}

template <typename T, int D, int MPW>
__global__ __launch_bounds__(kThreads) void score_stats_kernel(const Args a) {
  using GE = Geo<T, D>;
  __shared__ __align__(16) char lds[2][GE::kTileBytes];
  const int hu = blockIdx.y, tile = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int t0 = tile * kTokPerBlock;
  if (t0 >= u.n) return;
  const int n_sub = (min(t0 + kTokPerBlock, u.n) - t0 + 31) / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nn = lane & 31, hh = lane >> 5;
  const int n_mt = a.g.rows_pad / 32;

  uint4 qf[MPW][GE::kChunks];
  load_q<T, D, MPW>(a, u, wave, nn, hh, qf);
  float my[MPW][16], z[MPW][16];
#pragma unroll
  for (int i = 0; i < MPW; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) { my[i][v] = 0.f; z[i][v] = 0.f; }
  stats_sweep<T, D, MPW, false>(a, u, t0, n_sub, qf, my, z, lds[0], lds[1]);

  // Merge the 32 lanes of each half (they share rows); detect overflow.
  float zr[MPW][16];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      zr[i][v] = half_sum(z[i][v]);
      bad |= (wave + kWaves * i < n_mt) && !(zr[i][v] <= 0x1p126f);
    }
  }
  if (__syncthreads_or(bad)) {
    stats_sweep<T, D, MPW, true>(a, u, t0, n_sub, qf, my, z, lds[0], lds[1]);
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float m = half_max(my[i][v]);
        zr[i][v] = half_sum(z[i][v] * __builtin_amdgcn_exp2f(my[i][v] - m));
        my[i][v] = m;
      }
    }
  }
  float* out = a.part1 + (size_t(hu) * a.g.n_t1 + tile) * a.g.rows_pad * 2;
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int mt = wave + kWaves * i;
    if (mt < n_mt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        if (nn == v) {
          const int rho = mt * 32 + out_row(v, hh);
          *reinterpret_cast<float2*>(out + 2 * rho) = make_float2(my[i][v], zr[i][v]);
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void score_combine_kernel(const Args a) {
  const int hu = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) {
    if (threadIdx.x == 0) raise_status(a, kStatusBadItem);
    return;
  }
  const int n_tiles = (u.n + kTokPerBlock - 1) / kTokPerBlock;
  const float* part = a.part1 + size_t(hu) * a.g.n_t1 * a.g.rows_pad * 2;
  const float log2_gw = log2f(float(a.g.group * a.g.window));
  for (int rho = threadIdx.x; rho < a.g.rows_pad; rho += kThreads) {
    float beta = INFINITY;
    if (rho < a.g.rows) {
      float m = -INFINITY;
      for (int t = 0; t < n_tiles; ++t) m = fmaxf(m, part[(size_t(t) * a.g.rows_pad + rho) * 2]);
      float zsum = 0.f;
      for (int t = 0; t < n_tiles; ++t) {
        const float2 p = *reinterpret_cast<const float2*>(part + (size_t(t) * a.g.rows_pad + rho) * 2);
        zsum += p.y * __builtin_amdgcn_exp2f(p.x - m);
      }
      beta = m + log2f(zsum) + log2_gw;
    }
    a.beta[size_t(hu) * a.g.rows_pad + rho] = beta;
  }
}

template <typename T, int D, int MPW>
__global__ __launch_bounds__(kThreads) void score_probs_kernel(const Args a) {
  using GE = Geo<T, D>;
  __shared__ __align__(16) char lds[2][GE::kTileBytes];
  __shared__ float s_tok[kWaves][32];
  __shared__ float s_walk[kMaxWalkRows][32];
  const int hu = blockIdx.y, tile = blockIdx.x;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) return;
  const int t0 = tile * kTokPerBlock;
  if (t0 >= u.n) return;
  const int n_sub = (min(t0 + kTokPerBlock, u.n) - t0 + 31) / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nn = lane & 31, hh = lane >> 5;
  const Geometry& g = a.g;
  const int n_mt = g.rows_pad / 32;
  const float c = a.c_log2;

  uint4 qf[MPW][GE::kChunks];
  load_q<T, D, MPW>(a, u, wave, nn, hh, qf);
  float bt[MPW][16];
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int mt = wave + kWaves * i;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      bt[i][v] = mt < n_mt ? a.beta[size_t(hu) * g.rows_pad + mt * 32 + out_row(v, hh)] : INFINITY;
  }
  float gacc[kMaxWalk][kMaxWalk];
#pragma unroll
  for (int t = 0; t < kMaxWalk; ++t)
#pragma unroll
    for (int t2 = 0; t2 < kMaxWalk; ++t2) gacc[t][t2] = 0.f;

  float* a_out = a.a + size_t(hu) * g.max_tokens;
  float* p_out = a.p + size_t(hu) * g.walk * g.max_tokens;
  const float wf = float(g.window);

  uint4 pre[GE::kLoads];
  load_tile_regs<T, D>(u.k, t0, u.n, pre);
  store_tile_lds<T, D>(lds[0], pre);
  __syncthreads();
  for (int st = 0; st < n_sub; ++st) {
    char* cur = lds[st & 1];
    char* nxt = lds[(st + 1) & 1];
    if (st + 1 < n_sub) load_tile_regs<T, D>(u.k, t0 + 32 * (st + 1), u.n, pre);
    uint4 kf[GE::kChunks];
    read_frag<T, D>(cur, nn, hh, kf);
    float tp = 0.f;
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int mt = wave + kWaves * i;
      if (mt < n_mt) {
        const floatx16_t acc = mfma_tile<T, D>(qf[i], kf);
        const bool walk_tile = mt * 32 < g.walk_rows;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = __builtin_amdgcn_exp2f(fmaf(acc[v], c, -bt[i][v]));
          tp += e;
          if (walk_tile) {
            const int rho = mt * 32 + out_row(v, hh);
            if (rho < g.walk_rows) s_walk[rho][nn] = e;
          }
        }
      }
    }
    tp += __shfl_xor(tp, 32, 64);
    if (hh == 0) s_tok[wave][nn] = tp;
    __syncthreads();
    if (threadIdx.x < 32) {
      const int j = threadIdx.x;
      const int tok = t0 + 32 * st + j;
      if (tok < u.n) {
        a_out[tok] = ((s_tok[0][j] + s_tok[1][j]) + s_tok[2][j]) + s_tok[3][j];
        float pt[kMaxWalk];
#pragma unroll
        for (int t = 0; t < kMaxWalk; ++t) {
          pt[t] = 0.f;
          if (t < g.walk) {
            float s = 0.f;
            for (int i = 0; i < g.group; ++i) s += s_walk[t * g.group + i][j];
            pt[t] = wf * s;
            p_out[size_t(t) * g.max_tokens + tok] = pt[t];
          }
        }
        // Off-diagonal: <P_t, P_t'> for t' < t; diagonal: the row sum |P_t|_1.
#pragma unroll
        for (int t = 0; t < kMaxWalk; ++t)
#pragma unroll
          for (int t2 = 0; t2 <= t; ++t2)
            gacc[t][t2] = fmaf(pt[t], t2 == t ? 1.f : pt[t2], gacc[t][t2]);
      }
    }
    if (st + 1 < n_sub) store_tile_lds<T, D>(nxt, pre);
    __syncthreads();
  }
  if (wave == 0) {
    float* gout = a.gram + (size_t(hu) * g.n_t2 + tile) * (kMaxWalk * kMaxWalk);
#pragma unroll
    for (int t = 0; t < kMaxWalk; ++t) {
#pragma unroll
      for (int t2 = 0; t2 <= t; ++t2) {
        if (t < g.walk) {
          const float s = half_sum(gacc[t][t2]);
          if (lane == 0) gout[t * kMaxWalk + t2] = s;
        }
      }
    }
  }
}

int mtiles_per_wave(const Geometry& g) {
  const int n_mt = g.rows_pad / 32;
  const int per = (n_mt + kWaves - 1) / kWaves;
  return per <= 1 ? 1 : per <= 2 ? 2 : 4;
}

template <int MPW, typename T, int D>
hipError_t launch_stats_t(const Args& a, hipStream_t s, dim3 grid) {
  hipLaunchKernelGGL((score_stats_kernel<T, D, MPW>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
template <int MPW, typename T, int D>
hipError_t launch_probs_t(const Args& a, hipStream_t s, dim3 grid) {
  hipLaunchKernelGGL((score_probs_kernel<T, D, MPW>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool kProbs>
hipError_t launch_pass(const Args& a, hipStream_t s) {
  const Geometry& g = a.g;
  const dim3 grid(kProbs ? g.n_t2 : g.n_t1, g.n_hu);
  const int mpw = mtiles_per_wave(g);
#define NX_PASS(MPW, T, D) \
  return kProbs ? launch_probs_t<MPW, T, D>(a, s, grid) : launch_stats_t<MPW, T, D>(a, s, grid)
#define NX_PASS_MPW(T, D)                 \
  switch (mpw) {                          \
    case 1: NX_PASS(1, T, D);             \
    case 2: NX_PASS(2, T, D);             \
    default: NX_PASS(4, T, D);            \
  }
  if (g.dtype == NX_BF16) {
    if (g.head_dim == 128) { NX_PASS_MPW(uint16_t, 128) }
    NX_PASS_MPW(uint16_t, 64)
  }
  if (g.head_dim == 128) { NX_PASS_MPW(float, 128) }
  NX_PASS_MPW(float, 64)
#undef NX_PASS_MPW
#undef NX_PASS
}

}  // namespace

hipError_t launch_score_stats(const Args& a, hipStream_t s) { return launch_pass<false>(a, s); }

hipError_t launch_score_combine(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(score_combine_kernel, dim3(a.g.n_hu), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_score_probs(const Args& a, hipStream_t s) { return launch_pass<true>(a, s); }

}  // namespace nx
