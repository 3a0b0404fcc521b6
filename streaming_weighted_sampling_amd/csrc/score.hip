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
// C[8*(v/4) + 4*(l/32) + v%4][l % 32].  Workgroups of 4 wavefronts owning one
// 32-row tile each up to 128 rows; above, 8 wavefronts owning two tiles each
// (up to 512 rows).

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
  static constexpr int kCpr = kRowBytes / 16;                  // 16-B chunks per row
  static constexpr int kTileBytes = 32 * kRowBytes;            // one sub-tile, no padding
  static_assert(kCpr == 8 || kCpr == 16 || kCpr == 32, "row of 128, 256 or 512 bytes");
  // LDS holds chunk s of row r at slot s ^ swz(r): the 16 rows that a
  // ds_read_b128 serves together then fall in 16 different 16-B bank groups.
  __device__ static int swz(int row) { return kCpr == 8 ? (row >> 1) & 7 : row & 15; }
  // Ring slots: LDS for the K sub-tiles in flight (pass 1 at four
  // workgroups per CU, pass 2 at three next to its walk buffers; 160 KB of
  // LDS per CU).
  static constexpr int kSlotsStats = kTileBytes <= 4096 ? 8 : (39 * 1024) / kTileBytes;
  static constexpr int kSlotsProbs = kTileBytes <= 4096 ? 8 : (32 * 1024) / kTileBytes;
  static_assert(kSlotsStats >= 2 && kSlotsProbs >= 2, "ring needs two slots");
};

__device__ inline int out_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

// Sum over aligned groups of b lanes (b a power of two up to 32, inside a
// lane half), every lane of a group receiving the group's sum in a fixed
// order: DPP lane moves inside a row of 16 (quad permutes for partners at
// distance 1 and 2, then the half-row and row mirrors, which pair each lane
// with the other quad / half of its row), and one cross-row permute for 32.
__device__ inline float dpp_add(float x, int ctrl_sel) {
  int v;
  switch (ctrl_sel) {
    case 0: v = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: v = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    case 2: v = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: v = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return x + __int_as_float(v);
}
__device__ inline float group_sum(float x, int b) {
  if (b >= 2) x = dpp_add(x, 0);
  if (b >= 4) x = dpp_add(x, 1);
  if (b >= 8) x = dpp_add(x, 2);
  if (b >= 16) x = dpp_add(x, 3);
  if (b >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

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

template <typename T, int D, int MPW, int NW = kWaves>
__device__ inline void load_q(const Args& a, const HeadUnit& u, int wave, int nn, int hh,
                              uint4 (&qf)[MPW][Geo<T, D>::kChunks]) {
  using GE = Geo<T, D>;
  const int n_mt = a.g.rows_pad / 32;
  const Buf qb(u.q, uint32_t(a.g.group * a.g.window * GE::kRowBytes));
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int mt = wave + NW * i;
    int qh = 0, wpos = 0;
    const bool ok = mt < n_mt && row_source(a.g, mt * 32 + nn, qh, wpos);
    const uint32_t src = uint32_t((qh * a.g.window + wpos) * GE::kRowBytes + hh * GE::kHalfBytes);
#pragma unroll
    for (int c = 0; c < GE::kChunks; ++c)
      qf[i][c] = ok ? qb.ld16(src + 16 * c) : make_uint4(0, 0, 0, 0);
  }
}

template <typename T, int D>
__device__ inline void read_frag(const char* lds, int nn, int hh, uint4 (&kf)[Geo<T, D>::kChunks]) {
  using GE = Geo<T, D>;
  const char* p = lds + nn * GE::kRowBytes;
  const int x = GE::swz(nn);
#pragma unroll
  for (int c = 0; c < GE::kChunks; ++c)
    kf[c] = *reinterpret_cast<const uint4*>(p + (((hh * GE::kChunks + c) ^ x) << 4));
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

// Streams the block's K sub-tiles (32 tokens each) through a ring of kSlots
// LDS slots filled by global -> LDS copies, kSlots - 1 sub-tiles ahead of the
// one being consumed, without holding them in registers.  The copies are
// issued by the wavefronts of the last kLoaders roles only (role: a
// permutation of the wavefront index): every vector-memory operation
// of a wavefront counts against the one vmcnt, so a wavefront that also
// stores to global memory would, when it waits for its copies, wait for its
// stores as well.  Per sub-tile: the loaders wait for their copies of it, one
// barrier (everyone's copies landed, everyone is done with the slot about to
// be refilled), refill, body(st, lds).  Rows past the cache end read as zero.
// Ends on a barrier.
template <typename T, int D, int kSlots, int kLoaders, int NW, bool kNT, typename Body>
__device__ inline void sweep_tiles_impl(const HeadUnit& u, int t0, int n_sub, char* ring, int role,
                                        Body&& body) {
  using GE = Geo<T, D>;
  constexpr int kPerWave = GE::kTileBytes / (1024 * kLoaders);   // copies per loader per tile
  static_assert(kPerWave >= 1 && kPerWave * 1024 * kLoaders == GE::kTileBytes, "tile split");
  static_assert((kSlots - 2) * kPerWave < 64, "vmcnt range");
  const int t1 = min(t0 + 32 * n_sub, u.n);
  const LdsDma dma(u.k + int64_t(t0) * GE::kRowBytes, uint32_t((t1 - t0) * GE::kRowBytes), kNT);
  const int lw = role - (NW - kLoaders);   // loader index, < 0: not a loader
  const bool loader = lw >= 0;
  const int lane = threadIdx.x & 63;
  // Copy i of loader lw fills LDS chunk (i * kLoaders + lw) * 64 + lane.
  uint32_t voff[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int lc = (i * kLoaders + lw) * 64 + lane;
    const int row = lc / GE::kCpr, slot = lc % GE::kCpr;
    voff[i] = uint32_t(row * GE::kRowBytes + ((slot ^ GE::swz(row)) << 4));
  }
  const uint32_t ring_lds = lds_address(ring) + uint32_t(lw * 1024);
  auto issue = [&](int st) {
    if (!loader) return;
    const uint32_t dst = ring_lds + uint32_t((st % kSlots) * GE::kTileBytes);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      dma.template load16_t<kNT>(dst + uint32_t(i * kLoaders * 1024), voff[i] + uint32_t(st * GE::kTileBytes));
  };
#pragma unroll
  for (int r = 0; r < kSlots - 1; ++r)
    if (r < n_sub) issue(r);
  // The caller's own loads (query fragments, row offsets) were issued before
  // the ring: let them and the prologue land together, once.  Otherwise the
  // compiler, which does not see the ring copies, would place a full vmcnt(0)
  // in front of the first use of those registers inside the loop.
  vm_wait<0>();
  for (int st = 0; st < n_sub; ++st) {
    if (loader) {
      if (st + kSlots - 2 < n_sub)
        vm_wait<(kSlots - 2) * kPerWave>();
      else
        vm_wait<0>();
    }
    __syncthreads();
    if (st + kSlots - 1 < n_sub) issue(st + kSlots - 1);
    body(st, ring + (st % kSlots) * GE::kTileBytes);
  }
  __syncthreads();
}

// The sweep, unswitched on the non-temporal hint of the K copies (wave-uniform):
// the copy issue inside the loop then carries no branch.
template <typename T, int D, int kSlots, int kLoaders, int NW, typename Body>
__device__ inline void sweep_tiles(const HeadUnit& u, int t0, int n_sub, char* ring, int role, bool nt,
                                   Body&& body) {
  if (nt)
    sweep_tiles_impl<T, D, kSlots, kLoaders, NW, true>(u, t0, n_sub, ring, role, body);
  else
    sweep_tiles_impl<T, D, kSlots, kLoaders, NW, false>(u, t0, n_sub, ring, role, body);
}

// Pass 1 over the block's tokens.  kExact = false keeps one shift per row (the
// row max over the first 32 tokens) and adds 2^(y - shift) per logit;
// kExact = true keeps a per-lane running max (two exponentials per logit) and
// only runs when the cheap sweep overflowed.
template <typename T, int D, int MPW, int NW, bool kExact>
__device__ inline void stats_sweep(const Args& a, const HeadUnit& u, int t0, int n_sub,
                                   const uint4 (&qf)[MPW][Geo<T, D>::kChunks],
                                   float (&my)[MPW][16], float (&z)[MPW][16], char* ring) {
  using GE = Geo<T, D>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nn = lane & 31, hh = lane >> 5;
  const int n_mt = a.g.rows_pad / 32;
  const float c = a.c_log2;
  // Every wavefront copies K, at least one 1-KB copy each per sub-tile.
  constexpr int kLoaders = NW < GE::kTileBytes / 1024 ? NW : GE::kTileBytes / 1024;
  sweep_tiles<T, D, GE::kSlotsStats, kLoaders, NW>(u, t0, n_sub, ring, wave, a.k_stream_nt1 != 0,
                                                   [&](int st, const char* cur) {
    uint4 kf[GE::kChunks];
    read_frag<T, D>(cur, nn, hh, kf);
    const bool full = t0 + 32 * st + 32 <= u.n;      // wave-uniform
    const bool valid = t0 + 32 * st + nn < u.n;
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      if (wave + NW * i < n_mt) {
        const floatx16_t acc = mfma_tile<T, D>(qf[i], kf);
        if constexpr (!kExact) {
          if (st == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) my[i][v] = half_max(valid ? acc[v] * c : -INFINITY);
          }
          if (full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) z[i][v] += __builtin_amdgcn_exp2f(fmaf(acc[v], c, -my[i][v]));
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float e = __builtin_amdgcn_exp2f(fmaf(acc[v], c, -my[i][v]));
              z[i][v] += valid ? e : 0.f;
            }
          }
        } else {
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
  });
}

// Pass 1 on one (head unit, tile) item: writes the tile's (max, sum) pair
// for every window row.
template <typename T, int D, int MPW, int NW>
__device__ inline void stats_item(const Args& a, const HeadUnit& u, int hu, int tile, char* smem) {
  using GE = Geo<T, D>;
  const int tpb = a.g.tok_per_block;
  const int t0 = tile * tpb;
  if (t0 >= u.n) return;
  const int n_sub = (min(t0 + tpb, u.n) - t0 + 31) / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nn = lane & 31, hh = lane >> 5;
  const int n_mt = a.g.rows_pad / 32;

  uint4 qf[MPW][GE::kChunks];
  load_q<T, D, MPW, NW>(a, u, wave, nn, hh, qf);
  float my[MPW][16], z[MPW][16];
#pragma unroll
  for (int i = 0; i < MPW; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) { my[i][v] = 0.f; z[i][v] = 0.f; }
  stats_sweep<T, D, MPW, NW, false>(a, u, t0, n_sub, qf, my, z, smem);

  // Merge the 32 lanes of each half (they share rows); detect overflow.
  float zr[MPW][16];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      zr[i][v] = half_sum(z[i][v]);
      bad |= (wave + NW * i < n_mt) && !(zr[i][v] <= 0x1p126f);
    }
  }
  if (__syncthreads_or(bad)) {
#pragma unroll
    for (int i = 0; i < MPW; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) { my[i][v] = -INFINITY; z[i][v] = 0.f; }
    stats_sweep<T, D, MPW, NW, true>(a, u, t0, n_sub, qf, my, z, smem);
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
    const int mt = wave + NW * i;
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

// Merge the tile pairs of every window row of one head unit in tile order:
// beta_r = max_r + log2(Z_r) + log2(G*W) (one row per thread, nthreads threads
// from tid; tile pairs are loaded 16 at a time so the loads overlap), into
// out[rho] for rho < rows_pad.
__device__ inline void combine_rows(const Args& a, const HeadUnit& u, int hu, float* out, int tid,
                                    int nthreads) {
  const int n_tiles = (u.n + a.g.tok_per_block - 1) / a.g.tok_per_block;
  const float* part = a.part1 + size_t(hu) * a.g.n_t1 * a.g.rows_pad * 2;
  const float log2_gw = log2f(float(a.g.group * a.g.window));
  constexpr int kBatch = 16;
  for (int rho = tid; rho < a.g.rows_pad; rho += nthreads) {
    float beta = INFINITY;
    if (rho < a.g.rows) {
      float m = -INFINITY, zsum = 0.f;
      for (int t0 = 0; t0 < n_tiles; t0 += kBatch) {
        float2 p[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          p[i] = t0 + i < n_tiles
                     ? *reinterpret_cast<const float2*>(part + (size_t(t0 + i) * a.g.rows_pad + rho) * 2)
                     : make_float2(-INFINITY, 0.f);
        float mb = m;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) mb = fmaxf(mb, p[i].x);
        float zb = zsum * __builtin_amdgcn_exp2f(m - mb);
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (t0 + i < n_tiles) zb += p[i].y * __builtin_amdgcn_exp2f(p[i].x - mb);
        m = mb;
        zsum = zb;
      }
      beta = m + log2f(zsum) + log2_gw;
    }
    out[rho] = beta;
  }
}

// The row merge of one head unit by a whole workgroup, into the workspace.
__device__ inline void combine_unit(const Args& a, int hu) {
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid) {
    if (threadIdx.x == 0) raise_status(a, kStatusBadItem);
    return;
  }
  combine_rows(a, u, hu, a.beta + size_t(hu) * a.g.rows_pad, threadIdx.x, kThreads);
}

// Walk modes of pass 2 (template parameter, chosen on the host).
constexpr int kWalkNone = 0;    // H = 0
constexpr int kWalkFast4 = 1;   // G = 4, H <= 4: P_t from register group sums
constexpr int kWalkFast8 = 2;   // G = 8, H <= 4
constexpr int kWalkLds = 3;     // any other shape: walk rows through LDS
constexpr int kWalkFast4Deep = 4;   // G = 4, 6 < H <= 8
constexpr int kWalkFast4Mid = 5;    // G = 4, 4 < H <= 6 (fewer Gram pairs per lane than Deep,
                                    // which keeps the kernel within 128 VGPRs)
constexpr int kWalkFast4H3 = 6;     // G = 4, H = 3 exactly (no per-row depth tests)
constexpr int kWalkFast8H3 = 7;     // G = 8, H = 3 exactly
constexpr int kWalkGlobal = 8;      // deep walks: every row tile stores its P_t rows (no Gram here)
constexpr int kWalkFast4H5 = 9;     // G = 4, H = 5 exactly (15 Gram pairs, no per-row depth tests)

// Pass 2 on one (head unit, tile) item.
//
// Every wave owns whole M-tiles (window rows) and all 32 tokens of each
// sub-tile.  Work that combines values across waves runs one sub-tile late,
// from LDS, in the shadow of the next sub-tile's MFMA and exponentials, so
// the one barrier per sub-tile of the K sweep is the only synchronisation.
// Roles are numbered r = (wave + blockIdx.x + blockIdx.y) mod 4, so that the
// extra work of roles 0 and 1 does not always land on the same SIMDs:
//   * role r owns M-tiles r, r + 4, ...; it leaves its partial of a_j for the
//     sub-tile's 32 tokens in LDS, and half 0 of role 1 adds the partials in
//     role (= M-tile) order and stores a_j;
//   * the walk rows live in M-tile 0 (role 0).  For G = 4 or 8 with
//     G*H <= 32 each walk row covers whole 4-row groups of the MFMA output,
//     so role 0 forms P_t in registers from in-lane group sums and one
//     half-swap; other shapes leave the e values in LDS and role 0 sums them
//     one sub-tile later.  Either way P_t goes to global memory and to LDS
//     (for H = 3 at token granularity only to LDS: role 1 then stores a_j
//     and P_1..P_3 of each token as one 16-byte record).
//     Roles 0 and 1 issue every global store of the pass and roles 2 and 3
//     every K copy, so that no ring wait also waits for stores;
//   * the Gram partials <P_t, P_t'> (diagonal |P_t|_1) accumulate one (or,
//     for the LDS walk, two) sub-tiles late: half-wave k = 2r + half owns the
//     pairs p = 7 - k, 15 - k, ... (p = t(t+1)/2 + t') at one token per lane.
// Every sum runs in a fixed order, whatever the roles.
template <typename T, int D, int kWalk, int NW>
constexpr int probs_smem_bytes() {
  return Geo<T, D>::kSlotsProbs * Geo<T, D>::kTileBytes +
         int(sizeof(float)) * 2 * 32 * ((kWalk == kWalkLds ? kMaxWalkRows : 0) + kMaxWalk + NW);
}

// kBlocks: the call selects blocks of b > 1 tokens (b = 1 kernels carry no
// block-sum code, which keeps them within 128 VGPRs).
template <typename T, int D, int MPW, int NW, int kWalk, bool kBlocks>
__device__ inline void probs_item(const Args& a, const HeadUnit& u, int hu, int tile, char* smem) {
  using GE = Geo<T, D>;
  constexpr bool kHasWalk = kWalk != kWalkNone;
  constexpr bool kGlobal = kWalk == kWalkGlobal;
  constexpr bool kHasGram = kHasWalk && !kGlobal;   // Gram partials formed in this pass
  constexpr int kExactH = kWalk == kWalkFast4H3 || kWalk == kWalkFast8H3 ? 3
                         : kWalk == kWalkFast4H5                        ? 5
                                                                        : 0;
  constexpr bool kG8 = kWalk == kWalkFast8 || kWalk == kWalkFast8H3;   // walk rows span 8 output rows
  constexpr bool kFastWalk = kWalk == kWalkFast4 || kWalk == kWalkFast8 || kWalk == kWalkFast4Deep ||
                             kWalk == kWalkFast4Mid || kExactH > 0;
  constexpr int kMaxT = kExactH > 0                                ? kExactH
                        : kWalk == kWalkFast8 || kWalk == kWalkFast4 ? 4
                        : kWalk == kWalkFast4Mid                   ? 6
                                                                   : kMaxWalk;   // deepest walk
  // Exactly three walk rows at token granularity: a_j and P_1..P_3 leave as one
  // 16-byte record per token (the rule of packed_rows: G = 4 or 8, H = 3, b = 1).
  constexpr bool kPacked = kExactH == 3 && !kBlocks;
  constexpr int kHalfWaves = 2 * NW;
  constexpr int kPairsPerLane = (kMaxT * (kMaxT + 1) / 2 + kHalfWaves - 1) / kHalfWaves;
  auto s_pt = reinterpret_cast<float (*)[kMaxWalk][32]>(smem + GE::kSlotsProbs * GE::kTileBytes);
  auto s_a = reinterpret_cast<float (*)[NW][32]>(smem + GE::kSlotsProbs * GE::kTileBytes +
                                                     2 * kMaxWalk * 32 * 4);
  auto s_walk = reinterpret_cast<float (*)[kMaxWalkRows][32]>(
      smem + GE::kSlotsProbs * GE::kTileBytes + 2 * (kMaxWalk + NW) * 32 * 4);
  const int tpb = a.g.tok_per_block;
  const int t0 = tile * tpb;
  if (t0 >= u.n) return;
  const int n_sub = (min(t0 + tpb, u.n) - t0 + 31) / 32;
  const int lane = threadIdx.x & 63, nn = lane & 31, hh = lane >> 5;
  const int role = ((threadIdx.x >> 6) + blockIdx.x + blockIdx.y) & (NW - 1);
  const Geometry& g = a.g;
  const int n_mt = g.rows_pad / 32;
  const int row_roles = min(n_mt, NW);
  const float c = a.c_log2;
  // == g.walk for the mode the host picked (a constant for the exact-depth modes)
  const int walk = kExactH > 0 ? kExactH : min(g.walk, kMaxT);
  const int n_pairs = walk * (walk + 1) / 2;
  const int pg = kHalfWaves - 1 - (2 * role + hh);   // first Gram pair of this half-wave

  uint4 qf[MPW][GE::kChunks];
  load_q<T, D, MPW, NW>(a, u, role, nn, hh, qf);
  // beta of this unit's rows: from the row merge, or (small calls, no merge
  // launch) merged here into the LDS the ring fills only after the barrier.
  const float* beta = a.beta + size_t(hu) * g.rows_pad;
  if (a.beta_in_probs) {
    float* s_beta = reinterpret_cast<float*>(smem);
    combine_rows(a, u, hu, s_beta, threadIdx.x, 64 * NW);
    __syncthreads();
    beta = s_beta;
  }
  float bt[MPW][16];
#pragma unroll
  for (int i = 0; i < MPW; ++i) {
    const int mt = role + NW * i;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      bt[i][v] = mt < n_mt ? beta[mt * 32 + out_row(v, hh)] : INFINITY;
  }
  if (a.beta_in_probs) __syncthreads();   // every wavefront has read the merge's LDS
  // This lane's Gram pairs (t, t'), 3 bits each, packed 6 bits per pair.
  uint32_t pairs = 0;
  float gacc[kPairsPerLane];
#pragma unroll
  for (int k = 0; k < kPairsPerLane; ++k) {
    const int p = pg + kHalfWaves * k;
    int t = 0;
    while ((t + 1) * (t + 2) / 2 <= p) ++t;
    const int t2 = p - t * (t + 1) / 2;
    pairs |= uint32_t(((t & 7) << 3) | (t2 & 7)) << (6 * k);
    gacc[k] = 0.f;
  }

  const Buf a_out(a.a + size_t(hu) * g.max_tokens * (kPacked ? 4 : 1),
                  uint32_t(g.max_tokens * (kPacked ? 16 : 4)));
  const Buf p_out(a.p + size_t(hu) * g.walk * g.max_tokens, uint32_t(g.walk * g.max_tokens * 4));
  const float wf = float(g.window);

  // P_t of token t0 + 32 s + nn (lanes of half 0): global and LDS; tokens past
  // the cache end enter the Gram as zero.
  // With blocks (b > 1) the values of a block's b lanes are summed (BlockSum_b
  // of Eq. 1); the block's first lane stores the sum at the block index and
  // holds it in LDS, the other lanes hold 0, so the Gram sees block rows.
  const int blk = kBlocks ? g.block : 1;
  const bool lead = (nn & (blk - 1)) == 0;
  auto put_walk = [&](int s, const float (&pt)[kMaxT]) {
    const int tok = t0 + 32 * s + nn;
    const bool ok = tok < u.n;
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      if (t < walk) {
        if (blk == 1) {
          if (!kPacked && ok) p_out.stf(uint32_t((t * g.max_tokens + tok) * 4), pt[t]);
          s_pt[s & 1][t][nn] = ok ? pt[t] : 0.f;
        } else {
          const float v = group_sum(ok ? pt[t] : 0.f, blk);
          if (lead && ok) p_out.stf(uint32_t((t * g.max_tokens + tok / blk) * 4), v);
          s_pt[s & 1][t][nn] = lead ? v : 0.f;
        }
      }
    }
  };
  // LDS walk rows of sub-tile s (role 0, half 0).
  auto walk_lds = [&](int s) {
    if (role != 0 || hh != 0) return;
    float pt[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      pt[t] = 0.f;
      if (t < walk) {
        float sum = 0.f;
        for (int i = 0; i < g.group; ++i) sum += s_walk[s & 1][t * g.group + i][nn];
        pt[t] = wf * sum;
      }
    }
    put_walk(s, pt);
  };
  // The Gram step is split into its LDS reads (issued before the K fragment
  // reads of the next sub-tile) and its accumulation (after that sub-tile's
  // MFMA chain has been issued), so that neither waits on the critical path.
  // Every half-wave runs kcap iterations (uniform); pairs past n_pairs read
  // in-bounds rows and are not accumulated.
  const int kcap = (n_pairs + kHalfWaves - 1) / kHalfWaves;
  auto gram_load = [&](int s, float (&gx)[kPairsPerLane], float (&gy)[kPairsPerLane]) {
    const float* sp = &s_pt[s & 1][0][nn];
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) {
      if (k < kcap) {
        const uint32_t t = (pairs >> (6 * k + 3)) & 7, t2 = (pairs >> (6 * k)) & 7;
        gx[k] = sp[32 * t];
        gy[k] = sp[32 * t2];
      }
    }
  };
  auto gram_add = [&](const float (&gx)[kPairsPerLane], const float (&gy)[kPairsPerLane]) {
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) {
      if (k < kcap) {
        const uint32_t t = (pairs >> (6 * k + 3)) & 7, t2 = (pairs >> (6 * k)) & 7;
        const float f = fmaf(gx[k], t2 == t ? 1.f : gy[k], gacc[k]);
        gacc[k] = pg + kHalfWaves * k < n_pairs ? f : gacc[k];
      }
    }
  };
  auto gram_step = [&](int s) {
    float gx[kPairsPerLane], gy[kPairsPerLane];
    gram_load(s, gx, gy);
    gram_add(gx, gy);
  };
  // a_j of sub-tile s: M-tile-ordered sum of the partials (role 1, half 0),
  // likewise split into the reads and the sum and store.
  auto a_load = [&](int s, float (&la)[NW]) {
#pragma unroll
    for (int r = 0; r < NW; ++r) la[r] = s_a[s & 1][r][nn];
  };
  // Packed records: P_t of sub-tile s was left in LDS by role 0 before the
  // barrier that ended sub-tile s (the Gram step reads the same slots).
  auto p_load = [&](int s, float (&lp)[3]) {
#pragma unroll
    for (int t = 0; t < 3; ++t) lp[t] = s_pt[s & 1][t][nn];
  };
  auto a_put_rec = [&](int s, float sum, const float (&lp)[3]) {   // lanes of half 0
    const int tok = t0 + 32 * s + nn;
    if (tok < u.n)
      a_out.st16(uint32_t(tok * 16), make_uint4(__float_as_uint(sum), __float_as_uint(lp[0]),
                                                __float_as_uint(lp[1]), __float_as_uint(lp[2])));
  };
  auto a_put = [&](int s, float sum) {   // lanes of half 0
    const int tok = t0 + 32 * s + nn;
    if constexpr (kPacked) {
      float lp[3];
      p_load(s, lp);
      a_put_rec(s, sum, lp);
    } else if (blk == 1) {
      if (tok < u.n) a_out.stf(uint32_t(tok * 4), sum);
    } else {
      sum = group_sum(tok < u.n ? sum : 0.f, blk);
      if (lead && tok < u.n) a_out.stf(uint32_t((tok / blk) * 4), sum);
    }
  };
  auto a_store = [&](int s, const float (&la)[NW], const float (&lp)[3]) {
    if (hh != 0) return;
    float sum = la[0];
#pragma unroll
    for (int r = 1; r < NW; ++r)
      if (r < row_roles) sum += la[r];
    if constexpr (kPacked) a_put_rec(s, sum, lp);
    else a_put(s, sum);
  };
  auto a_final = [&](int s) {
    if (role != 1) return;
    if constexpr (NW > kWaves) {
      // Each lane half sums half of the partials (in role order), one swap
      // adds the two halves.
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < NW / 2; ++r) {
        const int rr = hh * (NW / 2) + r;
        if (rr < row_roles) part += s_a[s & 1][rr][nn];
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part),
                                                       false, false);
      const float sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (hh == 0) a_put(s, sum);
    } else {
      float la[NW], lp[3] = {};
      a_load(s, la);
      if constexpr (kPacked) p_load(s, lp);
      a_store(s, la, lp);
    }
  };

  // Deep walks: P_t = W * (sum of its G rows) for the tokens of sub-tile st.
  // Lane (nn, hh) holds rows 8q + 4hh + r (q, r < 4) in e[4q + r] and their
  // quad sums in sq[q]; a group of G rows is then a sum of e's (G <= 2), a
  // quad sum (G = 4), or quad sums of both halves (G >= 8, one swap).
  auto store_walk_rows = [&](int mt, int st, const float (&e)[16], const float (&sq)[4]) {
    const int G = g.group;
    const int tok = t0 + 32 * st + nn;
    const bool ok = tok < u.n;
    // Group of rows rho0 .. rho0 + G - 1; every lane takes part (the block
    // sums move values across lanes), lanes with mine set store.
    auto put = [&](int rho0, float sum, bool mine) {
      const int t = rho0 / G;
      float v = wf * sum;
      if (blk == 1) {
        if (mine && ok && t < g.walk) p_out.stf(uint32_t((t * g.max_tokens + tok) * 4), v);
      } else {
        v = group_sum(ok ? v : 0.f, blk);
        if (mine && lead && ok && t < g.walk)
          p_out.stf(uint32_t((t * g.max_tokens + tok / blk) * 4), v);
      }
    };
    if (G <= 4) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = mt * 32 + 8 * q + 4 * hh;
        if (G == 4) {
          put(r0, sq[q], true);
        } else if (G == 2) {
          put(r0, e[4 * q] + e[4 * q + 1], true);
          put(r0 + 2, e[4 * q + 2] + e[4 * q + 3], true);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) put(r0 + r, e[4 * q + r], true);
        }
      }
    } else {
      // Sums of G / 8 consecutive quads (rows 8q .. 8q + 8 G/8 - 1 of one
      // half), then the two halves added by one swap (both halves then hold
      // the same sum, half 0 + half 1); half 0 stores.
      const int span = G / 8;   // 1, 2 or 4 quads
      float part[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) part[q] = sq[q];
      if (span >= 2) { part[0] += part[1]; part[2] += part[3]; }
      if (span >= 4) part[0] += part[2];
#pragma unroll
      for (int q = 0; q < 4; q += 1) {
        if (q % span != 0) continue;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[q]),
                                                         __float_as_uint(part[q]), false, false);
        const float sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        put(mt * 32 + 8 * q, sum, hh == 0);
      }
    }
  };

  sweep_tiles<T, D, GE::kSlotsProbs, 2, NW>(u, t0, n_sub, smem, role, a.k_stream_nt != 0,
                                           [&](int st, const char* cur) {
    // Lagged work on slots the previous barrier made visible: the LDS reads
    // now, ahead of the K fragment reads; the sums after the MFMA issue.
    // (The LDS walk mode keeps its lagged work in one piece, ahead of the
    // fragment reads: splitting it costs it occupancy.)
    // With 8 wavefronts the lagged work also stays in one piece: holding
    // eight a_j partials across the MFMA chains would spill.
    constexpr bool kSplitLag = kWalk != kWalkLds && NW == kWaves;
    const bool lag = st > 0;
    float la[NW], lp[3] = {}, gx[kPairsPerLane], gy[kPairsPerLane];
    if (lag) {
      if constexpr (kSplitLag) {
        if (role == 1) {
          a_load(st - 1, la);
          if constexpr (kPacked) p_load(st - 1, lp);
        }
        if constexpr (kFastWalk) gram_load(st - 1, gx, gy);
      } else if constexpr (kWalk == kWalkLds) {
        a_final(st - 1);
        walk_lds(st - 1);
        if (st > 1) gram_step(st - 2);
      } else {
        a_final(st - 1);
        if constexpr (kFastWalk) gram_step(st - 1);
      }
    }
    uint4 kf[GE::kChunks];
    read_frag<T, D>(cur, nn, hh, kf);
    float tp = 0.f;
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
      const int mt = role + NW * i;
      auto consume_lag = [&] {
        if constexpr (kSplitLag) {
          if (role == 1) a_store(st - 1, la, lp);
          if constexpr (kFastWalk) gram_add(gx, gy);
        }
      };
      if (mt >= n_mt && i == 0 && lag) consume_lag();
      if (mt < n_mt) {
        const floatx16_t acc = mfma_tile<T, D>(qf[i], kf);
        if (i == 0 && lag) consume_lag();
        float e[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) e[v] = __builtin_amdgcn_exp2f(fmaf(acc[v], c, -bt[i][v]));
        // Sums of the 4-row groups 8q + 4*half .. +3, then of the lane's 16
        // rows, as a tree (no chain of 16 dependent adds).
        float sq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sq[q] = (e[4 * q] + e[4 * q + 1]) + (e[4 * q + 2] + e[4 * q + 3]);
        tp += (sq[0] + sq[1]) + (sq[2] + sq[3]);
        if constexpr (kFastWalk && !kG8 && !kBlocks && !kPacked) {
          if (i == 0 && role == 0) {
            // G = 4 with planar walk rows: walk row t is the 4-row group
            // 8q + 4*half .. +3 with t = 2q + half, which this lane half
            // already sums in sq[q]; each half writes and stores its own rows
            // (no exchange between the halves, the stores split over both).
            // With packed records role 0 only fills LDS, where the exchange
            // below measured faster.
            const int tok = t0 + 32 * st + nn;
            const bool ok = tok < u.n;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int t = 2 * q + hh;
              if (t < walk) {
                const float v = wf * sq[q];
                if (ok) p_out.stf(uint32_t((t * g.max_tokens + tok) * 4), v);
                s_pt[st & 1][t][nn] = ok ? v : 0.f;
              }
            }
          }
        } else if constexpr (kFastWalk) {
          if (i == 0 && role == 0) {
            // Group sums S over rows 8q + 4*half .. +3; after the swap every
            // lane holds S for q' = 2q (half 0) and q' = 2q + 1 (half 1).
            float grp[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float sg = sq[q];
              const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sg),
                                                               __float_as_uint(sg), false, false);
              grp[2 * q] = __uint_as_float(sw[0]);
              grp[2 * q + 1] = __uint_as_float(sw[1]);
            }
            if (hh == 0) {
              float pt[kMaxT];
#pragma unroll
              for (int t = 0; t < kMaxT; ++t)
                pt[t] = wf * (!kG8 ? grp[t] : grp[2 * t] + grp[2 * t + 1]);
              put_walk(st, pt);
            }
          }
        } else if constexpr (kGlobal) {
          // Walk rows are rows 0 .. G*H - 1, G consecutive rows per window
          // slot t (G <= 32 divides the tile's 32 rows): a tile that holds
          // some of them sums each group and stores P_t of its 32 tokens.
          if (mt * 32 < g.walk_rows) store_walk_rows(mt, st, e, sq);
        } else if constexpr (kWalk == kWalkLds) {
          // Walk rows are rows 0 .. G*H - 1: every row tile that holds some
          // of them (G*H may exceed one tile's 32 rows) leaves their values.
          if (mt * 32 < g.walk_rows) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rho = mt * 32 + out_row(v, hh);
              if (rho < g.walk_rows) s_walk[st & 1][rho][nn] = e[v];
            }
          }
        }
      }
    }
    // tp over this wave's rows: own half + the other half (same token).
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tp), __float_as_uint(tp),
                                                     false, false);
    tp = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (role < row_roles && hh == 0) s_a[st & 1][role][nn] = tp;
  });
  // Drain the lagged work (the sweep ends on a barrier).
  a_final(n_sub - 1);
  if constexpr (kHasGram) {
    if constexpr (kWalk == kWalkLds) {
      if (n_sub > 1) gram_step(n_sub - 2);
      walk_lds(n_sub - 1);
      __syncthreads();
    }
    gram_step(n_sub - 1);
    // Each pair is owned by one half-wave: sum its 32 lanes in a fixed order.
    float* gout = a.gram + (size_t(hu) * g.n_t2 + tile) * (kMaxWalk * kMaxWalk);
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) {
      const int p = pg + kHalfWaves * k;
      if (p < n_pairs) {
        const float sum = half_sum(gacc[k]);
        if (nn == 0) {
          int t = 0;
          while ((t + 1) * (t + 2) / 2 <= p) ++t;
          gout[t * kMaxWalk + (p - t * (t + 1) / 2)] = sum;
        }
      }
    }
  }
}

// Pass 1: one workgroup per (tile, head unit).
// NW wavefronts of MPW row tiles per workgroup (4 x 1, or 8 x 2 above 4 row
// tiles): one tile per wavefront keeps its query fragments and row statistics
// within 128 VGPRs, four wavefronts per SIMD; two tiles take ~232 VGPRs, two
// wavefronts per SIMD (four tiles per wavefront took 252-256, one).
template <typename T, int D, int MPW, int NW>
__global__ __launch_bounds__(64 * NW) void score_stats_kernel(const Args a) {
  __shared__ __align__(16) char smem[Geo<T, D>::kSlotsStats * Geo<T, D>::kTileBytes];
  const int tile = blockIdx.x, hu = blockIdx.y;
  const HeadUnit u = head_unit(a, hu);
  if (u.valid) stats_item<T, D, MPW, NW>(a, u, hu, tile, smem);
}

// Row merge: one workgroup per head unit.
__global__ __launch_bounds__(kThreads) void score_combine_kernel(const Args a) {
  combine_unit(a, blockIdx.x);
}

// Pass 2: one workgroup per (tile, head unit).
// bf16 without blocks and with a register-lean walk form is held to 128 VGPRs
// (4 wavefronts per SIMD), which it reaches without spilling; fp32, blocks and
// the LDS, deep and global walk forms need more and run at 2-3.
template <typename T, int kWalk, bool kBlocks, int MPW>
constexpr int probs_min_waves() {
  return MPW == 1 && sizeof(T) == 2 && !kBlocks && kWalk != kWalkLds && kWalk != kWalkFast4Deep &&
                 kWalk != kWalkGlobal
             ? 4
             : 1;
}

template <typename T, int D, int MPW, int NW, int kWalk, bool kBlocks>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(probs_min_waves<T, kWalk, kBlocks, MPW>())))
void score_probs_kernel(const Args a) {
  __shared__ __align__(16) char smem[probs_smem_bytes<T, D, kWalk, NW>()];
  const int tile = blockIdx.x, hu = blockIdx.y;
  const HeadUnit u = head_unit(a, hu);
  if (u.valid) probs_item<T, D, MPW, NW, kWalk, kBlocks>(a, u, hu, tile, smem);
  else if (a.beta_in_probs && tile == 0 && threadIdx.x == 0) raise_status(a, kStatusBadItem);
}

int walk_mode(const Geometry& g) {
  if (g.walk == 0) return kWalkNone;
  if (g.deep) return kWalkGlobal;
  if (g.walk == 3 && g.group == 4) return kWalkFast4H3;
  if (g.walk == 3 && g.group == 8) return kWalkFast8H3;
  if (g.walk == 5 && g.group == 4) return kWalkFast4H5;
  if (g.walk <= 4 && g.group == 4) return kWalkFast4;
  if (g.walk <= 4 && g.group == 8) return kWalkFast8;
  if (g.walk <= 6 && g.group == 4) return kWalkFast4Mid;
  if (g.walk_rows <= 32 && g.group == 4) return kWalkFast4Deep;
  return kWalkLds;
}

// Wavefronts per workgroup: 4 (one row tile each) up to 4 row tiles, else 8
// (two row tiles each; the host allows at most 16 tiles: G*W <= 512).
int waves_per_group(const Geometry& g) { return g.rows_pad / 32 <= 4 ? 4 : 8; }

template <int MPW, int NW, typename T, int D, bool kBlocks>
void launch_probs(const Args& a, dim3 grid, hipStream_t s) {
  switch (walk_mode(a.g)) {
    case kWalkNone:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkNone, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast4:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast4, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast8:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast8, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast4H3:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast4H3, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast8H3:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast8H3, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast4Deep:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast4Deep, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast4Mid:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast4Mid, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkFast4H5:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkFast4H5, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    case kWalkGlobal:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkGlobal, kBlocks>), grid, dim3(64 * NW), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((score_probs_kernel<T, D, MPW, NW, kWalkLds, kBlocks>), grid, dim3(64 * NW), 0, s, a);
  }
}

// NW wavefronts of MPW row tiles each per workgroup: up to 4 row tiles, four
// wavefronts of one tile; above, eight wavefronts of two tiles (16 tiles: G*W
// up to 512 rows).  Two tiles per wavefront read each K fragment from LDS once
// for both MFMA chains (the 16 one-tile wavefronts of a 512-row workgroup
// re-read every sub-tile 16 times, as much LDS time as the MFMA work) and give
// each wavefront two independent chains; measured on the 70B-shaped share
// against sixteen one-tile wavefronts: 1.40 -> 1.31 ms (pass 1), 1.45 -> 1.32 ms
// (pass 2), three interleaved rounds.
template <bool kProbs, int NW, typename T, int D>
hipError_t launch_t(const Args& a, hipStream_t s) {
  constexpr int MPW = NW == 8 ? 2 : 1;
  const dim3 grid(a.g.n_tmax, a.g.n_hu);
  if constexpr (kProbs) {
    if (a.g.block > 1) launch_probs<MPW, NW, T, D, true>(a, grid, s);
    else launch_probs<MPW, NW, T, D, false>(a, grid, s);
  } else {
    hipLaunchKernelGGL((score_stats_kernel<T, D, MPW, NW>), grid, dim3(64 * NW), 0, s, a);
  }
  return hipGetLastError();
}

template <bool kProbs>
hipError_t launch_pass(const Args& a, hipStream_t s) {
  const Geometry& g = a.g;
  const int nw = waves_per_group(g);
#define NX_MPW(T, D)                                            \
  if (nw == 4) return launch_t<kProbs, 4, T, D>(a, s);          \
  return launch_t<kProbs, 8, T, D>(a, s);
  if (g.dtype == NX_BF16) {
    if (g.head_dim == 128) { NX_MPW(uint16_t, 128) }
    NX_MPW(uint16_t, 64)
  }
  if (g.head_dim == 128) { NX_MPW(float, 128) }
  NX_MPW(float, 64)
#undef NX_MPW
}

// ---------------------------------------------------------------------------
// Read-ceiling probe (measurement only): streams a buffer the way the score
// sweeps stream K.  The buffer is cut into "heads" of up to 2^22 rows of 256 B
// (1 GiB, so 32-bit buffer offsets address them); one workgroup reads
// `span` consecutive rows: 2048 (a score workgroup at 2048 tokens) for large
// buffers, fewer for small ones so that every buffer gets >= 2048 workgroups.  Mode 0 copies through the sweeps' LDS ring (global -> LDS, four
// slots of 8 KB, every wavefront a loader) and reads each slot back as MFMA
// fragments; mode 1 issues plain 16-B vector loads, eight in flight per lane.
// Every value read is folded into an XOR that is stored only if it equals an
// unlikely constant, so no load is dead and nothing else is written.
constexpr int kProbeRows = 2048;
constexpr int64_t kProbeHeadRows = int64_t(1) << 22;

template <int kMode>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, int64_t rows,
                                                               int span, uint32_t* sink) {
  using GE = Geo<uint16_t, 128>;
  __shared__ __align__(16) char smem[GE::kSlotsStats * GE::kTileBytes];
  const int64_t head_row0 = int64_t(blockIdx.y) * kProbeHeadRows;
  const int64_t head_rows = min(kProbeHeadRows, rows - head_row0);
  const int t0 = int(blockIdx.x) * span;
  if (t0 >= head_rows) return;
  const int n = int(head_rows);
  const char* base = src + head_row0 * GE::kRowBytes;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t acc = 0;
  if constexpr (kMode == 0) {
    HeadUnit u{};
    u.k = base;
    u.n = n;
    const int n_sub = (min(t0 + span, n) - t0 + 31) / 32;
    sweep_tiles<uint16_t, 128, GE::kSlotsStats, kWaves, kWaves>(u, t0, n_sub, smem, wave, false,
                                                                [&](int, const char* cur) {
      uint4 kf[GE::kChunks];
      read_frag<uint16_t, 128>(cur, lane & 31, lane >> 5, kf);
#pragma unroll
      for (int c = 0; c < GE::kChunks; ++c) acc ^= kf[c].x ^ kf[c].y ^ kf[c].z ^ kf[c].w;
    });
  } else {
    const int t1 = min(t0 + span, n);
    const Buf b(base + int64_t(t0) * GE::kRowBytes, uint32_t((t1 - t0) * GE::kRowBytes));
    const uint32_t bytes = uint32_t((t1 - t0) * GE::kRowBytes);
    constexpr int kInFlight = 8;
    for (uint32_t off = threadIdx.x * 16u; off < bytes; off += kThreads * 16u * kInFlight) {
      uint4 v[kInFlight];
#pragma unroll
      for (int i = 0; i < kInFlight; ++i) v[i] = b.ld16(off + uint32_t(i) * kThreads * 16u);
#pragma unroll
      for (int i = 0; i < kInFlight; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_score_stats(const Args& a, hipStream_t s) { return launch_pass<false>(a, s); }

hipError_t launch_score_combine(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(score_combine_kernel, dim3(a.g.n_hu), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_score_probs(const Args& a, hipStream_t s) { return launch_pass<true>(a, s); }

hipError_t launch_stream_read(const void* src, int64_t rows, int mode, uint32_t* sink,
                              hipStream_t s) {
  const int64_t heads = (rows + kProbeHeadRows - 1) / kProbeHeadRows;
  const int64_t per_head = rows < kProbeHeadRows ? rows : kProbeHeadRows;
  int span = kProbeRows;
  while (span > 32 && rows / span < 2048) span /= 2;
  const dim3 grid(unsigned((per_head + span - 1) / span), unsigned(heads));
  if (mode == 0)
    hipLaunchKernelGGL(stream_read_kernel<0>, grid, dim3(kThreads), 0, s,
                       static_cast<const char*>(src), rows, span, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<1>, grid, dim3(kThreads), 0, s,
                       static_cast<const char*>(src), rows, span, sink);
  return hipGetLastError();
}

}  // namespace nx
