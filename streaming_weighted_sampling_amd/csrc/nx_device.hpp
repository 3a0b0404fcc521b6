// Device helpers shared by the HIP kernels: head-unit resolution, the Philox
// generator, key encoding and wavefront reductions.  gfx950 only (wave64).
#pragma once

#include "nx_internal.hpp"

namespace nx {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Global memory through a buffer resource (MUBUF instructions).  Unlike FLAT
// accesses these count only against the vector-memory counter, so waiting for
// an LDS read never waits for in-flight global loads; loads at offsets past
// `bytes` return zero and stores there are dropped.  The base and size must
// be uniform across the wavefront.
constexpr int kRsrcWord3 = 0x00020000;   // gfx9: raw buffer, 32-bit data format
constexpr int kNonTemporal = 2;          // cache-policy bit for streaming stores

struct Buf {
  __amdgpu_buffer_rsrc_t r;
  __device__ Buf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3)) {}
  template <int kAux = 0>
  __device__ uint4 ld16(uint32_t off) const {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ float ldf(uint32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
  template <int kAux = 0>
  __device__ void st16(uint32_t off, uint4 v) const {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, kAux);
  }
  __device__ void stf(uint32_t off, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
  }
};

// Global -> LDS copies that bypass the VGPRs (buffer_load_dwordx4 with the lds
// modifier): lane l of the wavefront writes its 16 bytes to LDS address
// M0 + 16 * l, so one instruction fills 1 KB of LDS.  Issued through inline
// assembly so that the compiler does not order every later LDS read behind
// all such copies; the caller waits with vm_wait<>() and a barrier.  Offsets
// at or past `bytes` read as zero.  With `nt` (wave-uniform) the copies carry
// the non-temporal hint, for K streams far larger than the caches.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

struct LdsDma {
  i32x4_t r;
  bool nt;
  __device__ LdsDma(const void* base, uint32_t bytes, bool nt_ = false) : nt(nt_) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    r = i32x4_t{__builtin_amdgcn_readfirstlane(int(uint32_t(b))),
                __builtin_amdgcn_readfirstlane(int(uint32_t(b >> 32) & 0xFFFF)),
                __builtin_amdgcn_readfirstlane(int(bytes)), kRsrcWord3};
  }
  // The same copy with the hint fixed at compile time (no branch per copy).
  template <bool kNT>
  __device__ void load16_t(uint32_t lds_addr, uint32_t voff) const {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if constexpr (kNT)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                   :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r)
                   : "memory", "m0");
#pragma clang diagnostic pop
  }
  // lds_addr: wave-uniform LDS byte address of this wavefront's 1 KB block.
  __device__ void load16(uint32_t lds_addr, uint32_t voff) const {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if (nt)
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                   :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r)
                   : "memory", "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(r)
                   : "memory", "m0");
#pragma clang diagnostic pop
  }
};

// LDS byte address of a __shared__ object.
__device__ inline uint32_t lds_address(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Wait until at most N vector-memory operations of this wavefront are in
// flight (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The second sweep's per-token outputs of head unit hu: a_j at a[j * ts] and
// walk row P_t[j] at p[t * rs + j * ts] (planar rows, or 16-byte records
// (a, P_1, P_2, P_3) when the geometry packs them).
struct ScoreRows {
  const float* a;
  const float* p;
  int ts;
  size_t rs;
};
__device__ inline ScoreRows score_rows(const Args& a, int hu) {
  const size_t nm = size_t(a.g.max_tokens);
  if (a.g.packed) {
    const float* rec = a.a + size_t(hu) * nm * 4;
    return {rec, rec + 1, 4, 1};
  }
  return {a.a + size_t(hu) * nm, a.p + size_t(hu) * a.g.walk * nm, 1, nm};
}

// One KV head of one (sequence, layer) item, resolved on the device.
struct HeadUnit {
  const char* q;       // first query row of the GQA group (query head h * G)
  const char* k;       // this head's cache rows
  const char* v;
  int32_t* keep;       // this head's keep indices (budget entries)
  char* out_k;
  char* out_v;
  const char* app_k;
  const char* app_v;
  float* w_out;        // nullable: this head's weight export row (nu entries)
  int32_t* tokens_out; // nullable: where this head's row count after the event goes
  int32_t n, budget, kept, n_append;
  int32_t nu;          // selection units: ceil(n / block); kept = min(budget, nu) of them
  int32_t cap;         // keep row length: budget, or the per-head capacity
  uint32_t layer, unit_id;
  int32_t h;
  bool valid;
};

__device__ inline nx_unit load_item(const Args& a, int item) {
  if (a.units == nullptr) return a.single;
  return a.units[item];
}

// Resolve head unit `hu` (= item * H_kv + kv_head); checks the item's fields.
__device__ inline HeadUnit head_unit(const Args& a, int hu) {
  const Geometry& g = a.g;
  const int item = hu / g.h_kv;
  const int h = hu - item * g.h_kv;
  const nx_unit u = load_item(a, item);
  const int64_t esz = g.dtype == NX_BF16 ? 2 : 4;
  const int64_t d = g.head_dim;
  HeadUnit r;
  r.h = h;
  // Per-head resident counts (decode with per-head budgets), bounded by the
  // item's n_tokens.
  r.n = u.head_tokens != nullptr ? u.head_tokens[h] : u.n_tokens;
  // Per-head budgets: keep rows of `cap` entries; the head's own budget (given
  // ones at every stage, allocated ones once this call's allocation is in
  // place; before that, the capacity).
  const bool per_head = g.head_alloc != NX_HEADS_UNIFORM;
  const bool budgets_in = a.heads_live || g.head_alloc == NX_HEADS_GIVEN;
  r.cap = per_head && u.head_cap > 0 ? u.head_cap : u.budget;
  r.budget = !per_head ? u.budget
             : (budgets_in && u.head_budget != nullptr) ? u.head_budget[h] : r.cap;
  r.nu = (r.n + g.block - 1) / g.block;
  r.kept = r.budget < r.nu ? r.budget : r.nu;
  r.n_append = u.n_append;
  r.layer = u.layer;
  r.unit_id = u.seq_id * uint32_t(g.h_kv) + uint32_t(h);
  r.q = static_cast<const char*>(u.q) + int64_t(h) * g.group * g.window * d * esz;
  r.k = static_cast<const char*>(u.k) + int64_t(h) * u.kv_head_stride * esz;
  r.v = u.v ? static_cast<const char*>(u.v) + int64_t(h) * u.kv_head_stride * esz : nullptr;
  r.keep = u.keep ? u.keep + int64_t(h) * r.cap : nullptr;
  r.out_k = u.out_k ? static_cast<char*>(u.out_k) + int64_t(h) * u.out_head_stride * esz : nullptr;
  r.out_v = u.out_v ? static_cast<char*>(u.out_v) + int64_t(h) * u.out_head_stride * esz : nullptr;
  r.app_k = u.app_k ? static_cast<const char*>(u.app_k) + int64_t(h) * u.n_append * d * esz : nullptr;
  r.app_v = u.app_v ? static_cast<const char*>(u.app_v) + int64_t(h) * u.n_append * d * esz : nullptr;
  // The weight export keeps the item's row stride (units of n_tokens).
  r.w_out = u.out_w ? u.out_w + int64_t(h) * ((u.n_tokens + g.block - 1) / g.block) : nullptr;
  r.tokens_out = u.head_tokens_out ? u.head_tokens_out + h : nullptr;
  bool ok = u.n_tokens >= 1 && u.n_tokens <= g.max_n && r.n >= 1 && r.n <= u.n_tokens &&
            u.budget >= 1 &&
            u.n_append >= 0 && r.budget >= 1 && r.budget <= r.cap &&
            (a.n_sink + a.n_recent <= r.budget || r.budget >= r.nu) &&
            u.kv_head_stride >= int64_t(u.n_tokens) * d && u.q != nullptr && u.k != nullptr;
  if (per_head) ok = ok && u.head_cap >= 0 && u.head_budget != nullptr;
  // The counts written after the event must not change the ones this event reads.
  if (u.head_tokens != nullptr && u.head_tokens_out != nullptr)
    ok = ok && (u.head_tokens_out + g.h_kv <= u.head_tokens || u.head_tokens + g.h_kv <= u.head_tokens_out);
  // Rows of the kept units (whole blocks; a short last block only shortens it),
  // at most the capacity's.
  const int64_t kept_rows = min(int64_t(min(r.cap, r.nu)) * g.block, int64_t(r.n));
  if (u.out_k || u.out_v)
    ok = ok && u.out_head_stride >= (kept_rows + u.n_append) * d &&
         (kept_rows + u.n_append) * d * esz <= INT32_MAX;
  if (g.block > 1 && u.n_append > 0) ok = ok && r.n % g.block == 0;
  if (g.inplace)   // k / v are compacted in place and must hold the appended rows too
    ok = ok && u.out_k == nullptr && u.out_v == nullptr && u.v != nullptr &&
         u.kv_head_stride >= (kept_rows + u.n_append) * d &&
         (kept_rows + u.n_append) * d * esz <= INT32_MAX;
  if (u.n_append > 0) ok = ok && u.app_k != nullptr && u.app_v != nullptr;
  r.valid = ok;
  return r;
}

__device__ inline void raise_status(const Args& a, uint32_t bits) {
  atomicOr(a.status, bits);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// Philox-4x32 S-box with multipliers 0xD2511F53 / 0xCD9E8D57, the round key
// bumped by the Weyl constants 0x9E3779B9 / 0xBB67AE85 between rounds.
__device__ inline uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = uint64_t(0xD2511F53u) * c.x;
    const uint64_t p1 = uint64_t(0xCD9E8D57u) * c.z;
    const uint32_t hi0 = uint32_t(p0 >> 32), lo0 = uint32_t(p0);
    const uint32_t hi1 = uint32_t(p1 >> 32), lo1 = uint32_t(p1);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// 53-bit uniform in (0, 1] from the first two output words.
__device__ inline double philox_uniform53(uint32_t x0, uint32_t x1) {
  const uint64_t k53 = ((uint64_t(x0) << 32) | uint64_t(x1)) >> 11;
  return double(k53 + 1) * 0x1p-53;
}

// Order-preserving encoding of an fp64 key as uint64 (larger key, larger code).
// -0.0 is folded into +0.0 first.
__device__ inline uint64_t key_code(double x) {
  x = x + 0.0;
  const uint64_t b = uint64_t(__double_as_longlong(x));
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ inline double key_decode(uint64_t c) {
  const uint64_t b = (c >> 63) ? (c & 0x7FFFFFFFFFFFFFFFull) : ~c;
  return __longlong_as_double(static_cast<long long>(b));
}

// Sums / max over the 32 lanes that share a lane-half (xor masks below 32).
__device__ inline float half_sum(float x) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ inline float half_max(float x) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

}  // namespace nx
