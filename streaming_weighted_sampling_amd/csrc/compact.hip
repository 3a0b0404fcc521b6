// K/V compaction on gfx950: after an eviction event inference continues with
// the kept rows only ([Nexus] = "Forget Without Compromise: Nexus Sampling for
// Streaming KV-Cache Eviction Under Fixed Budgets", academ.us article page,
// section 2.1 streaming view).
//
// out[h, r, :] = cache[h, keep[h, r], :] for r < kept, as bit copies (with
// blocks of b tokens, whole blocks: out[h, r] = cache[h, keep[h, r / b] * b
// + r % b]), then the optional appended rows after the kept rows.  Each workgroup
// moves kCompactRows rows of K and of V; every lane moves 16-B chunks, so a
// 256-B row is one fully used 256-B segment read and written by 16 lanes.
// Loads and stores go through buffer resources sized to the head's rows.
// Output stores are non-temporal: the compacted cache is consumed by later
// decode steps, not by this event.
#include "nx_device.hpp"

namespace nx {
namespace {

constexpr int kThreads = 256;

// kRowBytes: 128, 256 or 512.  A block of kCompactRows rows is kCompactRows *
// kRowBytes / 16 chunks; each lane owns kPer of them (chunk c = lane + 256 i),
// loads every index, then every K and V chunk, then stores them all, so that
// 2 * kPer loads per lane are in flight at once.
template <int kRowBytes>
__global__ __launch_bounds__(kThreads) void kv_compact_kernel(const Args a) {
  constexpr int kPerRow = kRowBytes / 16;
  constexpr int kPer = kCompactRows * kPerRow / kThreads;
  static_assert(kPer * kThreads == kCompactRows * kPerRow, "block split");
  const int hu = blockIdx.y;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid || u.out_k == nullptr || u.out_v == nullptr || u.keep == nullptr) return;
  // Kept units are tokens (b = 1) or blocks of b tokens: output row r comes
  // from kept unit r / b, row r % b of it; rows past a short last block are
  // skipped.  Appended rows follow the kept rows.
  const int b = a.g.block;
  const int kept_rows = min(u.kept * b, u.n);
  const int rows = kept_rows + u.n_append;
  const uint32_t src_bytes = uint32_t(u.n) * kRowBytes;
  const uint32_t app_bytes = uint32_t(u.n_append) * kRowBytes;
  const Buf kb(u.k, src_bytes), vb(u.v, src_bytes);
  const Buf kab(u.app_k, app_bytes), vab(u.app_v, app_bytes);
  const Buf okb(u.out_k, uint32_t(rows) * kRowBytes), ovb(u.out_v, uint32_t(rows) * kRowBytes);
  bool bad = false;
  // Row blocks are strided by the grid, so any grid width covers every row.
  for (int r0 = blockIdx.x * kCompactRows; r0 < rows; r0 += gridDim.x * kCompactRows) {
    int src[kPer];    // byte offset of the chunk in its source, or -1
    bool app[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int r = r0 + c / kPerRow;
      const int off = (c % kPerRow) * 16;
      src[i] = -1;
      app[i] = false;
      if (r < kept_rows) {
        const int idx = u.keep[r / b];
        const int sr = idx * b + (r & (b - 1));
        if (idx < 0 || idx >= u.nu) bad = true;
        else if (sr < u.n) src[i] = sr * kRowBytes + off;
      } else if (r < rows) {
        src[i] = (r - kept_rows) * kRowBytes + off;
        app[i] = true;
      }
    }
    uint4 xk[kPer], xv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (src[i] >= 0) {
        xk[i] = app[i] ? kab.ld16(uint32_t(src[i])) : kb.ld16(uint32_t(src[i]));
        xv[i] = app[i] ? vab.ld16(uint32_t(src[i])) : vb.ld16(uint32_t(src[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (src[i] >= 0) {
        const int c = threadIdx.x + kThreads * i;
        const uint32_t dst = uint32_t((r0 + c / kPerRow) * kRowBytes + (c % kPerRow) * 16);
        okb.st16<kNonTemporal>(dst, xk[i]);
        ovb.st16<kNonTemporal>(dst, xv[i]);
      }
    }
  }
  if (__syncthreads_or(bad) && threadIdx.x == 0) raise_status(a, kStatusBadItem);
}

}  // namespace

hipError_t launch_kv_compact(const Args& a, hipStream_t s) {
  const int max_rows = a.g.max_out_rows > 0 ? a.g.max_out_rows : a.g.max_tokens;
  const dim3 grid((max_rows + kCompactRows - 1) / kCompactRows, a.g.n_hu);
  const int row_bytes = a.g.head_dim * (a.g.dtype == NX_BF16 ? 2 : 4);
  switch (row_bytes) {
    case 128: hipLaunchKernelGGL(kv_compact_kernel<128>, grid, dim3(kThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL(kv_compact_kernel<256>, grid, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL(kv_compact_kernel<512>, grid, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace nx
