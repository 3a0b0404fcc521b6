// K/V compaction on gfx950: after an eviction event inference continues with
// the kept rows only ([Nexus] = "Forget Without Compromise: Nexus Sampling for
// Streaming KV-Cache Eviction Under Fixed Budgets", academ.us article page,
// section 2.1 streaming view).
//
// out[h, r, :] = cache[h, keep[h, r], :] for r < kept, as bit copies, then the
// optional appended rows out[h, kept + i, :] = app[h, i, :].  Each workgroup
// moves kCompactRows rows of K and of V; every lane moves 16-B chunks, so a
// 256-B row is one fully used 256-B segment read and written by 16 lanes.
// Output stores are non-temporal: the compacted cache is consumed by later
// decode steps, not by this event.
#include "nx_device.hpp"

namespace nx {
namespace {

constexpr int kThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void kv_compact_kernel(const Args a) {
  const int hu = blockIdx.y;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid || u.out_k == nullptr || u.out_v == nullptr || u.keep == nullptr) return;
  const int rows = u.kept + u.n_append;
  if (int(blockIdx.x) * kCompactRows >= rows) return;
  const int row_bytes = a.g.head_dim * (a.g.dtype == NX_BF16 ? 2 : 4);
  const int per_row = row_bytes / 16;
  bool bad = false;
  // Row blocks are strided by the grid, so any grid width covers every row.
  for (int r0 = blockIdx.x * kCompactRows; r0 < rows; r0 += gridDim.x * kCompactRows) {
  const int r1 = min(r0 + kCompactRows, rows);
  for (int c = threadIdx.x; c < (r1 - r0) * per_row; c += kThreads) {
    const int r = r0 + c / per_row;
    const int col = c - (c / per_row) * per_row;
    const char* sk;
    const char* sv;
    if (r < u.kept) {
      const int idx = u.keep[r];
      if (idx < 0 || idx >= u.n) { bad = true; continue; }
      sk = u.k + int64_t(idx) * row_bytes;
      sv = u.v + int64_t(idx) * row_bytes;
    } else {
      sk = u.app_k + int64_t(r - u.kept) * row_bytes;
      sv = u.app_v + int64_t(r - u.kept) * row_bytes;
    }
    const u32x4 xk = *reinterpret_cast<const u32x4*>(sk + 16 * col);
    const u32x4 xv = *reinterpret_cast<const u32x4*>(sv + 16 * col);
    __builtin_nontemporal_store(xk, reinterpret_cast<u32x4*>(u.out_k + int64_t(r) * row_bytes + 16 * col));
    __builtin_nontemporal_store(xv, reinterpret_cast<u32x4*>(u.out_v + int64_t(r) * row_bytes + 16 * col));
  }
  }
  if (__syncthreads_or(bad) && threadIdx.x == 0) raise_status(a, kStatusBadItem);
}

}  // namespace

hipError_t launch_kv_compact(const Args& a, hipStream_t s) {
  const int max_rows = a.g.max_out_rows > 0 ? a.g.max_out_rows : a.g.max_tokens;
  const dim3 grid((max_rows + kCompactRows - 1) / kCompactRows, a.g.n_hu);
  hipLaunchKernelGGL(kv_compact_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace nx
