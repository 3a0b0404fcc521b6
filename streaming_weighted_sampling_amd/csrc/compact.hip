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
// Loads and stores are non-temporal: every source row is read once, and the
// compacted cache is consumed by later decode steps, not by this event.
#include <algorithm>

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
  // The head's row count after the event (the next event's resident count).
  if (blockIdx.x == 0 && threadIdx.x == 0 && u.tokens_out != nullptr) *u.tokens_out = rows;
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
        xk[i] = app[i] ? kab.ld16<kNonTemporal>(uint32_t(src[i])) : kb.ld16<kNonTemporal>(uint32_t(src[i]));
        xv[i] = app[i] ? vab.ld16<kNonTemporal>(uint32_t(src[i])) : vb.ld16<kNonTemporal>(uint32_t(src[i]));
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

// In-place compaction (hole filling) for streaming.  With kept rows in
// ascending keep[0..kept) (with blocks of b tokens: the kept blocks' rows,
// row i = keep[i / b] * b + i % b, kept = the kept rows; hole filling at row
// level moves whole aligned blocks whenever kept is a multiple of b, and a
// short last block splits no other block), let c = #{keep[i] < kept}: rows keep[c..kept) are
// the movers (kept rows at or past position kept) and the evicted positions
// below kept are the holes, equally many.  The j-th mover goes to the j-th
// hole; since keep[i] - i counts the holes before keep[i], the j-th hole is
// j + i + 1 for the last i < c with keep[i] - i <= j (or j when none).
// Sources (>= kept) and destinations (< kept) are disjoint; the appended rows
// are written by a second kernel so that none overwrites a mover before it is
// read.  Rows move as 16-B chunks, one kCompactRows block of movers per
// workgroup.
constexpr int kLdsKeep = 12288;   // keep entries staged in LDS for the searches (48 KB)

// Moves the movers of one head unit; keep(i) reads keep entry i.  The two
// callers pass a reader of the LDS copy or of the array in memory, each
// naming its own address space, so that no LDS access goes through a generic
// pointer (a flat access whose base register lies outside the LDS aperture
// faults even when the immediate offset would bring it back inside).
template <int kRowBytes, typename Keep>
__device__ __forceinline__ bool fill_holes(const HeadUnit& u, int kept, Keep keep) {
  constexpr int kPerRow = kRowBytes / 16;
  constexpr int kRowsPerPass = kThreads / kPerRow;
  // c = #{keep[i] < kept}: the entries are ascending, so a binary search.
  int lo = 0, hi = kept;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (keep(mid) < kept) lo = mid + 1; else hi = mid;
  }
  const int c = lo;
  const int movers = kept - c;
  // Sources lie below n, destinations below kept; the head holds
  // max(n, kept + n_append) rows (both bounds are checked in head_unit).
  const uint32_t head_bytes = uint32_t(max(u.n, kept + u.n_append)) * kRowBytes;
  const Buf kb(u.k, head_bytes), vb(u.v, head_bytes);
  const int col = threadIdx.x % kPerRow;
  constexpr int kPasses = kCompactRows / kRowsPerPass;
  static_assert(kPasses * kRowsPerPass == kCompactRows, "whole passes");
  bool bad = false;
  for (int m0 = blockIdx.x * kCompactRows; m0 < movers; m0 += gridDim.x * kCompactRows) {
    // Every pass's source and hole first (LDS searches), then all loads, then
    // all stores: one memory round trip per block instead of one per pass.
    int src[kPasses], hole[kPasses];
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const int j = m0 + int(threadIdx.x) / kPerRow + q * kRowsPerPass;
      src[q] = -1;
      if (j < movers) {
        const int sr = keep(c + j);
        // last i < c with keep[i] - i <= j
        int l = 0, h = c;
        while (l < h) {
          const int mid = (l + h) >> 1;
          if (keep(mid) - mid <= j) l = mid + 1; else h = mid;
        }
        const int ho = j + l;
        if (sr < kept || sr >= u.n || ho >= kept) {
          bad = true;
        } else {
          src[q] = sr;
          hole[q] = ho;
        }
      }
    }
    uint4 xk[kPasses], xv[kPasses];
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      if (src[q] >= 0) {
        xk[q] = kb.ld16<kNonTemporal>(uint32_t(src[q] * kRowBytes + 16 * col));
        xv[q] = vb.ld16<kNonTemporal>(uint32_t(src[q] * kRowBytes + 16 * col));
      }
    }
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      if (src[q] >= 0) {
        kb.st16<kNonTemporal>(uint32_t(hole[q] * kRowBytes + 16 * col), xk[q]);
        vb.st16<kNonTemporal>(uint32_t(hole[q] * kRowBytes + 16 * col), xv[q]);
      }
    }
  }
  return bad;
}

template <int kRowBytes>
__global__ __launch_bounds__(kThreads) void kv_fill_holes_kernel(const Args a) {
  __shared__ int32_t s_keep[kLdsKeep];
  const int hu = blockIdx.y;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid || u.keep == nullptr) return;
  const int b = a.g.block;
  const int kept = min(u.kept * b, u.n);   // kept rows
  // Movers are kept rows at or past kept, so at most n - kept of them; the
  // whole workgroup leaves together.
  if (int(blockIdx.x) * kCompactRows >= u.n - kept) return;
  bool bad;
  if (u.kept <= kLdsKeep) {
    // The searches read the keep array many times: stage it in LDS once.
    // (eight loads per thread in flight per round)
    for (int i0 = threadIdx.x; i0 < u.kept; i0 += 8 * kThreads) {
      int32_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q * kThreads;
        v[q] = i < u.kept ? u.keep[i] : 0;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q * kThreads;
        if (i < u.kept) s_keep[i] = v[q];
      }
    }
    __syncthreads();
    if (b == 1)
      bad = fill_holes<kRowBytes>(u, kept, [](int i) { return s_keep[i]; });
    else
      bad = fill_holes<kRowBytes>(u, kept, [b](int i) { return s_keep[i / b] * b + (i & (b - 1)); });
  } else {
    const int32_t* keep = u.keep;
    if (b == 1)
      bad = fill_holes<kRowBytes>(u, kept, [keep](int i) { return keep[i]; });
    else
      bad = fill_holes<kRowBytes>(u, kept, [keep, b](int i) { return keep[i / b] * b + (i & (b - 1)); });
  }
  if (__syncthreads_or(bad) && threadIdx.x == 0) raise_status(a, kStatusBadItem);
}

template <int kRowBytes>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(const Args a) {
  constexpr int kPerRow = kRowBytes / 16;
  constexpr int kRowsPerPass = kThreads / kPerRow;
  const int hu = blockIdx.y;
  const HeadUnit u = head_unit(a, hu);
  if (!u.valid || u.keep == nullptr) return;
  // Appended rows follow the kept rows (with blocks, n % b == 0 then holds).
  const int kept = min(u.kept * a.g.block, u.n);
  if (blockIdx.x == 0 && threadIdx.x == 0 && u.tokens_out != nullptr) *u.tokens_out = kept + u.n_append;
  if (u.n_append == 0) return;
  const uint32_t head_bytes = uint32_t(kept + u.n_append) * kRowBytes;
  const uint32_t app_bytes = uint32_t(u.n_append) * kRowBytes;
  const Buf kb(u.k, head_bytes), vb(u.v, head_bytes);
  const Buf kab(u.app_k, app_bytes), vab(u.app_v, app_bytes);
  const int col = threadIdx.x % kPerRow;
  constexpr int kPasses = kCompactRows / kRowsPerPass;
  for (int r0 = blockIdx.x * kCompactRows; r0 < u.n_append; r0 += gridDim.x * kCompactRows) {
    uint4 xk[kPasses], xv[kPasses];
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const int r = r0 + int(threadIdx.x) / kPerRow + q * kRowsPerPass;
      if (r < u.n_append) {
        const uint32_t off = uint32_t(r * kRowBytes + 16 * col);
        xk[q] = kab.ld16<kNonTemporal>(off);
        xv[q] = vab.ld16<kNonTemporal>(off);
      }
    }
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const int r = r0 + int(threadIdx.x) / kPerRow + q * kRowsPerPass;
      if (r < u.n_append) {
        const uint32_t off = uint32_t(r * kRowBytes + 16 * col);
        kb.st16<kNonTemporal>(uint32_t(kept * kRowBytes) + off, xk[q]);
        vb.st16<kNonTemporal>(uint32_t(kept * kRowBytes) + off, xv[q]);
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_compact(const Args& a, hipStream_t s) {
  const int max_rows = a.g.max_out_rows > 0 ? a.g.max_out_rows : a.g.max_tokens;
  const dim3 grid((max_rows + kCompactRows - 1) / kCompactRows, a.g.n_hu);
  const int row_bytes = a.g.head_dim * (a.g.dtype == NX_BF16 ? 2 : 4);
#define NX_LAUNCH(K, GRID)                                                                    \
  switch (row_bytes) {                                                                        \
    case 128: hipLaunchKernelGGL(K<128>, GRID, dim3(kThreads), 0, s, a); break;               \
    case 256: hipLaunchKernelGGL(K<256>, GRID, dim3(kThreads), 0, s, a); break;               \
    default: hipLaunchKernelGGL(K<512>, GRID, dim3(kThreads), 0, s, a); break;                \
  }
  if (a.g.inplace) {
    // Movers are at most the kept rows; the appended rows are max_out_rows - kept.
    // Both kernels stride their row blocks by the grid, and in the streaming
    // steady state only a few blocks per head unit hold work (the rows past
    // the kept count): about 2048 workgroups in all, not one per possible row
    // block, whose launch alone cost more than the moves.
    const int per_hu = std::max(1, std::min<int>(grid.x, 2048 / std::max(1, a.g.n_hu)));
    const dim3 g2(per_hu, a.g.n_hu);
    NX_LAUNCH(kv_fill_holes_kernel, g2)
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    NX_LAUNCH(kv_append_kernel, g2)
  } else {
    NX_LAUNCH(kv_compact_kernel, grid)
  }
#undef NX_LAUNCH
  return hipGetLastError();
}

}  // namespace nx
