/*
 * nexus.h -- C ABI of the Nexus Sampling eviction step for AMD Instinct MI355X (gfx950).
 *
 * The method ([Nexus]): "Forget Without Compromise: Nexus Sampling for Streaming
 * KV-Cache Eviction Under Fixed Budgets" (academ.us article page).  One eviction
 * event keeps B of the N resident positions of every KV head and continues with
 * the kept K and V rows (section 2.1, streaming view).  The kept set is drawn by
 * weighted reservoir sampling (section 2.3, Eq. 6) on the Nexus weight
 * w = a + lambda * c~ + eps * r (section 2.2, Eqs. 2-5), where a is the direct
 * attention of a window of W recent queries (section 2.1, Eq. 1; section 2.2,
 * Eq. 3) and c~ the normalised alignment-weighted walk over the same rows
 * (section 2.2, Eq. 4).
 *
 * Granularity is one token (block size b = 1), the reservoir uses one uniform
 * per token (n = 1) and the A-Res key ln(u)/w in fp64.  The uniform comes from
 * Philox4x32-10 (Salmon et al., SC'11) with counter
 * (token, seq_id * n_kv_heads + kv_head, layer, step) and key (seed lo, seed hi):
 * u = ((((x0 << 32) | x1) >> 11) + 1) * 2^-53 in (0, 1].
 * Equal keys: the larger (newer) token index wins.  Kept indices are ascending.
 *
 * Conventions for every entry point:
 *  - Buffers are device memory owned by the caller (for example torch tensors).
 *    The library allocates nothing and keeps no per-call state outside the
 *    caller's workspace.
 *  - Work is enqueued on desc->stream (a hipStream_t; NULL = legacy default
 *    stream) and the call returns at once.  Calls that share a workspace must
 *    be ordered on one stream.
 *  - Host-side argument errors return a negative nx_status before anything is
 *    enqueued.  Errors only the device can see (a non-finite weight, an invalid
 *    batch item) are recorded in a status word inside the workspace and
 *    reported by nx_read_device_status().
 *  - Layouts are row-major.  Q window: [n_q_heads, window, head_dim], row 0 the
 *    oldest query; query head g reads KV head g / (n_q_heads / n_kv_heads).
 *    K and V caches: [n_kv_heads][kv_head_stride elements], each head holding
 *    [n_tokens, head_dim] rows.  Outputs: keep indices [n_kv_heads, budget]
 *    (int32), out_k / out_v [n_kv_heads][out_head_stride elements] holding
 *    [kept, head_dim] rows, kept = min(budget, n_tokens).
 *  - Element types: NX_BF16 (bfloat16) or NX_F32, shared by Q, K, V and the
 *    outputs; head_dim 64 or 128.
 *  - Debugging: with the environment variable NX_DEBUG set to a non-empty value
 *    other than "0" (read at every call), each call is synchronous -- after
 *    every kernel stage the stream is synchronised and the HIP error state and
 *    the device status word are checked; the first failure is returned by the
 *    call itself (NX_EHIP, NX_ENONFINITE, NX_EINVAL) and the stage named on
 *    stderr.  The checks are skipped while desc->stream is being captured.
 */
#ifndef NEXUS_H
#define NEXUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nx_status;
enum {
  NX_OK = 0,
  NX_EINVAL = -1,        /* bad argument (null pointer, size, budget, walk depth) */
  NX_EALIAS = -2,        /* an output overlaps an input */
  NX_EWORKSPACE = -3,    /* workspace missing or smaller than nx_evict_workspace_bytes() */
  NX_EUNSUPPORTED = -4,  /* dtype / head_dim / group size outside the built kernels */
  NX_ENONFINITE = -5,    /* device: a Nexus weight was NaN or infinite */
  NX_EHIP = -6           /* a HIP runtime call failed */
};

enum { NX_BF16 = 0, NX_F32 = 1 };

/* Problem shape and parameters shared by the calls of one eviction event. */
typedef struct nx_desc {
  int32_t n_q_heads;        /* H_q, a multiple of n_kv_heads */
  int32_t n_kv_heads;       /* H_kv */
  int32_t head_dim;         /* D: 64 or 128 */
  int32_t window;           /* W >= 1: recent queries scored against the cache (section 2.1) */
  int32_t dtype;            /* NX_BF16 or NX_F32 */
  float lambda;             /* mixing weight of Eq. 2 (0.5 in section 5.1) */
  float eps_tie;            /* recency tie-break of Eq. 5 (1e-6 in section 5.1) */
  int32_t n_sink;           /* leading positions always kept (section 2.3, forced slots) */
  int32_t n_recent;         /* trailing positions always kept (section 2.3, forced slots) */
  uint32_t layer;           /* Philox counter word 2 */
  uint32_t step;            /* Philox counter word 3 (eviction event number) */
  uint32_t seq_id;          /* sequence number for Philox counter word 1 (single-item calls) */
  int32_t max_out_rows;     /* batch calls: expected max of kept + n_append over the items;
                               sizes the compaction grid only (any value is correct, a
                               close bound is fastest); 0 means max_tokens */
  int64_t kv_head_stride;   /* elements between KV heads in k/v; 0 means n_tokens * head_dim */
  int64_t out_head_stride;  /* elements between KV heads in out_k/out_v; 0 means budget * head_dim
                               (budget * block * head_dim with blocks) */
  void* workspace;          /* device scratch, >= nx_evict_workspace_bytes(); zero-filled once
                               before first use and not modified by the caller afterwards */
  size_t workspace_bytes;
  void* stream;             /* hipStream_t */
  int32_t n_avg;            /* priority averaging count n of section 2.3 Eq. 6:
                               0 or 1: one draw per token, the key ln(u)/w (A-Res);
                               2 .. NX_MAX_AVG: pi = (1/n) sum_i u_i^(1/w), key ln(pi);
                               NX_TOPK (-1): the deterministic n -> infinity limit of
                               appendix 8.2, the B largest weights (key w);
                               anything else: NX_EINVAL */
  int32_t block;            /* units of selection (section 2.1, Eq. 1): 0 or 1 = tokens; b = 2, 4,
                               8, 16 or 32 = blocks of b consecutive tokens (the last block of a
                               head may be shorter), scored by BlockSum_b of the attention rows.
                               With b > 1 the budget, n_sink and n_recent count blocks, keep
                               indices are block indices, weight / key arrays hold
                               ceil(n_tokens / b) entries per head, and the compacted rows are
                               the kept blocks' rows in ascending block order (out_head_stride
                               >= budget * b rows; items with appended rows need n_tokens % b
                               == 0).  Other values: NX_EUNSUPPORTED. */
  int32_t compact;          /* NX_COMPACT_COPY (0): kept rows copied in ascending order to
                               out_k / out_v.  NX_COMPACT_INPLACE (1): k / v themselves are
                               compacted (section 2.1 continues with K_S, V_S; attention does
                               not depend on row order once positions are in K): the kept
                               rows at or past position kept move, the j-th of them
                               (ascending) into the j-th evicted slot below kept, and the
                               appended rows go to kept, kept + 1, ...; out_k / out_v must be
                               NULL and kv_head_stride must hold kept + n_append rows.  With
                               blocks the same holds for the kept blocks' rows (row i of the
                               kept rows is row i % b of block keep[i / b]), so aligned blocks
                               move whole.  Other values: NX_EINVAL. */
  int32_t head_alloc;       /* per-head budgets (appendix 10: a layer budget shared unevenly by
                               the heads), nx_evict_batch and nx_head_budgets only:
                               NX_HEADS_UNIFORM (0): every head keeps min(budget, units).
                               NX_HEADS_GIVEN (1): head h of an item keeps
                               min(head_budget[h], units) units, 1 <= head_budget[h] <= cap.
                               NX_HEADS_ALLOC (2): the library writes head_budget[h] =
                               min(f + c_h, cap, units), f = min(head_floor, Bbar),
                               Bbar = min(budget, units), c_h = the number of head h's units
                               among the n_kv_heads * (Bbar - f) largest Nexus weights of all
                               heads of the item (weights <= 0 count as 0; equal weights: the
                               lower head first), the head-adaptive rule of Ada-KV that
                               appendix 10 cites; then every head keeps its allocation.
                               With 1 or 2: cap = the item's head_cap (0: budget), keep rows
                               hold cap entries (entries past a head's kept count are set to
                               -1), out_head_stride >= cap rows (cap * block with blocks) plus
                               n_append (appended rows follow each head's own kept rows: the
                               decode regime, with nx_unit.head_tokens / head_tokens_out
                               carrying the per-head counts to the next event), and
                               head_budget must be non-NULL.  With per-head resident counts
                               the allocation takes Bbar = min(budget, the largest head's
                               units) and counts the largest weights over all heads' units;
                               each allocation is capped by its own head's units.  A
                               violation on the device marks the item bad.  Other values:
                               NX_EINVAL; nx_evict_step, nx_reservoir_select and
                               nx_kv_compact need 0. */
  int32_t head_floor;       /* NX_HEADS_ALLOC: per-head floor f >= 0 (units); an allocation
                               below n_sink + n_recent marks the item bad */
  float* out_w;             /* nx_evict_step only, nullable: [n_kv_heads][units] fp32 (units =
                               ceil(n_tokens / block), row stride units), written with the Nexus
                               weights w of section 2.2 Eq. 5 exactly as the selection of this call
                               used them, so that a caller can re-run the reservoir of section 2.3
                               on them; must not overlap any other buffer of the call */
} nx_desc;

#define NX_COMPACT_COPY 0
#define NX_COMPACT_INPLACE 1

#define NX_HEADS_UNIFORM 0
#define NX_HEADS_GIVEN 1
#define NX_HEADS_ALLOC 2
#define NX_MAX_ALLOC_HEADS 256   /* n_kv_heads limit of NX_HEADS_ALLOC */

#define NX_MAX_AVG 64
#define NX_TOPK (-1)

/*
 * One (sequence, layer) item of a batched eviction event.  An array of these
 * lives in DEVICE memory for nx_evict_batch.  Field meanings match
 * nx_evict_step; app_k / app_v (nullable) are n_append new K / V rows per KV
 * head ([n_kv_heads][n_append * head_dim], contiguous) written right after the
 * kept rows, so that a streaming cache is compacted and extended in one pass
 * (the append-then-evict loop of section 2.1).  out_head_stride must then
 * hold kept + n_append rows, and those rows of one KV head must span less
 * than 2^31 bytes.  An item that breaks a rule here is skipped and sets the
 * bad-item bit of the device status (NX_EINVAL from nx_read_device_status).
 */
typedef struct nx_unit {
  const void* q;
  const void* k;
  const void* v;
  int32_t* keep;
  void* out_k;
  void* out_v;
  const void* app_k;
  const void* app_v;
  int64_t kv_head_stride;   /* elements; must be >= n_tokens * head_dim */
  int64_t out_head_stride;  /* elements; must be >= (kept + n_append) * head_dim */
  int32_t n_tokens;
  int32_t budget;
  int32_t n_append;
  uint32_t layer;
  uint32_t seq_id;
  int32_t head_cap;         /* per-head capacity with desc->head_alloc != 0 (0: budget) */
  int32_t* head_budget;     /* [n_kv_heads] int32 device array with desc->head_alloc != 0:
                               read (NX_HEADS_GIVEN) or written (NX_HEADS_ALLOC); else ignored */
  float* out_w;             /* nullable: [n_kv_heads][units] fp32 (units = ceil(n_tokens_h / block)
                               of each head, row stride as for n_tokens), the Nexus weights w
                               (section 2.2 Eq. 5) the item's selection used */
  const int32_t* head_tokens;   /* nullable: [n_kv_heads] int32 device array of per-head resident
                               counts 1 <= n_tokens_h <= n_tokens (after per-head budgets the
                               heads of a streaming cache hold different numbers of rows);
                               NULL: every head holds n_tokens.  n_tokens bounds them (strides,
                               max_tokens); with blocks and appended rows each must be a multiple
                               of the block size */
  int32_t* head_tokens_out; /* nullable: [n_kv_heads] int32, written with each head's row count
                               after the event (kept rows + n_append), the head_tokens of the next
                               event; must not overlap head_tokens */
} nx_unit;

/*
 * Workspace bytes for calls with up to `max_units` items (1 for single-item
 * calls) of up to `max_tokens` tokens each and walk depth `walk_iters`.
 * Returns 0 if desc is invalid.  Pure host function.
 */
size_t nx_evict_workspace_bytes(const nx_desc* desc, int32_t max_tokens, int32_t max_units,
                                int32_t walk_iters);

/*
 * One eviction event for one (sequence, layer): score every resident token of
 * every KV head against the query window (section 2.1 Eq. 1, section 2.2
 * Eqs. 2-5), draw exactly min(budget, n_tokens) tokens per KV head by the A-Res
 * reservoir (section 2.3 Eq. 6, n = 1), and gather their K and V rows
 * (section 2.1: inference continues with the kept rows).
 *   q_window     [n_q_heads, window, head_dim]
 *   k_cache      [n_kv_heads][kv_head_stride]; v_cache likewise
 *   n_tokens     N >= 1 resident tokens per head
 *   budget       B >= 1 kept tokens per head (B >= N keeps all)
 *   walk_iters   H in [0, window] (H > window: NX_EINVAL): the H most recent window
 *                rows, oldest first, feed the walk (section 2.2 Eq. 4); H = 0 gives
 *                plain direct attention.  Built for H <= 64; above 8 (or above 64
 *                walk rows G * H) only with G = n_q_heads / n_kv_heads <= 32, where
 *                the walk rows take a separate Gram pass; other shapes:
 *                NX_EUNSUPPORTED
 *   seed         64-bit Philox key
 *   out_keep_idx [n_kv_heads, budget] int32, ascending; entries past `kept` untouched
 *   out_k, out_v [n_kv_heads][out_head_stride], must not overlap k_cache / v_cache;
 *                NULL with desc->compact == NX_COMPACT_INPLACE, which compacts k_cache
 *                and v_cache themselves (the caches are then written)
 * Errors: NX_EINVAL, NX_EALIAS, NX_EWORKSPACE, NX_EUNSUPPORTED, NX_EHIP.
 */
nx_status nx_evict_step(const nx_desc* desc, const void* q_window, const void* k_cache,
                        const void* v_cache, int32_t n_tokens, int32_t budget,
                        int32_t walk_iters, uint64_t seed, int32_t* out_keep_idx,
                        void* out_k, void* out_v);

/*
 * nx_evict_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels as nx_evict_step, but desc->workspace / workspace_bytes are
 * ignored: the scratch is a static device array of NX_SCRATCH_BYTES inside
 * the library, one per GPU, held until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipEventCreate; the stage profiler is off for it).
 * The caller still passes every input and output, as for nx_evict_step.
 *  - Shapes whose workspace (nx_evict_workspace_bytes with max_units = 1)
 *    exceeds NX_SCRATCH_BYTES return NX_EWORKSPACE before anything is enqueued
 *    (16 MiB holds, for example, 8 KV heads x 32768 tokens at walk depth 8).
 *  - The first call on a device looks up the array's address and clears its
 *    status word with a small kernel on desc->stream: make it outside graph
 *    capture.  nx_read_device_status with desc->workspace == NULL reads (and
 *    clears) that status word on the current device.
 *  - Every call on one GPU uses the same array, which keeps the last call's
 *    contents: calls that overlap in time on one GPU (other streams, other
 *    threads) race and must be serialised by the caller.
 * Errors: those of nx_evict_step, NX_EWORKSPACE as above, NX_EHIP when the
 * set-up fails.
 */
#define NX_SCRATCH_BYTES (16u << 20)

nx_status nx_evict_step_noalloc(const nx_desc* desc, const void* q_window, const void* k_cache,
                                const void* v_cache, int32_t n_tokens, int32_t budget,
                                int32_t walk_iters, uint64_t seed, int32_t* out_keep_idx,
                                void* out_k, void* out_v);

/*
 * The same event for `n_units` (sequence, layer) items in one launch per stage
 * (all layers of a model, or ragged sequences).  units_dev points to n_units
 * nx_unit records in device memory; desc supplies the shared shape, lambda,
 * eps_tie, forced slots, step and workspace (its seq_id, layer and strides are
 * ignored: each item carries its own).  max_tokens bounds every item's
 * n_tokens.  Items are checked on the device; a bad item is skipped and
 * reported as NX_EINVAL by nx_read_device_status().
 */
nx_status nx_evict_batch(const nx_desc* desc, const nx_unit* units_dev, int32_t n_units,
                         int32_t max_tokens, int32_t walk_iters, uint64_t seed);

/*
 * Scoring stage only: the Nexus weights w (section 2.2 Eq. 5) of every resident
 * token, out_w [n_kv_heads, n_tokens] fp32.
 */
nx_status nx_nexus_weights(const nx_desc* desc, const void* q_window, const void* k_cache,
                           int32_t n_tokens, int32_t walk_iters, float* out_w);

/*
 * Reservoir stage only (section 2.3 Eq. 6, n = 1) on given weights
 * w [n_kv_heads, n_tokens] fp32: Philox uniforms, fp64 keys ln(u)/w (w <= 0 gives
 * -inf, forced slots +inf), and the top-budget selection.
 *   out_keep_idx [n_kv_heads, budget] int32 ascending
 *   out_keys     nullable; [n_kv_heads, n_tokens] fp64 keys
 */
nx_status nx_reservoir_select(const nx_desc* desc, const float* w, int32_t n_tokens,
                              int32_t budget, uint64_t seed, int32_t* out_keep_idx,
                              double* out_keys);

/*
 * Per-head allocation only (desc->head_alloc == NX_HEADS_ALLOC, appendix 10) on
 * given weights w [n_kv_heads, n_tokens] fp32 of one item: writes
 * out_head_budget [n_kv_heads] int32 (device) by the rule under nx_desc.head_alloc
 * with layer budget `budget` per head and capacity head_cap (0: budget).
 * n_kv_heads <= NX_MAX_ALLOC_HEADS.  Errors: NX_EINVAL, NX_EWORKSPACE,
 * NX_EUNSUPPORTED, NX_EHIP.
 */
nx_status nx_head_budgets(const nx_desc* desc, const float* w, int32_t n_tokens, int32_t budget,
                          int32_t head_cap, int32_t* out_head_budget);

/*
 * Compaction stage only (section 2.1: continue with K_S, V_S): bit copies
 * out_k[h, r] = k[h, keep_idx[h, r]] and likewise for V, r < min(budget, n_tokens).
 * keep_idx entries must lie in [0, n_tokens).
 */
nx_status nx_kv_compact(const nx_desc* desc, const void* k_cache, const void* v_cache,
                        const int32_t* keep_idx, int32_t n_tokens, int32_t budget,
                        void* out_k, void* out_v);

/*
 * Waits for desc->stream, reads and clears the workspace status word (with
 * desc->workspace == NULL: the status word of nx_evict_step_noalloc's static
 * scratch on the current device).  Returns NX_OK, NX_ENONFINITE or NX_EINVAL
 * (a bad batch item), or NX_EHIP if a HIP call failed.
 */
nx_status nx_read_device_status(const nx_desc* desc);

/* Human-readable name of a status code.  Pure host function. */
const char* nx_status_str(nx_status status);

/*
 * Read-bandwidth probe (a measurement aid, not part of an eviction event): reads
 * `bytes` bytes at `src` (device memory, 16-B aligned, bytes a multiple of 256)
 * `passes` times, one kernel launch per pass, on `stream` (a hipStream_t), with
 * the score sweeps' access pattern: 256-B rows, up to 512 KB per workgroup (less for
 * small buffers, which still get >= 2048 workgroups when they hold >= 64K rows).
 *   mode 0: global -> LDS copies through the sweeps' ring of LDS slots
 *   mode 1: plain 16-byte vector loads into registers
 * sink: >= 1 KB of device memory that the kernels may write (it keeps the loads
 * live; nothing is written unless the XOR of all data hits a fixed value).
 * Errors: NX_EINVAL, NX_EUNSUPPORTED (more than 2^22 * 65535 rows), NX_EHIP.
 */
nx_status nx_stream_read(const void* src, size_t bytes, int32_t mode, int32_t passes, void* sink,
                         void* stream);

/*
 * Per-stage timing with HIP events recorded on desc->stream around the
 * kernel launches of later calls (process-wide; not thread-safe).
 * nx_profile_enable(mask) with mask != 0 clears the records and starts
 * recording around the stages whose bit (1 << stage index) is set in mask
 * (-1: every stage); nx_profile_enable(0) stops.  Each recorded launch adds
 * two event records to the stream, so a timed loop that needs one kernel's
 * duration should record that stage only.
 * nx_profile_read waits for the recorded events and fills, per stage index,
 * the summed milliseconds and the launch count; returns the number of stages.
 */
nx_status nx_profile_enable(int32_t stage_mask);
int32_t nx_profile_read(float* stage_ms, int32_t* stage_launches, int32_t max_stages);
const char* nx_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* NEXUS_H */
