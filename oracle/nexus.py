"""The Nexus Sampling eviction step, written out in fp64 numpy (test infrastructure).

Every function follows [Nexus] = "Forget Without Compromise: Nexus Sampling for
Streaming KV-Cache Eviction Under Fixed Budgets" (academ.us article page) and
says which passage.  No blocking, fusion or reordering beyond the definitions:
one BLAS matmul for the logits, then elementwise numpy.

Readings of passages the pages leave open:
  granularity  tokens by default, i.e. block size b = 1, so BlockSum_b and
               rownorm of section 2.1 Eq. (1) are identities on softmax rows;
               block = b > 1 scores, samples and keeps blocks of b tokens
               (the last block may be shorter), with the budget, the forced
               slots and the kept indices counted in blocks and the block
               index as the token word of the Philox counter.
  GQA          "head-averaged representations" (section 2.1): for KV head h the
               softmax rows of its G query heads h*G .. h*G+G-1 are averaged,
               per window row, in probability space.
  walk rows    Eq. (4) feeds one fresh window row per step: the H most recent
               rows W-H .. W-1, oldest first; H = 0 gives c~ = 0.
  ramp         Eq. (5) r_j = j/(N-1) with 0-based j (0 oldest, 1 newest);
               r = 0 when N = 1.
  n            Eq. (6) with n = 1 by default, its ordering that of the A-Res
               key ln(u)/w; n > 1 and the n -> infinity limit in head_keys.
  ties         equal keys: the larger (newer) index wins.
  w <= 0       key -inf (kept only when needed to fill B); non-finite w is an
               error.
  forced       the first n_sink and last n_recent positions get key +inf
               (section 2.3, forced slots).
  order        kept indices are returned ascending (cache order).

Pins (tests/test_oracle_nexus.py): the hand-computed tiny cache in
tests/golden/, closed forms (Q = 0 gives a = 1/N; identical rows; H = 1),
the walk's rank-1 decomposition (appendix 8.6), softmax against scipy,
permutation equivariance, and selection laws against exact enumeration
(oracle/enumerate.py) and the uniform-reservoir special case.
"""

import numpy as np

from . import philox

LAMBDA_DEFAULT = 0.5     # [Nexus] section 5.1: mixing weight
EPS_TIE_DEFAULT = 1e-6   # [Nexus] section 5.1: tie-break magnitude


# ----------------------------------------------------------------- inputs ----

def bf16_bits_to_f64(bits):
    """Exact fp64 value of raw bfloat16 bit patterns (uint16 array)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x, dtype):
    """Inputs as exact fp64: dtype 'bf16' means raw uint16 bit patterns."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ------------------------------------------------------------ Nexus score ----

def window_rows(q_grp, k):
    """Per-row distributions a^(q) of the window, averaged over the GQA group.

    [Nexus] section 2.1, Eq. (1): softmax(Q K^T / sqrt(D)) over the cached keys,
    one row per window query; at b = 1 BlockSum and rownorm change nothing.
    q_grp: [G, W, D] fp64 (the G query heads sharing one KV head); k: [N, D].
    Returns P: [W, N], P[w] = (1/G) * sum_i softmax_j(q_{i,w} . k_j / sqrt(D)).
    """
    q_grp = np.asarray(q_grp, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = k.shape[-1]
    logits = np.matmul(q_grp, k.T) / np.sqrt(d)               # [G, W, N]
    shifted = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(shifted)
    p = e / e.sum(axis=-1, keepdims=True)
    return p.mean(axis=0)


def block_rows(P, block):
    """[Nexus] section 2.1, Eq. (1) at block size b: rownorm(BlockSum_b(rows)).

    Block k holds tokens k*b .. min((k+1)*b, N) - 1 (N_k = ceil(N / b) blocks,
    the last one possibly shorter); each row is then divided by its sum.
    P: [W, N] -> [W, N_k].  b = 1 returns the rows renormalised only.
    """
    P = np.asarray(P, dtype=np.float64)
    W, N = P.shape
    nk = -(-N // block)
    pad = np.zeros((W, nk * block))
    pad[:, :N] = P
    S = pad.reshape(W, nk, block).sum(axis=2)
    return S / S.sum(axis=1, keepdims=True)


def direct_score(P):
    """[Nexus] section 2.2, Eq. (3): a = (1/W) sum_q a^(q), the uniform row average."""
    return np.asarray(P, dtype=np.float64).mean(axis=0)


def nexus_walk(P, walk_iters):
    """[Nexus] section 2.2, Eq. (4): the alignment-weighted walk, normalised.

    C starts at 0; each step takes the next window row a^(q) (rows W-H .. W-1,
    oldest first), sets gamma = 1 + <a^(q), C> using C before the update, then
    C <- C + gamma * a^(q).  Returns c~ = C / ||C||_1 (zeros when H = 0).
    """
    P = np.asarray(P, dtype=np.float64)
    W, N = P.shape
    if not 0 <= walk_iters <= W:
        raise ValueError("walk_iters must lie in [0, W]")
    C = np.zeros(N)
    for t in range(W - walk_iters, W):
        row = P[t]
        gamma = 1.0 + float(np.dot(row, C))
        C = C + gamma * row
    if walk_iters == 0:
        return np.zeros(N)
    return C / np.abs(C).sum()


def nexus_score(a, c, lam=LAMBDA_DEFAULT):
    """[Nexus] section 2.2, Eq. (2): s = a + lambda * c~."""
    return np.asarray(a, dtype=np.float64) + lam * np.asarray(c, dtype=np.float64)


def recency_weights(s, eps=EPS_TIE_DEFAULT):
    """[Nexus] section 2.2, Eq. (5): w_j = s_j + eps * r_j with r_j = j/(N-1)."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[-1]
    r = np.arange(n, dtype=np.float64) / (n - 1) if n > 1 else np.zeros(n)
    return s + eps * r


def head_weights(q_grp, k, walk_iters, lam=LAMBDA_DEFAULT, eps=EPS_TIE_DEFAULT, block=1):
    """All scoring stages for one KV head; returns a dict of the intermediates.
    block > 1 scores blocks of that many tokens (Eq. 1's BlockSum_b, rownorm)."""
    P = window_rows(q_grp, k)
    if block > 1:
        P = block_rows(P, block)
    a = direct_score(P)
    c = nexus_walk(P, walk_iters)
    s = nexus_score(a, c, lam)
    w = recency_weights(s, eps)
    return {"P": P, "a": a, "c": c, "s": s, "w": w}


# ------------------------------------------------------- reservoir select ----

def reservoir_keys(w, u, n_sink=0, n_recent=0):
    """Reservoir keys for one KV head; [Nexus] section 2.3, Eq. (6).

    u: [N] (one draw per token, n = 1) or [N, n].  The priority is
    pi_j = (1/n) sum_i u_ji^(1/w_j); the key is ln(pi_j), which orders the
    tokens the same way.  For n = 1 that is ln(u)/w (A-Res).  For n > 1 the
    sum is taken in the log domain, ln pi = logsumexp_i(ln(u_ji)/w_j) - ln n,
    because u^(1/w) underflows fp64 for the small weights of long caches.
    All in fp64.  w <= 0 gives -inf; the forced sink / recency positions
    (section 2.3) get +inf so that they always survive.
    """
    w = np.asarray(w, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite Nexus weight")
    n = w.shape[-1]
    pos = w > 0
    keys = np.full(n, -np.inf)
    if u.ndim == 1:
        keys[pos] = np.log(u[pos]) / w[pos]
    else:
        t = np.log(u[pos]) / w[pos][:, None]          # ln(u_ji^(1/w_j))
        m = t.max(axis=1)
        keys[pos] = m + np.log(np.exp(t - m[:, None]).sum(axis=1)) - np.log(u.shape[1])
    if n_sink:
        keys[:n_sink] = np.inf
    if n_recent:
        keys[n - n_recent:] = np.inf
    return keys


def topk_keys(w, n_sink=0, n_recent=0):
    """Keys of the deterministic limit n -> infinity of Eq. (6).

    [Nexus] appendix 8.2: the n-averaged priority tends to E[u^(1/w)] =
    w/(w+1), increasing in w, so the limit ranks by w itself: key = w (w > 0),
    -inf otherwise, +inf at the forced positions.
    """
    w = np.asarray(w, dtype=np.float64)
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite Nexus weight")
    n = w.shape[-1]
    keys = np.where(w > 0, w, -np.inf)
    if n_sink:
        keys[:n_sink] = np.inf
    if n_recent:
        keys[n - n_recent:] = np.inf
    return keys


def head_keys(w, n_tokens, unit_id, layer, step, seed, n_avg, n_sink=0, n_recent=0):
    """Keys of one KV head for averaging count n_avg: 0 or 1 -> n = 1,
    n >= 2 -> n draws, -1 -> the deterministic limit (top-B by w)."""
    if n_avg == -1:
        return topk_keys(w, n_sink, n_recent)
    if n_avg in (0, 1):
        u = unit_uniforms(n_tokens, unit_id, layer, step, seed)
    elif n_avg >= 2:
        j = np.arange(n_tokens, dtype=np.uint64)
        u = philox.uniforms_n(j, unit_id, layer, step, seed, n_avg)
    else:
        raise ValueError("n_avg must be -1, 0 or >= 1")
    return reservoir_keys(w, u, n_sink, n_recent)


def select_top(keys, budget):
    """Keep the `budget` largest keys; [Nexus] section 2.3 (keep the top K).

    Equal keys: the larger index wins.  budget >= N keeps everything.
    Returns the kept indices in ascending (cache) order.
    """
    keys = np.asarray(keys, dtype=np.float64)
    n = keys.shape[-1]
    if budget >= n:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), keys))   # ascending by key, then index
    return np.sort(order[n - budget:])


def unit_uniforms(n_tokens, unit_id, layer, step, seed):
    """The token uniforms of one KV head for one eviction event."""
    j = np.arange(n_tokens, dtype=np.uint64)
    return philox.uniforms(j, unit_id, layer, step, seed)


# ------------------------------------------------------------ whole step ----

def evict_step(q, k, v, budget, walk_iters, seed, *, dtype="bf16", layer=0,
               step=0, seq_id=0, lam=LAMBDA_DEFAULT, eps=EPS_TIE_DEFAULT,
               n_sink=0, n_recent=0, heads=None, n_avg=1, block=1, head_budgets=None,
               ada_floor=None, head_cap=None):
    """One eviction event for one (sequence, layer): every KV head.

    [Nexus] section 2.1 (streaming view): keep `budget` of the N resident
    positions per KV head and continue with the kept K and V rows.
    q: [H_q, W, D]; k, v: [H_kv, N, D] (raw bf16 bits when dtype == 'bf16').
    Query head g reads KV head g // G.  `heads` restricts the work to a
    subset of KV heads (results for the others are left out).  n_avg: the
    priority averaging count of Eq. (6), see head_keys.  block = b > 1: the
    units scored, sampled and kept are blocks of b tokens (section 2.1); then
    budget, n_sink and n_recent count blocks, keep holds block indices, and
    out_k / out_v are the rows of the kept blocks in ascending block order.
    Per-head budgets (appendix 10): head_budgets gives head h's kept count;
    ada_floor = f (not None) computes them with ada_head_budgets from the
    weights of all heads (capacity head_cap, default budget).  k and v may
    also be lists of per-head [N_h, D] arrays: after per-head budgets the
    heads of a streaming cache hold different numbers of rows.
    Returns dict with per-head lists: w, keys, keep (ascending), out_k, out_v,
    and "budgets" (the per-head kept counts used).
    """
    q = np.asarray(q)
    k = [np.asarray(x) for x in k]
    v = [np.asarray(x) for x in v]
    h_q, W, d = q.shape
    h_kv = len(k)
    if len(v) != h_kv or any(len(kh) != len(vh) for kh, vh in zip(k, v)):
        raise ValueError("k and v must hold the same rows")
    if h_kv == 0 or h_q % h_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    if budget < 1 or min(len(x) for x in k) < 1:
        raise ValueError("budget and n_tokens must be >= 1")
    if n_sink + n_recent > budget:
        raise ValueError("forced slots exceed the budget")
    if block < 1:
        raise ValueError("block must be >= 1")
    g = h_q // h_kv
    heads = range(h_kv) if heads is None else heads
    out = {"w": {}, "keys": {}, "keep": {}, "out_k": {}, "out_v": {}, "budgets": {}}
    weights = {}
    for h in (range(h_kv) if ada_floor is not None else heads):
        q_grp = as_f64(q[h * g:(h + 1) * g], dtype)
        weights[h] = head_weights(q_grp, as_f64(k[h], dtype), walk_iters, lam, eps, block)["w"]
    if ada_floor is not None:
        head_budgets = ada_head_budgets([weights[h] for h in range(h_kv)], budget, ada_floor,
                                        budget if head_cap is None else head_cap)
    for h in heads:
        w = weights[h]
        nu = w.shape[-1]
        n = len(k[h])
        b_h = budget if head_budgets is None else int(head_budgets[h])
        if n_sink + n_recent > b_h:
            raise ValueError("forced slots exceed the head's budget")
        keys = head_keys(w, nu, seq_id * h_kv + h, layer, step, seed, n_avg, n_sink,
                         n_recent)
        keep = select_top(keys, b_h)
        rows = np.concatenate([np.arange(b * block, min((b + 1) * block, n)) for b in keep])
        out["w"][h] = w
        out["keys"][h] = keys
        out["keep"][h] = keep
        out["budgets"][h] = b_h
        out["out_k"][h] = k[h][rows]
        out["out_v"][h] = v[h][rows]
    return out


def select_from_weights(w, budget, seed, *, layer=0, step=0, seq_id=0,
                        n_sink=0, n_recent=0, n_avg=1, head_budgets=None):
    """Reservoir selection on given weights w: [H_kv, N] (any precision), or a
    list of per-head weight vectors of their own lengths.

    The oracle run on someone else's scores: same Philox stream, fp64 keys,
    full sort.  Returns (keys: [H_kv, N], or a list for ragged heads; list of
    ascending keep arrays).
    """
    rows = [np.asarray(x, dtype=np.float64).ravel() for x in w]
    h_kv = len(rows)
    ragged = len({len(x) for x in rows}) > 1
    keys = [None] * h_kv
    keeps = []
    for h in range(h_kv):
        keys[h] = head_keys(rows[h], len(rows[h]), seq_id * h_kv + h, layer, step, seed, n_avg,
                            n_sink, n_recent)
        keeps.append(select_top(keys[h], budget if head_budgets is None else
                                int(head_budgets[h])))
    return (keys if ragged else np.stack(keys)), keeps


# ------------------------------------------------- per-head budgets ----

def ada_head_budgets(w, budget, floor, cap=None):
    """Per-head budgets of one item: [Nexus] appendix 10 layers the
    head-adaptive allocation of Ada-KV (its reference [12]) on a score: a fixed
    budget for the layer, redistributed over its heads.  The pages give only
    that aim; this is the allocation of Ada-KV itself, a top-K over the
    scores of all heads together, on the Nexus weights, with a per-head floor:

      N_h = head h's units, Bbar = min(budget, max_h N_h), f = min(floor, Bbar),
      K = H (Bbar - f);
      order all (head h, unit j) by weight, largest first (weights <= 0 all
      count as 0), equal weights: the smaller head first;
      c_h = how many of the first K belong to head h;
      B_h = min(f + c_h, cap, N_h)   (cap: the per-head capacity, default budget).

    w: [H, N] weights of the item's KV heads (any precision), or a list of H
    per-head weight vectors of their own lengths N_h (a streaming cache after
    earlier per-head budgets: each head holds its own number of rows).
    Returns int64 [H].
    """
    rows = [np.asarray(x, dtype=np.float64).ravel() for x in w]
    h_kv = len(rows)
    sizes = np.array([len(x) for x in rows], dtype=np.int64)
    if budget < 1 or floor < 0:
        raise ValueError("budget must be >= 1 and floor >= 0")
    if h_kv == 0 or sizes.min() < 1:
        raise ValueError("every head needs at least one unit")
    if not all(np.all(np.isfinite(x)) for x in rows):
        raise ValueError("non-finite Nexus weight")
    cap = budget if cap is None else cap
    bbar = min(budget, int(sizes.max()))
    f = min(floor, bbar)
    k = h_kv * (bbar - f)
    val = np.concatenate([np.where(x > 0, x, 0.0) for x in rows])
    head = np.repeat(np.arange(h_kv), sizes)
    order = np.lexsort((head, -val))          # weight descending, then head ascending
    counts = np.bincount(head[order[:k]], minlength=h_kv)
    return np.minimum(np.minimum(f + counts, cap), sizes).astype(np.int64)


# ------------------------------------------------- in-place compaction ----

def inplace_layout(keep, n_tokens):
    """Where each kept row lands when the cache is compacted in place.

    [Nexus] section 2.1 continues with K_S, V_S; attention does not depend on
    the order of the cached rows once positions are encoded in K, so only the
    kept rows at or past position `kept` (= len(keep)) must move: the j-th of
    them (ascending) fills the j-th evicted position below `kept`
    (ascending).  Returns new_pos [len(keep)]: the new row of keep[i].
    """
    keep = np.asarray(keep, dtype=np.int64)
    kept = len(keep)
    stay = keep < kept
    holes = np.setdiff1d(np.arange(kept), keep[stay])
    movers = keep[~stay]
    if len(holes) != len(movers):
        raise AssertionError("holes and movers must pair up")
    new_pos = keep.copy()
    new_pos[~stay] = holes
    return new_pos


def compact_inplace(cache, keep, appended=None):
    """The cache after in-place compaction of one head: cache [N, D] (a copy is
    returned), keep ascending; appended rows, if any, go to kept, kept+1, ..."""
    out = np.array(cache, copy=True)
    keep = np.asarray(keep, dtype=np.int64)
    kept = len(keep)
    new_pos = inplace_layout(keep, cache.shape[0])
    moved = new_pos != keep
    out[new_pos[moved]] = np.asarray(cache)[keep[moved]]
    if appended is not None and len(appended):
        out[kept:kept + len(appended)] = appended
    return out
