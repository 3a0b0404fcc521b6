"""Long-run survival of tokens under streaming eviction (test infrastructure).

Only tests, the smoke check and the CPU baseline of the benchmark use this
module; the library never does.

[Nexus] = "Forget Without Compromise: Nexus Sampling for Streaming KV-Cache
Eviction Under Fixed Budgets" (academ.us article page).  Section 3 argues
that under deterministic top-K a token survives e events only if it clears
the cutoff at every one of them, while under the weighted reservoir its
survival is a product of per-event inclusion probabilities, each positive
when its weight is (appendix 8.3, Lemma 1).  This module computes both for
small streams whose weights are given per (event, token):

* kept_set_law: the law of the kept set of one event under successive
  sampling (the law of keeping the K largest u^(1/w), section 2.3), by
  enumerating ordered prefixes, in exact rationals;
* reservoir_survival_exact: the survival probability of every token after
  every event of a stream, by summing over all resident-set paths;
* topk_survival: the same stream under deterministic top-K by weight;
* reservoir_survival_mc: the stream run with the oracle's own Philox keys,
  one replica per KV-head counter, so that a device run on the same seeds
  follows the same paths.

A stream: the cache starts with tokens 0 .. n0-1 in cache order; at event e
every resident token j has weight weight_of(e, j) > 0, the kept tokens stay
in cache order and `n_append` new tokens (the next ids) follow them.

Pinned in tests/test_oracle_survival.py (hand-computed set law, equal-weight
closed form (B/N)^e, budget 1, an independent top-K formulation, Monte Carlo
against the exact law, Lemma 1's positivity and collapse).
"""

from collections import defaultdict
from fractions import Fraction
from itertools import permutations

import numpy as np

from . import nexus


def _frac(x):
    return x if isinstance(x, Fraction) else Fraction(float(x))


def kept_set_law(weights, budget):
    """{frozenset of positions: probability} for one event (N <= 8, w > 0).

    Successive sampling: the next kept position is drawn with probability
    proportional to its weight among those not yet drawn; the kept set is
    the set of the first `budget` draws.
    """
    w = [_frac(x) for x in weights]
    n = len(w)
    if n > 8:
        raise ValueError("enumeration is meant for N <= 8")
    if any(x <= 0 for x in w):
        raise ValueError("the exact law needs positive weights")
    if budget >= n:
        return {frozenset(range(n)): Fraction(1)}
    law = defaultdict(Fraction)
    total = sum(w)
    for prefix in permutations(range(n), budget):
        p = Fraction(1)
        left = total
        for i in prefix:
            p *= w[i] / left
            left -= w[i]
        law[frozenset(prefix)] += p
    return dict(law)


def reservoir_survival_exact(weight_of, n0, budget, n_append, events):
    """alive[e][j] = P(token j resident after event e), exact, e = 0 .. events-1.

    The state is the distribution over resident id tuples (cache order); each
    event maps every tuple through kept_set_law and appends the new ids.
    """
    dist = {tuple(range(n0)): Fraction(1)}
    next_id = n0
    alive_by_event = []
    for e in range(events):
        arrived = tuple(range(next_id, next_id + n_append))
        nxt = defaultdict(Fraction)
        for res, p in dist.items():
            law = kept_set_law([weight_of(e, j) for j in res], budget)
            for kept, q in law.items():
                nxt[tuple(res[i] for i in sorted(kept)) + arrived] += p * q
        next_id += n_append
        dist = dict(nxt)
        alive = defaultdict(Fraction)
        for res, p in dist.items():
            for j in res:
                alive[j] += p
        alive_by_event.append(dict(alive))
    return alive_by_event


def topk_survival(weight_of, n0, budget, n_append, events):
    """Resident id sets after each event under deterministic top-K by weight
    (ties: the later cache position wins, as in the reservoir's tie rule)."""
    res = list(range(n0))
    next_id = n0
    out = []
    for e in range(events):
        w = np.array([float(weight_of(e, j)) for j in res])
        keep = nexus.select_top(nexus.topk_keys(w), budget)
        res = [res[i] for i in keep] + list(range(next_id, next_id + n_append))
        next_id += n_append
        out.append(set(res))
    return out


def reservoir_survival_mc(weight_of, n0, budget, n_append, events, replicas, seed,
                          first_step=0):
    """Resident ids [replicas, n] after each event, sampled with the oracle's keys.

    Replica r uses the Philox counter of KV head r of sequence 0, layer 0, at
    step first_step + e: the counter a device selection over `replicas` heads
    uses.  Returns a list of int64 arrays, one per event.
    """
    res = np.tile(np.arange(n0, dtype=np.int64), (replicas, 1))
    next_id = n0
    out = []
    for e in range(events):
        w = np.vectorize(lambda j: float(weight_of(e, int(j))))(res)
        _, keeps = nexus.select_from_weights(w, budget, seed, step=first_step + e)
        kept = np.stack([res[r, k] for r, k in enumerate(keeps)])
        new = np.tile(np.arange(next_id, next_id + n_append, dtype=np.int64), (replicas, 1))
        res = np.concatenate([kept, new], axis=1)
        next_id += n_append
        out.append(res)
    return out
