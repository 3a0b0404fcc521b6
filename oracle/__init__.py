"""Plain, slow, fp64 CPU oracle of the Nexus Sampling eviction step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library and imports nothing from it; the two meet only through the seeded
input generators in ``workloads/``, which hold none of the method's arithmetic.

Source of every definition here (cited as [Nexus]):
  "Forget Without Compromise: Nexus Sampling for Streaming KV-Cache Eviction
  Under Fixed Budgets" (academ.us article page), sections 2.1-2.3 and
  appendix 8.

Modules
  philox     Philox4x32-10 counter-based generator, from the published
             definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
             as easy as 1, 2, 3", SC'11), in numpy uint64 arithmetic.
  nexus      the eviction step: window attention, Nexus walk, weights,
             A-Res keys, selection, compaction.
  enumerate  exact inclusion probabilities of weighted sampling without
             replacement by enumeration of orders (N <= 8).

Pinning status (what each function is checked against) is listed in the
header of each module.
"""

from . import philox, nexus, enumerate  # noqa: F401
