"""Seeded synthetic inputs for the eviction step (shared by tests and the benchmark).

This package holds input generation only: no step of the scoring, sampling or
compaction arithmetic.  It is the one module that both the oracle-side tests
and the HIP-side tests / benchmark import.
"""

from .synth import (  # noqa: F401
    WORKLOADS, Workload, budget_for, gen_layer, gen_model, gen_stream_rows,
    gen_stream_queries, ragged_lengths, bf16_bits, fill_layer_, SurvivalSpec, SURVIVAL,
    survival_initial, survival_event,
)
