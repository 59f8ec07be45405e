"""Seeded synthetic inputs shared by the fp64 oracle tests, the HIP parity tests and
the benchmark.  This package holds data generation only: no attention, masking,
merging or gradient arithmetic lives here."""

from .workloads import (  # noqa: F401
    CONFIGS,
    METRIC_CONFIG,
    Workload,
    bf16_round,
    chunk_view,
    draw_packed_lengths,
    make_workload,
    zigzag_indices,
    zigzag_take,
)
