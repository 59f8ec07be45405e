"""Seeded synthetic inputs shared by the fp64 oracle tests, the HIP parity tests and
the benchmark.  This package holds data generation only: no attention, masking,
merging or gradient arithmetic lives here."""

from .workloads import (  # noqa: F401
    CONFIGS,
    CTX64K_FWD,
    LLAMA3_8K_BWD,
    LLAMA3_8K_FWD,
    METRIC_CONFIG,
    PACKED16K_FWD,
    TINY_RING,
    Workload,
    bf16_round,
    chunk_view,
    draw_packed_lengths,
    make_workload,
    zigzag_indices,
    zigzag_take,
)
