"""fp64 CPU oracle of one context-parallel rank's share of ring attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.  It shares
no code with the HIP library.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    allowed_mask,
    attention_bwd_full,
    attention_bwd_rows,
    attention_full,
    attention_rows,
    bwd_delta,
    live_pairs,
    lse_merge,
    ring_backward,
    ring_forward,
    ring_schedule,
    segment_ids,
)
