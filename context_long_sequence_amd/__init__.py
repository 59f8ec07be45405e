"""One context-parallel rank's share of ring attention on AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libringattn.so`` (C ABI in include/ringattn.h);
this package is its ctypes binding plus the ring schedule simulated on one GPU.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    RingAttnError,
    library_path,
    load,
    lse_merge,
    ring_attn_bwd_preprocess,
    ring_attn_bwd_step,
    ring_attn_bwd_step_noalloc,
    ring_attn_fwd_step,
    ring_attn_fwd_step_merge,
    ring_recv_copy,
    segment_mask_from_pos,
)
from .ring import (  # noqa: F401
    RingSlots,
    RingWorkspace,
    ZigzagWorkspace,
    ring_backward,
    ring_backward_overlapped,
    ring_backward_zigzag,
    ring_forward,
    ring_forward_overlapped,
    ring_forward_zigzag,
    ring_schedule,
    zigzag_halves,
    zigzag_pairs,
    gather_kv,
    gathered_backward,
    gathered_forward,
    scatter_dkv,
    ulysses_backward,
    ulysses_forward,
)
