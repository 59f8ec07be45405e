"""The ring, simulated on one GPU: an ordered host loop over KV chunk buffers that
calls the C-ABI entry points in the order one context-parallel rank would.

Rank r holds query chunk r.  At ring step i it holds KV chunk (r - i) mod CP —
its own chunk first, then the chunks its predecessor passes on (aicassindra,
"Transformer math: SP math", section on context parallelism: K/V blocks rotate
around a ring; axolotl docs "Sequence Parallelism", Implementation Details:
equal contiguous chunks per rank).  The loop only schedules; every step of the
arithmetic runs in the HIP library.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence

import torch

from . import _lib


def ring_schedule(rank: int, cp: int) -> List[int]:
    """KV chunk held at each ring step by `rank`."""
    return [(rank - i) % cp for i in range(cp)]


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


class RingWorkspace:
    """Device temporaries of the ring loops (the only memory beyond inputs/outputs).
    Sized O(Sq * Hq * d); reusable across calls of the same shape."""

    def __init__(self, B: int, Sq: int, Hq: int, d: int, device, backward: bool = False):
        self.o_step = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=device)
        self.lse_step = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device)
        self.o_acc = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=device)
        self.delta = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device) if backward else None

    def nbytes(self) -> int:
        ts = [self.o_step, self.lse_step, self.o_acc, self.delta]
        return sum(t.numel() * t.element_size() for t in ts if t is not None)


def ring_forward(q_local: torch.Tensor, k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor],
                 rank: int, cp: int, *, causal: bool = True, scale: Optional[float] = None,
                 seg_ids: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, workspace: Optional[RingWorkspace] = None,
                 stream=None, step_hook=None):
    """Forward of one rank's share.  Returns (O in q's dtype, LSE fp32 [B, Hq, Sq]).

    q_local [B, C, Hq, d]; k_chunks/v_chunks: cp tensors [B, C, Hkv, d] (chunk c covers
    global tokens [c*C, (c+1)*C)); seg_ids [B, S] int32 global segment ids or None.
    """
    B, C, Hq, d = q_local.shape
    if len(k_chunks) != cp or len(v_chunks) != cp:
        raise ValueError("need one K and one V chunk per ring rank")
    sc = _scale(d, scale)
    ws = workspace or RingWorkspace(B, C, Hq, d, q_local.device)
    if out is None:
        out = torch.empty_like(q_local)
    if lse is None:
        lse = torch.empty((B, Hq, C), dtype=torch.float32, device=q_local.device)
    o_acc = ws.o_acc
    q_offset = rank * C
    for i, c in enumerate(ring_schedule(rank, cp)):
        kc, vc = k_chunks[c], v_chunks[c]
        first = i == 0
        _lib.ring_attn_fwd_step(q_local, kc, vc, o_acc if first else ws.o_step, lse if first else ws.lse_step,
                                q_offset=q_offset, kv_offset=c * kc.shape[1], causal=causal, scale=sc,
                                seg_ids=seg_ids, stream=stream)
        if step_hook is not None:
            step_hook("fwd_step", i)
        last = i == cp - 1
        if not first:
            _lib.lse_merge(o_acc, lse, ws.o_step, ws.lse_step, o_out=out if last else None, stream=stream)
            if step_hook is not None:
                step_hook("merge", i)
        elif last:
            _lib.lse_merge(o_acc, lse, None, None, o_out=out, stream=stream)
    return out, lse


def ring_backward(q_local: torch.Tensor, k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor],
                  o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor, rank: int, cp: int, *,
                  causal: bool = True, scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                  dq: Optional[torch.Tensor] = None, dk_chunks: Optional[Sequence[torch.Tensor]] = None,
                  dv_chunks: Optional[Sequence[torch.Tensor]] = None, delta: Optional[torch.Tensor] = None,
                  stream=None, step_hook=None):
    """Backward of one rank's share, from the forward's final O and LSE.

    Returns (dQ fp32 [B, C, Hq, d], dK list, dV list) where dK[c]/dV[c] fp32 hold this
    rank's contribution to chunk c's gradient.  Given accumulators are added to (+=).
    """
    B, C, Hq, d = q_local.shape
    sc = _scale(d, scale)
    dev = q_local.device
    if dq is None:
        dq = torch.zeros((B, C, Hq, d), dtype=torch.float32, device=dev)
    if dk_chunks is None:
        dk_chunks = [torch.zeros(k.shape, dtype=torch.float32, device=dev) for k in k_chunks]
    if dv_chunks is None:
        dv_chunks = [torch.zeros(v.shape, dtype=torch.float32, device=dev) for v in v_chunks]
    if delta is None:
        delta = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    _lib.ring_attn_bwd_preprocess(o, d_o, delta, stream=stream)
    if step_hook is not None:
        step_hook("bwd_preprocess", 0)
    for i, c in enumerate(ring_schedule(rank, cp)):
        kc, vc = k_chunks[c], v_chunks[c]
        _lib.ring_attn_bwd_step(q_local, kc, vc, d_o, lse, delta, dq, dk_chunks[c], dv_chunks[c],
                                q_offset=rank * C, kv_offset=c * kc.shape[1], causal=causal, scale=sc,
                                seg_ids=seg_ids, stream=stream)
        if step_hook is not None:
            step_hook("bwd_step", i)
    return dq, list(dk_chunks), list(dv_chunks)
