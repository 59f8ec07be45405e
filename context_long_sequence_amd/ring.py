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

import functools
import math
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib


def ring_schedule(rank: int, cp: int) -> List[int]:
    """KV chunk held at each ring step by `rank`."""
    return [(rank - i) % cp for i in range(cp)]


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _torch_stream(stream) -> torch.cuda.Stream:
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _on_stream(fn):
    """Runs `fn` with its `stream` argument as torch's current stream, so that the
    temporaries it allocates (and the fills that zero them) belong to the stream its
    kernels run on: the caching allocator then never hands their memory to other
    work while those kernels may still use it."""

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        with torch.cuda.stream(_torch_stream(kw.get("stream"))):
            return fn(*args, **kw)

    return wrapper


def _used_on(stream: torch.cuda.Stream, tensors) -> None:
    """Marks tensors that kernels on a second stream use, so that freeing them waits
    for that stream's work as well."""
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


class RingWorkspace:
    """Device temporaries of the ring loops (the only memory beyond inputs/outputs):
    the fp32 running O of the forward (each step's partial is folded into it inside
    the step's launch, so no per-step buffer exists) and the backward's delta.
    Sized O(Sq * Hq * d); reusable across calls of the same shape."""

    def __init__(self, B: int, Sq: int, Hq: int, d: int, device, backward: bool = False):
        self.o_acc = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=device)
        self.delta = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device) if backward else None

    def nbytes(self) -> int:
        ts = [self.o_acc, self.delta]
        return sum(t.numel() * t.element_size() for t in ts if t is not None)


def _fold_step(q, kc, vc, o_acc, lse_acc, first: bool, last: bool, out, *, q_offset: int, kv_offset: int,
               causal: bool, scale: float, seg_ids, stream, step_hook=None, step: int = 0):
    """One ring step into the running (o_acc, lse_acc): the first step writes it
    (ring_attn_fwd_step), every later one folds its partial into it in the same
    launch (ring_attn_fwd_step_merge); the last step also writes `out` (q's dtype)."""
    if first:
        _lib.ring_attn_fwd_step(q, kc, vc, o_acc, lse_acc, q_offset=q_offset, kv_offset=kv_offset, causal=causal,
                                scale=scale, seg_ids=seg_ids, stream=stream)
        if step_hook is not None:
            step_hook("fwd_step", step)
        if last:  # a single step: only the conversion
            _lib.lse_merge(o_acc, lse_acc, None, None, o_out=out, stream=stream)
            if step_hook is not None:
                step_hook("merge", step)
    else:
        _lib.ring_attn_fwd_step_merge(q, kc, vc, o_acc, lse_acc, q_offset=q_offset, kv_offset=kv_offset,
                                      causal=causal, scale=scale, seg_ids=seg_ids, o_out=out if last else None,
                                      stream=stream)
        if step_hook is not None:
            step_hook("fwd_step", step)


@_on_stream
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
    q_offset = rank * C
    for i, c in enumerate(ring_schedule(rank, cp)):
        kc, vc = k_chunks[c], v_chunks[c]
        _fold_step(q_local, kc, vc, ws.o_acc, lse, i == 0, i == cp - 1, out, q_offset=q_offset,
                   kv_offset=c * kc.shape[1], causal=causal, scale=sc, seg_ids=seg_ids, stream=stream,
                   step_hook=step_hook, step=i)
    return out, lse


@_on_stream
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


# ---- load-balanced causal layout ----------------------------------------------------
# With contiguous chunks and a causal mask, rank r has (r + 1/2) chunks' worth of
# visible pairs, so the last rank sets the pace (aicassindra, "Transformer math: SP
# math": the causal load-balance problem).  In the balanced ("zigzag") layout the
# row is cut into 2*cp equal halves and rank r holds halves r and 2*cp-1-r (its
# query, key and value rows, in that order); every rank then has the same number of
# visible pairs, 2*cp*h^2 + h for halves of h tokens.  The ring is unchanged: at
# step i rank r holds the K/V rows of rank (r - i) mod cp.  Each (query half, key
# half) pair is one call of the step entry points with the halves' true global
# offsets, so the causal rule and packed-row segment ids apply as everywhere else;
# pairs in which every key lies after every query are skipped.

def zigzag_halves(rank: int, cp: int) -> Tuple[int, int]:
    """Half-chunk indices held by `rank` (each half covers h = S / (2 cp) tokens)."""
    return rank, 2 * cp - 1 - rank


def zigzag_pairs(rank: int, cp: int, h: int, causal: bool = True) -> List[Tuple[int, int, int, int]]:
    """Live (ring step, KV rank, query half j, key half k) in ring order; j, k in {0, 1}
    index the halves of `zigzag_halves`.  A pair is dropped when, under the causal
    rule, its first key lies after its last query."""
    qh = zigzag_halves(rank, cp)
    out = []
    for i, c in enumerate(ring_schedule(rank, cp)):
        kh = zigzag_halves(c, cp)
        for j in range(2):
            for k in range(2):
                if causal and kh[k] * h > qh[j] * h + h - 1:
                    continue
                out.append((i, c, j, k))
    return out


class ZigzagWorkspace:
    """Device temporaries of the balanced-layout ring loops: per-half running O and
    the backward's delta ([2, Hq, h]: one row block per half)."""

    def __init__(self, h: int, Hq: int, d: int, device, backward: bool = False):
        self.o_acc = torch.empty((2, h, Hq, d), dtype=torch.float32, device=device)
        self.delta = torch.empty((2, Hq, h), dtype=torch.float32, device=device) if backward else None

    def nbytes(self) -> int:
        ts = [self.o_acc, self.delta]
        return sum(t.numel() * t.element_size() for t in ts if t is not None)


def _half(t: torch.Tensor, j: int, h: int) -> torch.Tensor:
    return t[:, j * h:(j + 1) * h]


@_on_stream
def ring_forward_zigzag(q_local: torch.Tensor, k_ranks: Sequence[torch.Tensor], v_ranks: Sequence[torch.Tensor],
                        rank: int, cp: int, *, causal: bool = True, scale: Optional[float] = None,
                        seg_ids: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, workspace: Optional[ZigzagWorkspace] = None,
                        stream=None, step_hook=None):
    """Forward of one rank's share in the balanced layout.  Returns (O [1, 2h, Hq, d] in
    q's dtype, LSE fp32 [2, Hq, h]: row block j = query half j).

    q_local [1, 2h, Hq, d] holds the rank's two query halves; k_ranks/v_ranks: cp
    tensors [1, 2h, Hkv, d], the K/V rows of each rank in the same layout; seg_ids
    [1, S] int32 global segment ids or None.  Batch 1 (the half views must be
    contiguous)."""
    B, S2, Hq, d = q_local.shape
    if B != 1 or S2 % 2:
        raise ValueError("the balanced layout takes batch 1 and an even local length")
    if len(k_ranks) != cp or len(v_ranks) != cp:
        raise ValueError("need the K and V rows of every ring rank")
    h = S2 // 2
    sc = _scale(d, scale)
    ws = workspace or ZigzagWorkspace(h, Hq, d, q_local.device)
    if out is None:
        out = torch.empty_like(q_local)
    if lse is None:
        lse = torch.empty((2, Hq, h), dtype=torch.float32, device=q_local.device)
    qh = zigzag_halves(rank, cp)
    pairs = zigzag_pairs(rank, cp, h, causal)
    last_of = {j: max(n for n, p in enumerate(pairs) if p[2] == j) for j in range(2) if any(p[2] == j for p in pairs)}
    seen = [False, False]
    for n, (i, c, j, k) in enumerate(pairs):
        kh = zigzag_halves(c, cp)
        acc, lacc = ws.o_acc[j:j + 1], lse[j:j + 1]
        _fold_step(_half(q_local, j, h), _half(k_ranks[c], k, h), _half(v_ranks[c], k, h), acc, lacc,
                   not seen[j], last_of[j] == n, _half(out, j, h), q_offset=qh[j] * h, kv_offset=kh[k] * h,
                   causal=causal, scale=sc, seg_ids=seg_ids, stream=stream, step_hook=step_hook, step=i)
        seen[j] = True
    for j in range(2):
        if not seen[j]:  # no visible key at all (not reachable under the causal rule)
            raise ValueError("a query half has no live key half")
    return out, lse


@_on_stream
def ring_backward_zigzag(q_local: torch.Tensor, k_ranks: Sequence[torch.Tensor], v_ranks: Sequence[torch.Tensor],
                         o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor, rank: int, cp: int, *,
                         causal: bool = True, scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                         dq: Optional[torch.Tensor] = None, dk_ranks: Optional[Sequence[torch.Tensor]] = None,
                         dv_ranks: Optional[Sequence[torch.Tensor]] = None,
                         workspace: Optional[ZigzagWorkspace] = None, stream=None, step_hook=None):
    """Backward of one rank's share in the balanced layout, from the forward's final O
    and LSE [2, Hq, h].  Returns (dQ fp32 [1, 2h, Hq, d], dK list, dV list): dK[c]/dV[c]
    [1, 2h, Hkv, d] fp32 hold this rank's contribution to rank c's K/V rows.  Given
    accumulators are added to (+=)."""
    B, S2, Hq, d = q_local.shape
    if B != 1 or S2 % 2:
        raise ValueError("the balanced layout takes batch 1 and an even local length")
    h = S2 // 2
    sc = _scale(d, scale)
    dev = q_local.device
    ws = workspace or ZigzagWorkspace(h, Hq, d, dev, backward=True)
    if dq is None:
        dq = torch.zeros((1, S2, Hq, d), dtype=torch.float32, device=dev)
    if dk_ranks is None:
        dk_ranks = [torch.zeros(k.shape, dtype=torch.float32, device=dev) for k in k_ranks]
    if dv_ranks is None:
        dv_ranks = [torch.zeros(v.shape, dtype=torch.float32, device=dev) for v in v_ranks]
    for j in range(2):
        _lib.ring_attn_bwd_preprocess(_half(o, j, h), _half(d_o, j, h), ws.delta[j:j + 1], stream=stream)
    if step_hook is not None:
        step_hook("bwd_preprocess", 0)
    qh = zigzag_halves(rank, cp)
    for i, c, j, k in zigzag_pairs(rank, cp, h, causal):
        kh = zigzag_halves(c, cp)
        _lib.ring_attn_bwd_step(_half(q_local, j, h), _half(k_ranks[c], k, h), _half(v_ranks[c], k, h),
                                _half(d_o, j, h), lse[j:j + 1], ws.delta[j:j + 1], _half(dq, j, h),
                                _half(dk_ranks[c], k, h), _half(dv_ranks[c], k, h),
                                q_offset=qh[j] * h, kv_offset=kh[k] * h, causal=causal, scale=sc,
                                seg_ids=seg_ids, stream=stream)
        if step_hook is not None:
            step_hook("bwd_step", i)
    return dq, list(dk_ranks), list(dv_ranks)


# ---- overlapped receives --------------------------------------------------------------
# A rank passes its K/V on while it attends to the chunk it holds (aicassindra,
# "Transformer math: SP math": K/V blocks rotate around the ring; axolotl docs
# "Sequence Parallelism", introduction: partial results are aggregated as chunks
# pass around the ring).  Here the receive of the next step's chunk is a
# device-to-device copy on the DMA engines (`ring_recv_copy`), from the buffer
# standing for the peer's chunk into one of two receive slots, issued on a second
# stream while the current step computes;
# events order each copy after the step that last read its slot and before the step
# that reads it.  In the backward the fp32 dK/dV partials travel with their chunk:
# received with it, added to in place by the step, sent on after it.

class RingSlots:
    """Two receive slots for K and V (and, for the backward, the travelling dK/dV)."""

    def __init__(self, k_like: torch.Tensor, v_like: torch.Tensor, backward: bool = False):
        self.k = [torch.empty_like(k_like) for _ in range(2)]
        self.v = [torch.empty_like(v_like) for _ in range(2)]
        self.dk = [torch.empty(k_like.shape, dtype=torch.float32, device=k_like.device) for _ in range(2)] \
            if backward else None
        self.dv = [torch.empty(v_like.shape, dtype=torch.float32, device=v_like.device) for _ in range(2)] \
            if backward else None

    def nbytes(self) -> int:
        ts = self.k + self.v + (self.dk or []) + (self.dv or [])
        return sum(t.numel() * t.element_size() for t in ts)


def _streams(stream, comm_stream, device):
    compute = torch.cuda.current_stream(device) if stream is None else stream
    if not isinstance(compute, torch.cuda.Stream):
        raise TypeError("the overlapped ring needs torch.cuda.Stream objects")
    comm = torch.cuda.Stream(device) if comm_stream is None else comm_stream
    return compute, comm


@_on_stream
def ring_forward_overlapped(q_local: torch.Tensor, k_chunks: Sequence[torch.Tensor],
                            v_chunks: Sequence[torch.Tensor], rank: int, cp: int, *, causal: bool = True,
                            scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            workspace: Optional[RingWorkspace] = None, slots: Optional[RingSlots] = None,
                            stream=None, comm_stream=None):
    """`ring_forward` with the chunk of step i+1 received while step i computes.
    Same kernels in the same order, so the results are bit-identical."""
    B, C, Hq, d = q_local.shape
    sc = _scale(d, scale)
    dev = q_local.device
    compute, comm = _streams(stream, comm_stream, dev)
    ws = workspace or RingWorkspace(B, C, Hq, d, dev)
    sl = slots or RingSlots(k_chunks[0], v_chunks[0])
    if slots is None:
        _used_on(comm, sl.k + sl.v)
    if out is None:
        out = torch.empty_like(q_local)
    if lse is None:
        lse = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    sched = ring_schedule(rank, cp)
    comm.wait_stream(compute)  # the chunks may have been produced on the compute stream
    received: List[Optional[torch.cuda.Event]] = [None, None]
    released: List[Optional[torch.cuda.Event]] = [None, None]

    def receive(i):
        s, c = i % 2, sched[i]
        if released[s] is not None:
            comm.wait_event(released[s])
        _lib.ring_recv_copy(sl.k[s], k_chunks[c], stream=comm)
        _lib.ring_recv_copy(sl.v[s], v_chunks[c], stream=comm)
        received[s] = torch.cuda.Event()
        received[s].record(comm)

    o_acc = ws.o_acc
    for i, c in enumerate(sched):
        if i + 1 < cp:
            receive(i + 1)
        if i == 0:
            kc, vc = k_chunks[c], v_chunks[c]  # the rank's own chunk needs no receive
        else:
            compute.wait_event(received[i % 2])
            kc, vc = sl.k[i % 2], sl.v[i % 2]
        _fold_step(q_local, kc, vc, o_acc, lse, i == 0, i == cp - 1, out, q_offset=rank * C,
                   kv_offset=c * kc.shape[1], causal=causal, scale=sc, seg_ids=seg_ids, stream=compute)
        if i > 0:
            released[i % 2] = torch.cuda.Event()
            released[i % 2].record(compute)
    return out, lse


@_on_stream
def ring_backward_overlapped(q_local: torch.Tensor, k_chunks: Sequence[torch.Tensor],
                             v_chunks: Sequence[torch.Tensor], o: torch.Tensor, lse: torch.Tensor,
                             d_o: torch.Tensor, rank: int, cp: int, *, causal: bool = True,
                             scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                             dq: Optional[torch.Tensor] = None, dk_chunks: Optional[Sequence[torch.Tensor]] = None,
                             dv_chunks: Optional[Sequence[torch.Tensor]] = None, delta: Optional[torch.Tensor] = None,
                             slots: Optional[RingSlots] = None, stream=None, comm_stream=None):
    """`ring_backward` with receives (K, V and the travelling dK/dV partial of the next
    chunk) overlapped with the current step, and each partial sent on after its step.
    dk_chunks[c]/dv_chunks[c] stand for the partial that arrives with chunk c; on
    return they hold it plus this rank's contribution, bit-identical to
    `ring_backward`."""
    B, C, Hq, d = q_local.shape
    sc = _scale(d, scale)
    dev = q_local.device
    compute, comm = _streams(stream, comm_stream, dev)
    sl = slots or RingSlots(k_chunks[0], v_chunks[0], backward=True)
    if sl.dk is None:
        raise ValueError("the backward needs slots with dK/dV buffers")
    dk_given, dv_given = dk_chunks, dv_chunks
    if dq is None:
        dq = torch.zeros((B, C, Hq, d), dtype=torch.float32, device=dev)
    if dk_chunks is None:
        dk_chunks = [torch.zeros(k.shape, dtype=torch.float32, device=dev) for k in k_chunks]
    if dv_chunks is None:
        dv_chunks = [torch.zeros(v.shape, dtype=torch.float32, device=dev) for v in v_chunks]
    if delta is None:
        delta = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    if slots is None:
        _used_on(comm, sl.k + sl.v + sl.dk + sl.dv)
    for given, made in ((dk_given, dk_chunks), (dv_given, dv_chunks)):
        if given is None:
            _used_on(comm, made)
    sched = ring_schedule(rank, cp)
    comm.wait_stream(compute)
    _lib.ring_attn_bwd_preprocess(o, d_o, delta, stream=compute)
    received: List[Optional[torch.cuda.Event]] = [None, None]

    def receive(i):
        # in comm-stream order after the send of step i-2, which used this slot
        s, c = i % 2, sched[i]
        for dst, src in ((sl.k[s], k_chunks[c]), (sl.v[s], v_chunks[c]), (sl.dk[s], dk_chunks[c]),
                         (sl.dv[s], dv_chunks[c])):
            _lib.ring_recv_copy(dst, src, stream=comm)
        received[s] = torch.cuda.Event()
        received[s].record(comm)

    for i, c in enumerate(sched):
        if i + 1 < cp:
            receive(i + 1)
        if i == 0:
            kc, vc, dkc, dvc = k_chunks[c], v_chunks[c], dk_chunks[c], dv_chunks[c]
        else:
            s = i % 2
            compute.wait_event(received[s])
            kc, vc, dkc, dvc = sl.k[s], sl.v[s], sl.dk[s], sl.dv[s]
        _lib.ring_attn_bwd_step(q_local, kc, vc, d_o, lse, delta, dq, dkc, dvc,
                                q_offset=rank * C, kv_offset=c * kc.shape[1], causal=causal, scale=sc,
                                seg_ids=seg_ids, stream=compute)
        if i > 0:  # send the partial on once the step has added to it
            done = torch.cuda.Event()
            done.record(compute)
            comm.wait_event(done)
            _lib.ring_recv_copy(dk_chunks[c], dkc, stream=comm)
            _lib.ring_recv_copy(dv_chunks[c], dvc, stream=comm)
    compute.wait_stream(comm)  # the last sends are part of the result
    return dq, list(dk_chunks), list(dv_chunks)


# ---- head-sharded share (Ulysses) ---------------------------------------------------
# Instead of cutting the sequence, a rank holds Hq/cp query heads and Hkv/cp KV heads
# of the whole row (aicassindra, "Transformer math: SP math", the head-sharded
# alternative to the ring; the all-to-all that moves a rank's sequence chunk into
# this layout and back is the multi-GPU part, left out).  Its share is plain masked
# attention over the full row: one forward step call and one backward step call
# with offsets 0 — the same kernels at a different shape, no merges.

@_on_stream
def ulysses_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = True,
                    scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    o_f32: Optional[torch.Tensor] = None, stream=None):
    """q [B, S, Hq', d], k/v [B, S, Hkv', d] (the rank's heads of the whole row).
    Returns (O in q's dtype, LSE fp32 [B, Hq', S])."""
    B, S, Hq, d = q.shape
    sc = _scale(d, scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    if o_f32 is None:
        o_f32 = torch.empty((B, S, Hq, d), dtype=torch.float32, device=dev)
    _lib.ring_attn_fwd_step(q, k, v, o_f32, lse, q_offset=0, kv_offset=0, causal=causal, scale=sc,
                            seg_ids=seg_ids, stream=stream)
    _lib.lse_merge(o_f32, lse, None, None, o_out=out, stream=stream)
    return out, lse


@_on_stream
def ulysses_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                     d_o: torch.Tensor, *, causal: bool = True, scale: Optional[float] = None,
                     seg_ids: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
                     dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                     delta: Optional[torch.Tensor] = None, stream=None):
    """Gradients of `ulysses_forward` (fp32; given accumulators are added to)."""
    B, S, Hq, d = q.shape
    sc = _scale(d, scale)
    dev = q.device
    if dq is None:
        dq = torch.zeros((B, S, Hq, d), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.zeros(v.shape, dtype=torch.float32, device=dev)
    if delta is None:
        delta = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    _lib.ring_attn_bwd_preprocess(o, d_o, delta, stream=stream)
    _lib.ring_attn_bwd_step(q, k, v, d_o, lse, delta, dq, dk, dv, q_offset=0, kv_offset=0, causal=causal,
                            scale=sc, seg_ids=seg_ids, stream=stream)
    return dq, dk, dv


# ---- gathered-KV share (llama3-style) ------------------------------------------------
# The alternative to the ring that packing-aware trainers use by default (axolotl docs
# "Sequence Parallelism", the ring_attn_func options): every rank gathers the K/V of
# the whole row, then its contiguous query chunk attends to it once, segment ids
# handling packed samples.  `heads_k_stride` there bounds the gathered memory by
# gathering a few KV heads per round; with 288 GB of HBM per GPU the whole row's K/V
# (256 MiB at 64K, 8 KV heads, d = 128) is gathered at once.  On one GPU the gather
# is cp device-to-device copies (DMA engines) of the chunk buffers into one [B, S,
# Hkv, d] buffer; the backward's reduce-scatter returns each chunk's dK/dV rows to
# the chunk accumulators the same way.

@_on_stream
def gather_kv(k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor],
              k_all: Optional[torch.Tensor] = None, v_all: Optional[torch.Tensor] = None, stream=None):
    """Concatenate the chunks along the row into k_all/v_all [B, S, Hkv, d] (batch 1: the
    chunk rows of one batch row are contiguous in the gathered buffer)."""
    B, C, Hkv, d = k_chunks[0].shape
    if B != 1:
        raise ValueError("the gathered share takes batch 1")
    cp = len(k_chunks)
    if k_all is None:
        k_all = torch.empty((1, cp * C, Hkv, d), dtype=k_chunks[0].dtype, device=k_chunks[0].device)
    if v_all is None:
        v_all = torch.empty((1, cp * C, Hkv, d), dtype=v_chunks[0].dtype, device=v_chunks[0].device)
    for c in range(cp):
        _lib.ring_recv_copy(k_all[:, c * C:(c + 1) * C], k_chunks[c], stream=stream)
        _lib.ring_recv_copy(v_all[:, c * C:(c + 1) * C], v_chunks[c], stream=stream)
    return k_all, v_all


@_on_stream
def gathered_forward(q_local: torch.Tensor, k_all: torch.Tensor, v_all: torch.Tensor, rank: int, *,
                     causal: bool = True, scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     o_f32: Optional[torch.Tensor] = None, stream=None):
    """The rank's contiguous query chunk q_local [B, C, Hq, d] against the gathered row
    k_all/v_all [B, S, Hkv, d].  Returns (O in q's dtype, LSE fp32 [B, Hq, C])."""
    B, C, Hq, d = q_local.shape
    sc = _scale(d, scale)
    dev = q_local.device
    if out is None:
        out = torch.empty_like(q_local)
    if lse is None:
        lse = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    if o_f32 is None:
        o_f32 = torch.empty((B, C, Hq, d), dtype=torch.float32, device=dev)
    _lib.ring_attn_fwd_step(q_local, k_all, v_all, o_f32, lse, q_offset=rank * C, kv_offset=0, causal=causal,
                            scale=sc, seg_ids=seg_ids, stream=stream)
    _lib.lse_merge(o_f32, lse, None, None, o_out=out, stream=stream)
    return out, lse


@_on_stream
def gathered_backward(q_local: torch.Tensor, k_all: torch.Tensor, v_all: torch.Tensor, o: torch.Tensor,
                      lse: torch.Tensor, d_o: torch.Tensor, rank: int, *, causal: bool = True,
                      scale: Optional[float] = None, seg_ids: Optional[torch.Tensor] = None,
                      dq: Optional[torch.Tensor] = None, dk_all: Optional[torch.Tensor] = None,
                      dv_all: Optional[torch.Tensor] = None, delta: Optional[torch.Tensor] = None, stream=None):
    """Gradients of `gathered_forward`: dQ [B, C, Hq, d] and this rank's contribution to
    the whole row's dK/dV [B, S, Hkv, d] (fp32; given accumulators are added to).  Rows
    [c*C, (c+1)*C) of dk_all/dv_all belong to chunk c (`scatter_dkv` returns them)."""
    B, C, Hq, d = q_local.shape
    sc = _scale(d, scale)
    dev = q_local.device
    if dq is None:
        dq = torch.zeros((B, C, Hq, d), dtype=torch.float32, device=dev)
    if dk_all is None:
        dk_all = torch.zeros(k_all.shape, dtype=torch.float32, device=dev)
    if dv_all is None:
        dv_all = torch.zeros(v_all.shape, dtype=torch.float32, device=dev)
    if delta is None:
        delta = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    _lib.ring_attn_bwd_preprocess(o, d_o, delta, stream=stream)
    _lib.ring_attn_bwd_step(q_local, k_all, v_all, d_o, lse, delta, dq, dk_all, dv_all, q_offset=rank * C,
                            kv_offset=0, causal=causal, scale=sc, seg_ids=seg_ids, stream=stream)
    return dq, dk_all, dv_all


@_on_stream
def scatter_dkv(dk_all: torch.Tensor, dv_all: torch.Tensor, dk_chunks: Sequence[torch.Tensor],
                dv_chunks: Sequence[torch.Tensor], stream=None) -> None:
    """Copy row block c of the gathered-row gradients into the chunk accumulators
    dk_chunks[c]/dv_chunks[c] (the reduce-scatter's data movement for this rank)."""
    C = dk_chunks[0].shape[1]
    for c in range(len(dk_chunks)):
        _lib.ring_recv_copy(dk_chunks[c], dk_all[:, c * C:(c + 1) * C], stream=stream)
        _lib.ring_recv_copy(dv_chunks[c], dv_all[:, c * C:(c + 1) * C], stream=stream)
