"""Seeded synthetic workloads for one context-parallel rank's share of ring attention.

The pages measure on real model activations that are not available here, so
i.i.d. N(0,1) tensors of the same shapes stand in for post-RoPE Q/K/V and for the
upstream gradient dO.  The shapes follow the pages' workloads:

* a Llama-3-8B-style run at 8K context split over 4 context-parallel ranks
  (axolotl docs "Sequence Parallelism", section Example; 32 query heads, 8 KV
  heads, head dim 128 are the Llama-3-8B attention dimensions);
* one representative 64K step (archcrux, "sequence-parallel long-context
  attention OOM"), here rank 7 of 8;
* sample-packed rows whose position ids restart at 0 at every sample start
  (axolotl docs "Sequence Parallelism", section Sample Packing with Sequence
  Parallelism).

Recipe (every tensor has its own counter-free numpy PCG64 stream so that one
chunk can be drawn without drawing the whole sequence):

* chunk ``c`` of Q is ``default_rng([seed, 0, c]).standard_normal((B, C, Hq, d), float32)``;
* chunk ``c`` of K / V uses stream ``[seed, 1, c]`` / ``[seed, 2, c]`` with shape (B, C, Hkv, d);
* dO (the local shard only) uses stream ``[seed, 3]``;
* packed sample lengths use stream ``[seed, 4]``: integers uniform on [512, 4096]
  inclusive, drawn until the total reaches S, the last one truncated;
* bf16 workloads round every float32 draw to bfloat16 (round to nearest even) and
  keep the rounded values in float32 arrays, so both sides read identical values.

Nothing here computes attention, masks, merges, segment ids or gradients.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    S: int          # total (global) sequence length
    CP: int         # context-parallel degree (number of contiguous chunks)
    rank: int       # the rank whose share is evaluated
    Hq: int
    Hkv: int
    d: int
    dtype: str      # "f32" or "bf16"
    causal: bool
    packed: bool    # sample-packed row (position ids restart per sample)
    backward: bool  # whether dO is part of the workload
    seed: int
    min_len: int = 512
    max_len: int = 4096

    @property
    def C(self) -> int:
        return self.S // self.CP

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


TINY_RING = Config("tiny_ring_fp32_S1k_cp4_r3", 1, 1024, 4, 3, 1, 1, 64, "f32", True, False, False, 1)
LLAMA3_8K_FWD = Config("llama3_8b_S8k_cp4_r3_fwd", 1, 8192, 4, 3, 32, 8, 128, "bf16", True, False, False, 2)
CTX64K_FWD = Config("ctx64k_cp8_r7_fwd", 1, 65536, 8, 7, 32, 8, 128, "bf16", True, False, False, 3)
PACKED16K_FWD = Config("packed16k_cp4_r2_fwd", 1, 16384, 4, 2, 32, 8, 128, "bf16", True, True, False, 4)
LLAMA3_8K_BWD = Config("llama3_8b_S8k_cp4_r3_bwd", 1, 8192, 4, 3, 32, 8, 128, "bf16", True, False, True, 5)

# The five workloads by name.
CONFIGS = {c.name: c for c in (TINY_RING, LLAMA3_8K_FWD, CTX64K_FWD, PACKED16K_FWD, LLAMA3_8K_BWD)}

# The headline measurement: the 64K share, forward and backward.
METRIC_CONFIG = CTX64K_FWD.with_(name="ctx64k_cp8_r7_fwd_bwd", backward=True)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def draw_packed_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> np.ndarray:
    """Sample lengths ~ integer Uniform[lo, hi], drawn until they cover ``total``;
    the last one is truncated so the lengths sum to exactly ``total``."""
    lengths = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lengths.append(n)
        acc += n
    return np.asarray(lengths, dtype=np.int64)


@dataclasses.dataclass
class Workload:
    cfg: Config
    q_chunks: list          # CP arrays [B, C, Hq, d] float32 (bf16-exact for bf16 configs)
    k_chunks: list          # CP arrays [B, C, Hkv, d]
    v_chunks: list
    do: Optional[np.ndarray]  # [B, C, Hq, d] for the evaluated rank, or None
    position_ids: np.ndarray  # [B, S] int32 (global row)
    sample_index: np.ndarray  # [B, S] int64: which packed sample each token came from
    lengths: Optional[np.ndarray]

    @property
    def q_local(self) -> np.ndarray:
        return self.q_chunks[self.cfg.rank]

    def q_full(self) -> np.ndarray:
        return np.concatenate(self.q_chunks, axis=1)

    def k_full(self) -> np.ndarray:
        return np.concatenate(self.k_chunks, axis=1)

    def v_full(self) -> np.ndarray:
        return np.concatenate(self.v_chunks, axis=1)


def _normal(seed_words, shape, bf16: bool) -> np.ndarray:
    rng = np.random.default_rng(list(seed_words))
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_round(x) if bf16 else x


def make_workload(cfg: Config, q_chunks: Optional[list] = None, seed: Optional[int] = None) -> Workload:
    """Draw the workload of ``cfg``.  ``q_chunks`` restricts which Q chunks are drawn
    (others are None); by default all are drawn (small configs) — the evaluated rank's
    chunk is always drawn."""
    if cfg.S % cfg.CP != 0:
        raise ValueError("S must be divisible by CP")
    seed = cfg.seed if seed is None else seed
    B, C, bf16 = cfg.B, cfg.C, cfg.dtype == "bf16"
    want_q = set(range(cfg.CP)) if q_chunks is None else set(q_chunks) | {cfg.rank}
    qs = [(_normal((seed, 0, c), (B, C, cfg.Hq, cfg.d), bf16) if c in want_q else None)
          for c in range(cfg.CP)]
    ks = [_normal((seed, 1, c), (B, C, cfg.Hkv, cfg.d), bf16) for c in range(cfg.CP)]
    vs = [_normal((seed, 2, c), (B, C, cfg.Hkv, cfg.d), bf16) for c in range(cfg.CP)]
    do = _normal((seed, 3), (B, C, cfg.Hq, cfg.d), bf16) if cfg.backward else None
    if cfg.packed:
        rng = np.random.default_rng([seed, 4])
        pos_rows, idx_rows, lengths_all = [], [], []
        for _ in range(B):
            lengths = draw_packed_lengths(rng, cfg.S, cfg.min_len, cfg.max_len)
            pos_rows.append(np.concatenate([np.arange(n) for n in lengths]))
            idx_rows.append(np.repeat(np.arange(len(lengths)), lengths))
            lengths_all.append(lengths)
        position_ids = np.stack(pos_rows).astype(np.int32)
        sample_index = np.stack(idx_rows).astype(np.int64)
        lengths = lengths_all[0] if B == 1 else lengths_all
    else:
        position_ids = np.tile(np.arange(cfg.S, dtype=np.int32), (B, 1))
        sample_index = np.zeros((B, cfg.S), dtype=np.int64)
        lengths = None
    return Workload(cfg, qs, ks, vs, do, position_ids, sample_index, lengths)


def chunk_view(x: np.ndarray, c: int, C: int) -> np.ndarray:
    """Rows [c*C, (c+1)*C) of a [B, S, ...] array (a view, no copy)."""
    return x[:, c * C:(c + 1) * C]


def zigzag_indices(S: int, cp: int, rank: int) -> np.ndarray:
    """Global token indices held by ``rank`` in the load-balanced causal layout: the
    row is cut into 2*cp equal halves and the rank holds halves rank and
    2*cp-1-rank, in that order.  Data placement only (used to lay out inputs)."""
    if S % (2 * cp):
        raise ValueError("S must be divisible by 2*cp")
    h = S // (2 * cp)
    lo, hi = rank, 2 * cp - 1 - rank
    return np.concatenate([np.arange(lo * h, (lo + 1) * h), np.arange(hi * h, (hi + 1) * h)])


def zigzag_take(x_full: np.ndarray, S: int, cp: int, rank: int) -> np.ndarray:
    """Rows of a [B, S, ...] array held by ``rank`` in the load-balanced layout."""
    return np.ascontiguousarray(x_full[:, zigzag_indices(S, cp, rank)])
