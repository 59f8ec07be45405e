"""Plain fp64 CPU oracle for one context-parallel rank's share of ring attention.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path and imports nothing from it.  It is written to be read against
the definitions, not to be fast.

What it computes, and the passages it follows:

* Attention must let every query see every key (aicassindra, "Transformer math:
  SP math", section "Context parallelism is the axis that is independent"); the
  quantity is scaled dot-product attention softmax(scale * Q K^T + mask) V with
  scale = 1/sqrt(d).  The pages do not print the formula; this is the standard
  definition and the plainest reading.
* Context parallelism splits the sequence into equal contiguous chunks, one per
  rank (axolotl docs "Sequence Parallelism", section Implementation Details), and
  rotates K/V chunks around a ring so that no device holds the whole sequence
  (aicassindra, same section).  Rank r at ring step i holds chunk (r - i) mod CP
  (direction not stated on the pages; reading documented with the design).
* The per-chunk partial results are combined ("aggregated through a ring
  communication pattern", axolotl docs, introduction) by the log-sum-exp merge,
  which reproduces the full softmax exactly.
* Packed rows: the sample index of each token is recovered from position_ids by a
  cumulative sum of the positions where a new sample starts, computed over the
  global row so a chunk beginning mid-sample keeps its sample (axolotl docs,
  section Mamba/SSM Hybrid Models, item on seq_idx); a query may attend only to
  keys of its own sample (section Sample Packing with Sequence Parallelism).
* The backward pass recomputes the probabilities from the saved log-sum-exp
  (archcrux: FlashAttention-style kernels avoid the S x S matrix but still have
  to backpropagate over the whole context; recomputation trades memory for
  compute) and uses the closed-form softmax-attention gradient.

Layouts (row-major): Q, O, dO [B, Sq, Hq, d]; K, V [B, Sk, Hkv, d]; LSE, delta
[B, Hq, Sq]; query head h reads KV head h // (Hq // Hkv).  Indices passed as
``q_idx`` / ``k_idx`` are GLOBAL token positions in the packed row.

Every function is fp64 throughout.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf

# Rows of one query block processed at once.  Rows of a softmax are independent,
# so splitting the query rows changes nothing but peak memory.
ROW_BLOCK = 256


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def segment_ids(position_ids: np.ndarray) -> np.ndarray:
    """seg[b, t] = #{t' <= t : position_ids[b, t'] == 0} - 1 over the global row.

    axolotl docs "Sequence Parallelism", section Mamba/SSM Hybrid Models: the
    sample index is derived from position_ids by a cumulative sum that stays
    correct when a chunk starts in the middle of a sample.  Tokens before the
    first zero (none in a well-formed packed row) get -1.
    """
    pos = np.asarray(position_ids)
    starts = (pos == 0).astype(np.int64)
    return (np.cumsum(starts, axis=-1) - 1).astype(np.int32)


def allowed_mask(q_idx, k_idx, causal: bool, seg_q=None, seg_k=None) -> np.ndarray:
    """allowed[i, j] for global query index q_idx[i] and key index k_idx[j].

    Causal: a key is visible iff it is not in the query's future (k <= q).
    Packed: additionally the key must belong to the query's sample.
    """
    q_idx = np.asarray(q_idx)
    k_idx = np.asarray(k_idx)
    m = np.ones((q_idx.size, k_idx.size), dtype=bool)
    if causal:
        m &= k_idx[None, :] <= q_idx[:, None]
    if (seg_q is None) != (seg_k is None):
        raise ValueError("seg_q and seg_k must both be given or both be None")
    if seg_q is not None:
        m &= np.asarray(seg_k)[None, :] == np.asarray(seg_q)[:, None]
    return m


def attention_rows(q, k, v, q_idx, k_idx, scale, causal, seg_q=None, seg_k=None):
    """Masked softmax attention of query rows ``q`` [Nq, Hq, d] against keys/values
    ``k``, ``v`` [Nk, Hkv, d] of one batch row.

    Returns (O [Nq, Hq, d], LSE [Hq, Nq]) in fp64 with LSE = ln sum_j exp(s_ij) over
    the allowed keys.  A row with no allowed key has O = 0 and LSE = -inf (the
    identity of the merge below).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Nq, Hq, d = q.shape
    Nk, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    o = np.zeros((Nq, Hq, d))
    lse = np.full((Hq, Nq), NEG_INF)
    if Nq == 0 or Nk == 0:
        return o, lse
    q_idx = np.asarray(q_idx)
    seg_q_arr = None if seg_q is None else np.asarray(seg_q)
    for r0 in range(0, Nq, ROW_BLOCK):
        rows = slice(r0, min(Nq, r0 + ROW_BLOCK))
        mask = allowed_mask(q_idx[rows], k_idx, causal,
                            None if seg_q_arr is None else seg_q_arr[rows], seg_k)
        live = mask.any(axis=1)
        if not live.any():
            continue  # no row of this block sees any key: O = 0, LSE = -inf as initialised
        for h in range(Hq):
            g = h // group
            s = scale * (q[rows, h, :] @ k[:, g, :].T)
            s = np.where(mask, s, NEG_INF)
            m = np.where(live, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])          # exp(-inf) = 0 on masked entries
            l = e.sum(axis=1)
            l_safe = np.where(live, l, 1.0)
            o[rows, h, :] = np.where(live[:, None], (e @ v[:, g, :]) / l_safe[:, None], 0.0)
            lse[h, rows] = np.where(live, m + np.log(l_safe), NEG_INF)
    return o, lse


def attention_full(q, k, v, q_idx, k_idx, scale, causal, seg_q=None, seg_k=None):
    """Batched wrapper: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d], seg_* [B, N] or None.
    Returns O [B, Nq, Hq, d], LSE [B, Hq, Nq]."""
    q = _f64(q)
    B = q.shape[0]
    outs = [attention_rows(q[b], k[b], v[b], q_idx, k_idx, scale, causal,
                           None if seg_q is None else seg_q[b],
                           None if seg_k is None else seg_k[b]) for b in range(B)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def lse_merge(o, lse, o_s, lse_s):
    """Merge two partial results of the same query rows.

    With L = ln sum over one key set and L_s over a disjoint key set,
    L' = ln(e^L + e^L_s) (evaluated as M + ln(e^(L-M) + e^(L_s-M)), M = max(L, L_s))
    and O' = e^(L - L') O + e^(L_s - L') O_s.  If both are -inf the pair is left as is.
    o, o_s [B, Sq, Hq, d]; lse, lse_s [B, Hq, Sq].
    """
    o, lse, o_s, lse_s = _f64(o), _f64(lse), _f64(o_s), _f64(lse_s)
    m = np.maximum(lse, lse_s)
    dead = m == NEG_INF
    m_safe = np.where(dead, 0.0, m)
    w = np.exp(lse - m_safe)
    w_s = np.exp(lse_s - m_safe)
    tot = np.where(dead, 1.0, w + w_s)
    lse_new = np.where(dead, NEG_INF, m_safe + np.log(tot))
    a = np.where(dead, 1.0, w / tot)          # dead rows keep o unchanged
    a_s = np.where(dead, 0.0, w_s / tot)
    # [B, Hq, Sq] -> [B, Sq, Hq, 1] to scale rows of O
    a = np.transpose(a, (0, 2, 1))[..., None]
    a_s = np.transpose(a_s, (0, 2, 1))[..., None]
    return a * o + a_s * o_s, lse_new


def ring_schedule(rank: int, cp: int):
    """Chunks rank ``rank`` holds at ring steps 0..cp-1: its own chunk first, then
    the chunks received from its predecessor, (rank - i) mod cp."""
    return [(rank - i) % cp for i in range(cp)]


def ring_forward(q_loc, k_chunks, v_chunks, rank, cp, scale, causal, seg=None,
                 partials=None):
    """The method itself in fp64: partial attention of the local query shard against
    each KV chunk in ring order, merged step by step.

    q_loc [B, C, Hq, d]; k_chunks/v_chunks: cp arrays [B, C, Hkv, d]; seg [B, S]
    global segment ids or None.  Returns (O, LSE).  If ``partials`` is a list, the
    per-step (chunk, O_c, LSE_c) are appended to it.
    """
    q_loc = _f64(q_loc)
    B, C, Hq, d = q_loc.shape
    q_idx = rank * C + np.arange(C)
    o = np.zeros((B, C, Hq, d))
    lse = np.full((B, Hq, C), NEG_INF)
    for c in ring_schedule(rank, cp):
        k_idx = c * C + np.arange(C)
        seg_q = None if seg is None else seg[:, rank * C:(rank + 1) * C]
        seg_k = None if seg is None else seg[:, c * C:(c + 1) * C]
        o_c, lse_c = attention_full(q_loc, k_chunks[c], v_chunks[c], q_idx, k_idx,
                                    scale, causal, seg_q, seg_k)
        if partials is not None:
            partials.append((c, o_c, lse_c))
        o, lse = lse_merge(o, lse, o_c, lse_c)
    return o, lse


def bwd_delta(o, do):
    """delta[b, h, i] = sum_d dO[b, i, h, :] * O[b, i, h, :] (rowsum of dO o O)."""
    return np.transpose(np.sum(_f64(do) * _f64(o), axis=-1), (0, 2, 1))


def attention_bwd_rows(q, k, v, do, lse, delta, q_idx, k_idx, scale, causal,
                       seg_q=None, seg_k=None):
    """Gradient contributions of one key set, for one batch row, given the FINAL
    log-sum-exp of every query row.

    P_ij = exp(s_ij - LSE_i) on allowed pairs (0 elsewhere);
    dV_g  += P^T dO_h;   dP = dO_h V_g^T;   dS = P o (dP - delta);
    dQ_h  += scale dS K_g;   dK_g += scale dS^T Q_h   (summed over the q-heads of g).

    q, do [Nq, Hq, d]; k, v [Nk, Hkv, d]; lse, delta [Hq, Nq].
    Returns (dQ [Nq, Hq, d], dK [Nk, Hkv, d], dV [Nk, Hkv, d]).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    lse, delta = _f64(lse), _f64(delta)
    Nq, Hq, d = q.shape
    Nk, Hkv, _ = k.shape
    group = Hq // Hkv
    dq = np.zeros((Nq, Hq, d))
    dk = np.zeros((Nk, Hkv, d))
    dv = np.zeros((Nk, Hkv, d))
    if Nq == 0 or Nk == 0:
        return dq, dk, dv
    q_idx = np.asarray(q_idx)
    seg_q_arr = None if seg_q is None else np.asarray(seg_q)
    for r0 in range(0, Nq, ROW_BLOCK):
        rows = slice(r0, min(Nq, r0 + ROW_BLOCK))
        mask = allowed_mask(q_idx[rows], k_idx, causal,
                            None if seg_q_arr is None else seg_q_arr[rows], seg_k)
        if not mask.any():
            continue  # no visible pair in this block: no contribution
        for h in range(Hq):
            g = h // group
            s = scale * (q[rows, h, :] @ k[:, g, :].T)
            p = np.where(mask, np.exp(np.where(mask, s, 0.0) - lse[h, rows][:, None]), 0.0)
            dv[:, g, :] += p.T @ do[rows, h, :]
            dp = do[rows, h, :] @ v[:, g, :].T
            ds = p * (dp - delta[h, rows][:, None])
            dq[rows, h, :] += scale * (ds @ k[:, g, :])
            dk[:, g, :] += scale * (ds.T @ q[rows, h, :])
    return dq, dk, dv


def attention_bwd_full(q, k, v, do, lse, delta, q_idx, k_idx, scale, causal,
                       seg_q=None, seg_k=None):
    """Batched wrapper of :func:`attention_bwd_rows`."""
    B = np.shape(q)[0]
    res = [attention_bwd_rows(q[b], k[b], v[b], do[b], lse[b], delta[b], q_idx, k_idx,
                              scale, causal,
                              None if seg_q is None else seg_q[b],
                              None if seg_k is None else seg_k[b]) for b in range(B)]
    return tuple(np.stack([r[i] for r in res]) for i in range(3))


def ring_backward(q_loc, k_chunks, v_chunks, o, lse, do, rank, cp, scale, causal, seg=None):
    """Backward of the local share, step by step in ring order.

    Uses the final merged (O, LSE) of the forward.  Returns dQ [B, C, Hq, d] (summed
    over all chunks) and per-chunk dK, dV lists (index = chunk id) holding this
    rank's contribution to every chunk's gradient.
    """
    q_loc = _f64(q_loc)
    B, C, Hq, d = q_loc.shape
    delta = bwd_delta(o, do)
    q_idx = rank * C + np.arange(C)
    dq = np.zeros((B, C, Hq, d))
    dks = [None] * cp
    dvs = [None] * cp
    for c in ring_schedule(rank, cp):
        k_idx = c * C + np.arange(C)
        seg_q = None if seg is None else seg[:, rank * C:(rank + 1) * C]
        seg_k = None if seg is None else seg[:, c * C:(c + 1) * C]
        dq_c, dks[c], dvs[c] = attention_bwd_full(q_loc, k_chunks[c], v_chunks[c], do, lse,
                                                  delta, q_idx, k_idx, scale, causal,
                                                  seg_q, seg_k)
        dq += dq_c
    return dq, dks, dvs


def live_pairs(q_idx, k_idx, causal, seg_q=None, seg_k=None) -> int:
    """Number of allowed (query, key) pairs: the unit of algorithmic work."""
    total = 0
    q_idx = np.asarray(q_idx)
    for r0 in range(0, q_idx.size, 4096):
        rows = slice(r0, r0 + 4096)
        total += int(allowed_mask(q_idx[rows], k_idx, causal,
                                  None if seg_q is None else np.asarray(seg_q)[rows],
                                  seg_k).sum())
    return total
