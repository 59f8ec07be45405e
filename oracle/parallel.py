"""Runs the fp64 oracle one query head at a time in a thread pool.

TEST INFRASTRUCTURE (like the rest of ``oracle/``): used by the full-size parity
tests and the ``cpu_baseline`` leg of ``bench.py`` only.

Attention is computed independently per query head (query head h reads KV head
h // (Hq // Hkv)), so calling the oracle on one head and its KV head at a time and
putting the results back together gives exactly what one call over all heads
gives; the only sum across heads is the GQA reduction of dK/dV, which the
definition states (dK_g, dV_g sum the contributions of every query head of group
g).  numpy releases the GIL inside BLAS calls and ufunc loops, so the heads run
in parallel on the host cores.  Nothing here changes the oracle's arithmetic.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from contextlib import nullcontext

import numpy as np

from .attention import attention_bwd_full, attention_full, ring_backward, ring_forward


def affinity_cores() -> int:
    """Cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def host_cores() -> int:
    """Worker threads to use: the affinity set, capped by OMP_NUM_THREADS when the
    environment sets it (a machine may give this process a share of its cores)."""
    n = affinity_cores()
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def blas_info() -> str:
    try:
        from threadpoolctl import threadpool_info

        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            return f"{infos[0].get('internal_api', '?')} {infos[0].get('version', '')}".strip()
    except Exception:  # noqa: BLE001 - optional dependency
        pass
    return "unknown"


def _single_thread_blas(workers: int):
    """With one worker per core, each worker's BLAS calls run on one thread."""
    if workers <= 1:
        return nullcontext()
    try:
        from threadpoolctl import threadpool_limits

        return threadpool_limits(limits=1, user_api="blas")
    except Exception:  # noqa: BLE001
        return nullcontext()


def map_heads(fn, heads, workers=None):
    """[fn(h) for h in heads], run in a pool of `workers` threads (default: host cores)."""
    heads = list(heads)
    workers = max(1, min(len(heads), workers or host_cores()))
    if workers == 1:
        return [fn(h) for h in heads]
    with _single_thread_blas(workers), ThreadPoolExecutor(max_workers=workers) as pool:
        return list(pool.map(fn, heads))


def _head(x, h):
    return x[:, :, h:h + 1]


def attention_full_heads(q, k, v, q_idx, k_idx, scale, causal, seg_q=None, seg_k=None, heads=None,
                         workers=None):
    """``attention_full`` for the query heads in `heads` (default: all).  Returns
    (O [B, Nq, len(heads), d], LSE [B, len(heads), Nq]) in the order of `heads`."""
    Hq, Hkv = q.shape[2], k.shape[2]
    group = Hq // Hkv
    heads = list(range(Hq)) if heads is None else list(heads)

    def one(h):
        g = h // group
        return attention_full(_head(q, h), _head(k, g), _head(v, g), q_idx, k_idx, scale, causal, seg_q, seg_k)

    res = map_heads(one, heads, workers)
    return np.concatenate([r[0] for r in res], axis=2), np.concatenate([r[1] for r in res], axis=1)


def attention_bwd_full_heads(q, k, v, do, lse, delta, q_idx, k_idx, scale, causal, seg_q=None, seg_k=None,
                             kv_heads=None, workers=None):
    """``attention_bwd_full`` for every query head of the KV heads in `kv_heads`
    (default: all).  lse, delta: [B, Hq, Nq] for all heads.  Returns dQ [B, Nq,
    len(kv_heads) * group, d] (those query heads, in order) and dK, dV [B, Nk,
    len(kv_heads), d]."""
    Hq, Hkv = q.shape[2], k.shape[2]
    group = Hq // Hkv
    kv_heads = list(range(Hkv)) if kv_heads is None else list(kv_heads)
    heads = [g * group + j for g in kv_heads for j in range(group)]

    def one(h):
        g = h // group
        return attention_bwd_full(_head(q, h), _head(k, g), _head(v, g), _head(do, h), lse[:, h:h + 1],
                                  delta[:, h:h + 1], q_idx, k_idx, scale, causal, seg_q, seg_k)

    res = map_heads(one, heads, workers)
    dq = np.concatenate([r[0] for r in res], axis=2)
    dk = np.concatenate([sum(res[i * group + j][1] for j in range(group)) for i in range(len(kv_heads))], axis=2)
    dv = np.concatenate([sum(res[i * group + j][2] for j in range(group)) for i in range(len(kv_heads))], axis=2)
    return dq, dk, dv


def ring_forward_heads(q_loc, k_chunks, v_chunks, rank, cp, scale, causal, seg=None, workers=None):
    """``ring_forward`` (the chunked, merged form) run per query head."""
    Hq, Hkv = q_loc.shape[2], k_chunks[0].shape[2]
    group = Hq // Hkv

    def one(h):
        g = h // group
        return ring_forward(_head(q_loc, h), [_head(x, g) for x in k_chunks], [_head(x, g) for x in v_chunks],
                            rank, cp, scale, causal, seg)

    res = map_heads(one, range(Hq), workers)
    return np.concatenate([r[0] for r in res], axis=2), np.concatenate([r[1] for r in res], axis=1)


def ring_backward_heads(q_loc, k_chunks, v_chunks, o, lse, do, rank, cp, scale, causal, seg=None, workers=None):
    """``ring_backward`` run per query head; dK/dV of each chunk summed over the query
    heads of each KV head's group."""
    Hq, Hkv = q_loc.shape[2], k_chunks[0].shape[2]
    group = Hq // Hkv

    def one(h):
        g = h // group
        return ring_backward(_head(q_loc, h), [_head(x, g) for x in k_chunks], [_head(x, g) for x in v_chunks],
                             _head(o, h), lse[:, h:h + 1], _head(do, h), rank, cp, scale, causal, seg)

    res = map_heads(one, range(Hq), workers)
    dq = np.concatenate([r[0] for r in res], axis=2)
    dks, dvs = [], []
    for c in range(cp):
        dks.append(np.concatenate([sum(res[g * group + j][1][c] for j in range(group)) for g in range(Hkv)],
                                  axis=2))
        dvs.append(np.concatenate([sum(res[g * group + j][2][c] for j in range(group)) for g in range(Hkv)],
                                  axis=2))
    return dq, dks, dvs
