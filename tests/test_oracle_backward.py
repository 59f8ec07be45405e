"""Pins of the oracle's backward pass (CPU only): central finite differences of the
forward definition, a hand-derived example (in test_oracle_merge), closed
identities of softmax-attention gradients, and cross-rank reconstruction."""

import math

import numpy as np
import pytest

import oracle


def _pos(rng, S):
    row = []
    while len(row) < S:
        n = int(rng.integers(1, max(2, S // 2) + 1))
        row.extend(range(n))
    return np.asarray([row[:S]], dtype=np.int32)


def _setup(seed, S, CP, Hq, Hkv, d, packed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, S, Hq, d))
    k = rng.standard_normal((1, S, Hkv, d))
    v = rng.standard_normal((1, S, Hkv, d))
    do = rng.standard_normal((1, S // CP, Hq, d))
    seg = oracle.segment_ids(_pos(rng, S)) if packed else None
    return q, k, v, do, seg


def _ring_grads(q, k, v, do, seg, r, CP, scale):
    S = q.shape[1]
    C = S // CP
    q_loc = q[:, r * C:(r + 1) * C]
    kc = [k[:, c * C:(c + 1) * C] for c in range(CP)]
    vc = [v[:, c * C:(c + 1) * C] for c in range(CP)]
    o, lse = oracle.ring_forward(q_loc, kc, vc, r, CP, scale, True, seg)
    dq, dks, dvs = oracle.ring_backward(q_loc, kc, vc, o, lse, do, r, CP, scale, True, seg)
    return o, lse, dq, np.concatenate(dks, axis=1), np.concatenate(dvs, axis=1)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2)])
def test_ring_backward_matches_finite_differences(packed, Hq, Hkv):
    S, CP, d = 8, 4, 3
    scale = 1 / math.sqrt(d)
    q, k, v, do, seg = _setup(100 + Hq + 10 * packed, S, CP, Hq, Hkv, d, packed)
    C = S // CP
    for r in (1, 3):
        _, _, dq, dk, dv = _ring_grads(q, k, v, do, seg, r, CP, scale)
        q_idx = r * C + np.arange(C)
        sq = None if seg is None else seg[:, r * C:(r + 1) * C]

        def loss(qq, kk, vv):
            o, _ = oracle.attention_full(qq, kk, vv, q_idx, np.arange(S), scale, True, sq, seg)
            return float(np.sum(do * o))

        h = 1e-6
        q_loc = q[:, r * C:(r + 1) * C].copy()
        for name, x, g in (("q", q_loc, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = {"q": q_loc, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name] = xp
                args_m[name] = xm
                fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                           - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=f"d{name} rank {r}")


@pytest.mark.parametrize("packed", [False, True])
def test_gradient_identities(packed):
    """Per KV head (summed over its query heads and over every chunk):
    sum over keys of dK = 0 (each row of dS sums to 0), sum over keys of dV = sum over
    queries of dO (rows of P sum to 1), and <dQ, Q> = <dK, K> (both equal sum dS*s)."""
    S, CP, Hq, Hkv, d = 48, 4, 4, 2, 8
    scale = 1 / math.sqrt(d)
    q, k, v, do, seg = _setup(7 + packed, S, CP, Hq, Hkv, d, packed)
    C = S // CP
    group = Hq // Hkv
    for r in range(CP):
        _, _, dq, dk, dv = _ring_grads(q, k, v, do, seg, r, CP, scale)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        for g in range(Hkv):
            np.testing.assert_allclose(dv[0, :, g].sum(axis=0),
                                       do[0, :, g * group:(g + 1) * group].sum(axis=(0, 1)), atol=1e-12)
        lhs = float(np.sum(dq * q[:, r * C:(r + 1) * C]))
        rhs = float(np.sum(dk * k))
        assert abs(lhs - rhs) < 1e-11 * max(1.0, abs(lhs))


@pytest.mark.parametrize("packed", [False, True])
def test_sum_over_ranks_gives_full_sequence_gradient(packed):
    """dK/dV contributions of every rank, summed, equal the gradient of attention over
    the whole row; every rank's dQ equals the corresponding rows of the full dQ."""
    S, CP, Hq, Hkv, d = 32, 4, 4, 1, 4
    scale = 0.5
    rng = np.random.default_rng(31 + packed)
    q = rng.standard_normal((1, S, Hq, d))
    k = rng.standard_normal((1, S, Hkv, d))
    v = rng.standard_normal((1, S, Hkv, d))
    do_full = rng.standard_normal((1, S, Hq, d))
    seg = oracle.segment_ids(_pos(rng, S)) if packed else None
    o, lse = oracle.attention_full(q, k, v, np.arange(S), np.arange(S), scale, True, seg, seg)
    delta = oracle.bwd_delta(o, do_full)
    dq_f, dk_f, dv_f = oracle.attention_bwd_full(q, k, v, do_full, lse, delta, np.arange(S),
                                                 np.arange(S), scale, True, seg, seg)
    C = S // CP
    dk_sum = np.zeros_like(dk_f)
    dv_sum = np.zeros_like(dv_f)
    for r in range(CP):
        sl = slice(r * C, (r + 1) * C)
        _, _, dq, dk, dv = _ring_grads(q, k, v, do_full[:, sl], seg, r, CP, scale)
        np.testing.assert_allclose(dq, dq_f[:, sl], atol=1e-12)
        dk_sum += dk
        dv_sum += dv
    np.testing.assert_allclose(dk_sum, dk_f, atol=1e-12)
    np.testing.assert_allclose(dv_sum, dv_f, atol=1e-12)


def test_future_chunk_contributes_nothing():
    """Under causal masking, a chunk after the local shard gets zero gradient."""
    S, CP, Hq, Hkv, d = 16, 4, 2, 1, 4
    q, k, v, do, _ = _setup(5, S, CP, Hq, Hkv, d, False)
    _, _, _, dk, dv = _ring_grads(q, k, v, do, None, 1, CP, 0.5)
    assert np.all(dk[:, 8:] == 0) and np.all(dv[:, 8:] == 0)
