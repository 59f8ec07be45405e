"""The per-head thread-pool runner gives what the oracle gives in one call (CPU)."""

import numpy as np

import oracle
from oracle import parallel as opar


def _data(rng, B=1, S=96, Hq=6, Hkv=2, d=8):
    q = rng.standard_normal((B, S, Hq, d))
    k = rng.standard_normal((B, S, Hkv, d))
    v = rng.standard_normal((B, S, Hkv, d))
    do = rng.standard_normal((B, S, Hq, d))
    return q, k, v, do


def test_forward_per_head_equals_one_call(rng):
    q, k, v, _ = _data(rng)
    idx = np.arange(q.shape[1])
    o, l = oracle.attention_full(q, k, v, idx, idx, 0.3, True)
    o2, l2 = opar.attention_full_heads(q, k, v, idx, idx, 0.3, True, workers=3)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    o3, l3 = opar.attention_full_heads(q, k, v, idx, idx, 0.3, True, heads=[5, 0])
    np.testing.assert_array_equal(o3, o[:, :, [5, 0]])
    np.testing.assert_array_equal(l3, l[:, [5, 0]])


def test_backward_per_head_equals_one_call(rng):
    q, k, v, do = _data(rng)
    idx = np.arange(q.shape[1])
    o, l = oracle.attention_full(q, k, v, idx, idx, 0.3, True)
    delta = oracle.bwd_delta(o, do)
    dq, dk, dv = oracle.attention_bwd_full(q, k, v, do, l, delta, idx, idx, 0.3, True)
    dq2, dk2, dv2 = opar.attention_bwd_full_heads(q, k, v, do, l, delta, idx, idx, 0.3, True, workers=4)
    # per-head sums of the GQA group are added in another order: rounding only
    np.testing.assert_allclose(dq2, dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk2, dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, rtol=0, atol=1e-12)
    dq3, dk3, dv3 = opar.attention_bwd_full_heads(q, k, v, do, l, delta, idx, idx, 0.3, True, kv_heads=[1])
    np.testing.assert_allclose(dq3, dq[:, :, 3:6], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk3, dk[:, :, 1:2], rtol=0, atol=1e-12)


def test_ring_per_head_equals_one_call(rng):
    q, k, v, do = _data(rng, S=64)
    cp, rank, C = 4, 2, 16
    kc = [k[:, c * C:(c + 1) * C] for c in range(cp)]
    vc = [v[:, c * C:(c + 1) * C] for c in range(cp)]
    ql, dol = q[:, rank * C:(rank + 1) * C], do[:, rank * C:(rank + 1) * C]
    o, l = oracle.ring_forward(ql, kc, vc, rank, cp, 0.5, True)
    o2, l2 = opar.ring_forward_heads(ql, kc, vc, rank, cp, 0.5, True, workers=2)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    dq, dks, dvs = oracle.ring_backward(ql, kc, vc, o, l, dol, rank, cp, 0.5, True)
    dq2, dks2, dvs2 = opar.ring_backward_heads(ql, kc, vc, o, l, dol, rank, cp, 0.5, True, workers=2)
    np.testing.assert_allclose(dq2, dq, rtol=0, atol=1e-12)
    for c in range(cp):
        np.testing.assert_allclose(dks2[c], dks[c], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dvs2[c], dvs[c], rtol=0, atol=1e-12)
