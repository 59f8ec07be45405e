"""GPU parity of each C-ABI entry point against the fp64 oracle on small seeded inputs
that span several tiles and ragged tails (sizes that are not tile multiples)."""

import math

import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_round
from tests.gpu_util import device, lib, lse_close, max_abs, rel_to_max, report, to_dev, to_np

pytestmark = pytest.mark.gpu


def _qkv(rng, B, Sq, Sk, Hq, Hkv, d, dtype):
    q = rng.standard_normal((B, Sq, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, Sk, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, Sk, Hkv, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v


def _packed_pos(rng, B, S, lo, hi, mid_start=False):
    rows = []
    for _ in range(B):
        row = list(range(3, 3 + int(rng.integers(lo, hi)))) if mid_start else []
        while len(row) < S:
            row.extend(range(int(rng.integers(lo, hi + 1))))
        rows.append(row[:S])
    return np.asarray(rows, dtype=np.int32)


TD = {"bf16": torch.bfloat16, "f32": torch.float32}


# ---- segment ids -------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,lo,hi,mid", [(1, 16384, 512, 4096, False), (3, 5000, 1, 50, True),
                                           (2, 1, 1, 1, False), (1, 100003, 1, 700, True),
                                           (2, 4097, 4097, 4097, False)])
def test_segment_mask_from_pos_bit_exact(B, S, lo, hi, mid):
    ra = lib()
    rng = np.random.default_rng(S + B)
    pos = _packed_pos(rng, B, S, lo, hi, mid)
    seg = torch.empty((B, S), dtype=torch.int32, device=device())
    ra.segment_mask_from_pos(to_dev(pos, torch.int32), seg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(seg.cpu().numpy(), oracle.segment_ids(pos))


# ---- merge -----------------------------------------------------------------------------------

# (1, 9, 100, 12): a head's 3 vectors straddle waves and passes of the per-row loop
# (300 vectors per row > 256 threads), so the running LSE must be read by every
# thread of a head before it is overwritten.
@pytest.mark.parametrize("B,Sq,Hq,d", [(1, 300, 4, 128), (2, 77, 3, 64), (1, 5, 1, 4), (1, 9, 100, 12)])
def test_lse_merge(B, Sq, Hq, d):
    ra = lib()
    rng = np.random.default_rng(Sq)
    o1 = rng.standard_normal((B, Sq, Hq, d)).astype(np.float32)
    o2 = rng.standard_normal((B, Sq, Hq, d)).astype(np.float32)
    l1 = (rng.standard_normal((B, Hq, Sq)) * 4 + 9).astype(np.float32)
    l2 = (rng.standard_normal((B, Hq, Sq)) * 4 + 9).astype(np.float32)
    # some rows dead in one or both partials (their O is 0 by the step contract)
    dead1 = rng.random((B, Hq, Sq)) < 0.2
    dead2 = rng.random((B, Hq, Sq)) < 0.2
    l1[dead1] = -np.inf
    l2[dead2] = -np.inf
    o1[np.transpose(dead1, (0, 2, 1))] = 0
    o2[np.transpose(dead2, (0, 2, 1))] = 0
    o_ref, l_ref = oracle.lse_merge(o1, l1, o2, l2)
    oa, la = to_dev(o1, torch.float32), to_dev(l1, torch.float32)
    out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=device())
    ra.lse_merge(oa, la, to_dev(o2, torch.float32), to_dev(l2, torch.float32), o_out=out)
    torch.cuda.synchronize()
    err = max_abs(to_np(oa), o_ref)
    lse_close(to_np(la), l_ref, 1e-5)
    report("lse_merge", o_err=err)
    assert err <= 1e-5
    # bf16 output is the RNE rounding of the merged fp32 O
    np.testing.assert_array_equal(out.float().cpu().numpy(), bf16_round(oa.cpu().numpy()))
    # rows dead in both partials are untouched
    both = np.transpose(dead1 & dead2, (0, 2, 1))
    assert np.all(to_np(oa)[both] == 0)


def test_lse_merge_with_dead_step_is_identity_bitwise():
    ra = lib()
    rng = np.random.default_rng(3)
    o1 = rng.standard_normal((1, 64, 2, 128)).astype(np.float32)
    l1 = rng.standard_normal((1, 2, 64)).astype(np.float32)
    oa, la = to_dev(o1, torch.float32), to_dev(l1, torch.float32)
    os_ = torch.zeros_like(oa)
    ls = torch.full_like(la, -math.inf)
    ra.lse_merge(oa, la, os_, ls)
    torch.cuda.synchronize()
    assert np.array_equal(oa.cpu().numpy(), o1) and np.array_equal(la.cpu().numpy(), l1)


def test_lse_merge_convert_only():
    ra = lib()
    rng = np.random.default_rng(4)
    o1 = rng.standard_normal((2, 33, 3, 64)).astype(np.float32)
    oa = to_dev(o1, torch.float32)
    la = torch.zeros((2, 3, 33), dtype=torch.float32, device=device())
    out = torch.empty((2, 33, 3, 64), dtype=torch.bfloat16, device=device())
    ra.lse_merge(oa, la, None, None, o_out=out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.float().cpu().numpy(), bf16_round(o1))


# ---- preprocess ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_bwd_preprocess(dtype, d):
    ra = lib()
    rng = np.random.default_rng(d)
    B, Sq, Hq = 2, 131, 3
    o = rng.standard_normal((B, Sq, Hq, d), dtype=np.float32)
    do = rng.standard_normal((B, Sq, Hq, d), dtype=np.float32)
    if dtype == "bf16":
        o, do = bf16_round(o), bf16_round(do)
    delta = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device())
    ra.ring_attn_bwd_preprocess(to_dev(o, TD[dtype]), to_dev(do, TD[dtype]), delta)
    torch.cuda.synchronize()
    err = max_abs(delta.cpu().numpy(), oracle.bwd_delta(o, do))
    assert err <= 1e-4 * math.sqrt(d)


# ---- one forward step ----------------------------------------------------------------------

STEP_CASES = [
    # (dtype, B, Sq, Sk, Hq, Hkv, d, q_off, kv_off, causal, packed)
    ("f32", 1, 256, 256, 1, 1, 64, 768, 512, True, False),
    ("f32", 1, 256, 256, 1, 1, 64, 768, 768, True, False),
    ("bf16", 1, 300, 200, 4, 2, 128, 500, 400, True, False),     # ragged, partly in the future
    ("bf16", 2, 130, 190, 4, 1, 128, 0, 0, False, False),        # non-causal, GQA 4:1, B=2
    ("bf16", 1, 257, 129, 2, 2, 64, 1000, 2000, True, False),    # chunk fully in the future
    ("bf16", 1, 200, 333, 6, 3, 64, 333, 0, True, False),
    ("f32", 2, 97, 150, 2, 1, 128, 150, 0, True, False),
    ("bf16", 1, 384, 384, 4, 2, 128, 384, 384, True, True),      # packed, diagonal chunk
    ("bf16", 2, 256, 320, 4, 4, 128, 640, 320, True, True),      # packed, earlier chunk
    ("f32", 1, 160, 96, 2, 1, 64, 256, 0, False, True),          # packed, non-causal
]


# Backward steps whose dK/dV grid (B * Hkv * ceil(Sk / 256) workgroups of 256 keys)
# reaches 256, the size at which the bf16 d=128 backward runs 64 keys per wave.
WIDE_BWD_CASES = [
    ("bf16", 1, 333, 800, 128, 64, 128, 900, 300, True, False),   # diagonal, ragged on both sides
    ("bf16", 2, 200, 1000, 64, 32, 128, 1000, 0, True, False),    # earlier chunk, ragged key tail
    ("bf16", 1, 150, 777, 256, 64, 128, 0, 0, False, False),      # non-causal, GQA 4:1
    ("bf16", 1, 512, 1024, 128, 64, 128, 512, 0, True, True),     # packed, diagonal chunk
    ("bf16", 1, 300, 1000, 64, 64, 128, 0, 1000, False, True),    # packed, non-causal
    ("bf16", 1, 100, 1024, 128, 64, 128, 0, 2048, True, False),   # chunk in the future: no live pair
    # dQ grid (B * Hkv * (group / h) * ceil(Sq / (256 / h)) workgroups, h = query heads per
    # workgroup: 4, 2 or 1 by the GQA group) also at 256 or more: 64 queries per wave
    ("bf16", 2, 500, 2000, 64, 16, 128, 1900, 300, True, False),  # group 4, diagonal, ragged
    ("bf16", 1, 1000, 1024, 128, 64, 128, 1024, 0, True, False),  # group 2, earlier chunk
    ("bf16", 1, 1000, 1100, 64, 64, 128, 0, 0, False, False),     # group 1, non-causal
    ("bf16", 2, 512, 2048, 64, 16, 128, 1536, 0, True, True),     # group 4, packed, diagonal
    ("bf16", 1, 1000, 1024, 64, 64, 128, 0, 1024, False, True),   # group 1, packed, non-causal
    ("bf16", 2, 500, 2000, 64, 16, 128, 0, 3000, True, False),    # chunk in the future
]

# Backward steps whose dK/dV workgroups (32 keys per wave) walk only 1, 2 or 3 query
# tiles, so that the copy pipeline runs its prologue alone or one or two loop steps
# (copies planned past the last tile have empty ranges).
SHORT_WALK_BWD_CASES = [
    ("bf16", 1, 64, 256, 2, 2, 128, 0, 0, False, False),      # 1 tile per workgroup
    ("bf16", 1, 128, 200, 2, 2, 128, 0, 0, False, False),     # 2 tiles, ragged key tail
    ("bf16", 1, 150, 128, 4, 4, 128, 0, 0, False, False),     # 3 tiles, ragged query tail
    ("bf16", 2, 64, 64, 8, 2, 128, 64, 64, True, False),      # diagonal, 4 positions (GQA 4:1)
]

# Forward steps on grids of 512 or more workgroups of 64-query waves (B * Hkv * (group
# / h) * ceil(Sq / (256 / h)), h = 4, 2 or 1 query heads per workgroup by the GQA
# group): the size at which the bf16 d=128 forward of packed rows runs 64 queries per
# wave, and wide grids of the 8-wave kernel otherwise.
WIDE_FWD_CASES = [
    ("bf16", 2, 4100, 600, 16, 4, 128, 500, 300, True, False),     # group 4, diagonal, ragged
    ("bf16", 1, 8200, 500, 16, 8, 128, 0, 0, False, False),        # group 2, non-causal
    ("bf16", 2, 4100, 700, 16, 16, 128, 4000, 3900, True, False),  # group 1, diagonal
    ("bf16", 2, 4100, 1000, 16, 4, 128, 1000, 0, True, True),      # group 4, packed, earlier chunk
    ("bf16", 1, 4096, 512, 32, 8, 128, 0, 5000, True, False),      # chunk in the future
]


# Packed rows with long samples (lengths drawn from the given range): whole query
# tiles and key blocks inside one sample, which run without the segment test.
LONG_SEG_CASES = [
    ("bf16", 1, 1024, 2048, 32, 8, 128, 2048, 0, True, (300, 1200)),    # earlier chunk
    ("bf16", 1, 1024, 1024, 32, 8, 128, 1024, 1024, True, (300, 1200)),  # diagonal chunk
    ("bf16", 2, 1000, 1100, 16, 4, 128, 1100, 0, True, (150, 900)),     # ragged tails
]
# Long samples on the wide grids: the forward's 64-query waves (unmasked tiles inside
# a sample), the 64-key dK/dV and 64-query dQ waves (sample spans from wave-wide
# searches).
WIDE_LONG_SEG_CASES = [
    ("bf16", 1, 4096, 2048, 32, 8, 128, 4096, 2048, True, (300, 1500)),  # forward, diagonal chunk
    ("bf16", 1, 512, 1024, 128, 64, 128, 512, 0, True, (300, 1500)),     # dK/dV 64 keys per wave
    ("bf16", 2, 512, 2048, 64, 16, 128, 1536, 0, True, (300, 1500)),     # dQ 64 queries per wave
]


def _step_case(case, seed):
    dtype, B, Sq, Sk, Hq, Hkv, d, q_off, kv_off, causal, packed = case
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, B, Sq, Sk, Hq, Hkv, d, dtype)
    S = max(q_off + Sq, kv_off + Sk)
    lo, hi = (20, 200) if packed is True else (packed or (0, 0))
    seg = oracle.segment_ids(_packed_pos(rng, B, S, lo, hi)) if packed else None
    return q, k, v, seg, S


@pytest.mark.parametrize("case", STEP_CASES + WIDE_FWD_CASES + LONG_SEG_CASES + WIDE_LONG_SEG_CASES[:1],
                         ids=lambda c: "-".join(map(str, c)))
def test_fwd_step_partial(case):
    ra = lib()
    dtype, B, Sq, Sk, Hq, Hkv, d, q_off, kv_off, causal, packed = case
    q, k, v, seg, S = _step_case(case, 17 + Sq + Sk)
    scale = 1 / math.sqrt(d)
    o_ref, l_ref = oracle.attention_full(q, k, v, q_off + np.arange(Sq), kv_off + np.arange(Sk), scale, causal,
                                         None if seg is None else seg[:, q_off:q_off + Sq],
                                         None if seg is None else seg[:, kv_off:kv_off + Sk])
    o = torch.full((B, Sq, Hq, d), float("nan"), dtype=torch.float32, device=device())
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=device())
    ra.ring_attn_fwd_step(to_dev(q, TD[dtype]), to_dev(k, TD[dtype]), to_dev(v, TD[dtype]), o, lse,
                          q_offset=q_off, kv_offset=kv_off, causal=causal, scale=scale,
                          seg_ids=None if seg is None else to_dev(seg, torch.int32))
    torch.cuda.synchronize()
    on, ln = to_np(o), to_np(lse)
    tol_o, tol_l = (1e-4, 1e-4) if dtype == "f32" else (2e-2, 1e-3)
    err_o = max_abs(on, o_ref)
    err_l = lse_close(ln, l_ref, tol_l)
    report("fwd_step", case=case, o_err=err_o, lse_err=err_l, o_rel=rel_to_max(on, o_ref))
    assert err_o <= tol_o
    if dtype == "bf16":
        assert rel_to_max(on, o_ref) <= 2e-2
    # rows without a visible key are exactly the merge identity
    dead = ~np.isfinite(l_ref)
    assert np.all(on[np.transpose(dead, (0, 2, 1))] == 0)


@pytest.mark.parametrize("case", STEP_CASES + WIDE_BWD_CASES + SHORT_WALK_BWD_CASES + LONG_SEG_CASES +
                         WIDE_LONG_SEG_CASES[1:], ids=lambda c: "-".join(map(str, c)))
def test_bwd_step(case):
    """One backward step with the oracle's own final LSE/delta as inputs: dQ, dK, dV."""
    ra = lib()
    dtype, B, Sq, Sk, Hq, Hkv, d, q_off, kv_off, causal, packed = case
    q, k, v, seg, S = _step_case(case, 91 + Sq + Sk)
    rng = np.random.default_rng(5 + Sq)
    do = rng.standard_normal((B, Sq, Hq, d), dtype=np.float32)
    if dtype == "bf16":
        do = bf16_round(do)
    scale = 1 / math.sqrt(d)
    # a "final" LSE from another key set so that rows are never empty: the chunk plus
    # the query's own position (the diagonal key)
    seg_q = None if seg is None else seg[:, q_off:q_off + Sq]
    seg_k = None if seg is None else seg[:, kv_off:kv_off + Sk]
    o_c, l_c = oracle.attention_full(q, k, v, q_off + np.arange(Sq), kv_off + np.arange(Sk), scale, causal,
                                     seg_q, seg_k)
    lse_fin = np.logaddexp(np.where(np.isfinite(l_c), l_c, -np.inf), rng.standard_normal(l_c.shape) + 2.0)
    delta = rng.standard_normal((B, Hq, Sq)) * 0.1
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd_full(q, k, v, do, lse_fin, delta, q_off + np.arange(Sq),
                                                       kv_off + np.arange(Sk), scale, causal, seg_q, seg_k)
    # accumulators start non-zero to check the += contract
    dq0 = rng.standard_normal((B, Sq, Hq, d)).astype(np.float32)
    dk0 = rng.standard_normal((B, Sk, Hkv, d)).astype(np.float32)
    dv0 = rng.standard_normal((B, Sk, Hkv, d)).astype(np.float32)
    dq, dk, dv = to_dev(dq0, torch.float32), to_dev(dk0, torch.float32), to_dev(dv0, torch.float32)
    ra.ring_attn_bwd_step(to_dev(q, TD[dtype]), to_dev(k, TD[dtype]), to_dev(v, TD[dtype]), to_dev(do, TD[dtype]),
                          to_dev(lse_fin.astype(np.float32), torch.float32),
                          to_dev(delta.astype(np.float32), torch.float32), dq, dk, dv,
                          q_offset=q_off, kv_offset=kv_off, causal=causal, scale=scale,
                          seg_ids=None if seg is None else to_dev(seg, torch.int32))
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "f32" else 3e-2
    errs = {}
    for name, got, g0, ref in (("dq", dq, dq0, dq_ref), ("dk", dk, dk0, dk_ref), ("dv", dv, dv0, dv_ref)):
        inc = to_np(got) - g0
        if np.max(np.abs(ref)) == 0:
            errs[name] = max_abs(inc, ref)
            assert errs[name] <= 1e-6
        else:
            errs[name] = rel_to_max(inc, ref)
            assert errs[name] <= tol, (name, errs[name])
    report("bwd_step", case=case, **errs)


@pytest.mark.parametrize("gain,causal,Sq,Sk,q_off,kv_off", [(3.0, True, 320, 320, 640, 640),
                                                             (3.0, False, 200, 450, 0, 0),
                                                             (5.0, True, 256, 384, 384, 0)])
def test_step_with_peaked_scores(gain, causal, Sq, Sk, q_off, kv_off):
    """Scores with a standard deviation of gain**2 (up to ~10x the N(0,1) case): the
    forward's running maximum jumps by many binades from tile to tile (its lazy
    rescale fires repeatedly) and P is nearly one-hot.  Forward O/LSE and the
    backward gradients (from that forward's own LSE) against the oracle."""
    ra = lib()
    rng = np.random.default_rng(int(gain * 100) + Sq)
    B, Hq, Hkv, d = 1, 4, 2, 128
    q = bf16_round(gain * rng.standard_normal((B, Sq, Hq, d), dtype=np.float32))
    k = bf16_round(gain * rng.standard_normal((B, Sk, Hkv, d), dtype=np.float32))
    v = bf16_round(rng.standard_normal((B, Sk, Hkv, d), dtype=np.float32))
    do = bf16_round(rng.standard_normal((B, Sq, Hq, d), dtype=np.float32))
    scale = 1 / math.sqrt(d)
    qpos, kpos = q_off + np.arange(Sq), kv_off + np.arange(Sk)
    o_ref, l_ref = oracle.attention_full(q, k, v, qpos, kpos, scale, causal, None, None)
    qd, kd, vd = to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16)
    o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=device())
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device())
    ra.ring_attn_fwd_step(qd, kd, vd, o, lse, q_offset=q_off, kv_offset=kv_off, causal=causal, scale=scale)
    torch.cuda.synchronize()
    err_o, err_l = max_abs(to_np(o), o_ref), lse_close(to_np(lse), l_ref, 1e-3)
    assert err_o <= 2e-2 and rel_to_max(to_np(o), o_ref) <= 2e-2
    assert err_l <= 1e-3
    live = np.isfinite(l_ref)
    delta = np.einsum("bqhd,bqhd->bhq", o_ref, do)
    lse_fin = np.where(live, l_ref, -np.inf)
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd_full(q, k, v, do, lse_fin, delta, qpos, kpos, scale, causal,
                                                       None, None)
    dq = torch.zeros((B, Sq, Hq, d), dtype=torch.float32, device=device())
    dk = torch.zeros((B, Sk, Hkv, d), dtype=torch.float32, device=device())
    dv = torch.zeros_like(dk)
    ra.ring_attn_bwd_step(qd, kd, vd, to_dev(do, torch.bfloat16), to_dev(lse_fin.astype(np.float32), torch.float32),
                          to_dev(delta.astype(np.float32), torch.float32), dq, dk, dv,
                          q_offset=q_off, kv_offset=kv_off, causal=causal, scale=scale)
    torch.cuda.synchronize()
    errs = {n: rel_to_max(to_np(g), r) for n, g, r in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref))}
    report("peaked_scores", gain=gain, causal=causal, o_err=err_o, lse_err=err_l, **errs)
    for n, e in errs.items():
        assert e <= 3e-2, (n, e)


@pytest.mark.parametrize("out", [None, "same", "f32"])
@pytest.mark.parametrize("case", STEP_CASES + WIDE_FWD_CASES[:1] + WIDE_FWD_CASES[3:4],
                         ids=lambda c: "-".join(map(str, c)))
def test_fwd_step_merge_equals_step_then_merge(case, out):
    """ring_attn_fwd_step_merge gives the same bits as ring_attn_fwd_step followed by
    lse_merge: running result with live rows, rows that have seen no key yet
    (LSE = -inf), and steps whose rows see no key of the chunk."""
    ra = lib()
    dtype, B, Sq, Sk, Hq, Hkv, d, q_off, kv_off, causal, packed = case
    q, k, v, seg, S = _step_case(case, 31 + Sq + Sk)
    rng = np.random.default_rng(7 + Sk)
    o0 = rng.standard_normal((B, Sq, Hq, d)).astype(np.float32)
    l0 = (rng.standard_normal((B, Hq, Sq)) + 3.0).astype(np.float32)
    l0[:, :, ::5] = -np.inf
    qd, kd, vd = to_dev(q, TD[dtype]), to_dev(k, TD[dtype]), to_dev(v, TD[dtype])
    segd = None if seg is None else to_dev(seg, torch.int32)
    kw = dict(q_offset=q_off, kv_offset=kv_off, causal=causal, scale=1 / math.sqrt(d), seg_ids=segd)
    out_dtype = None if out is None else (TD[dtype] if out == "same" else torch.float32)

    def new_out():
        return None if out_dtype is None else torch.full((B, Sq, Hq, d), float("nan"), dtype=out_dtype,
                                                         device=device())

    oa, la, outa = to_dev(o0, torch.float32), to_dev(l0, torch.float32), new_out()
    o_s = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=device())
    l_s = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device())
    ra.ring_attn_fwd_step(qd, kd, vd, o_s, l_s, **kw)
    ra.lse_merge(oa, la, o_s, l_s, o_out=outa)
    ob, lb, outb = to_dev(o0, torch.float32), to_dev(l0, torch.float32), new_out()
    ra.ring_attn_fwd_step_merge(qd, kd, vd, ob, lb, o_out=outb, **kw)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert torch.equal(la, lb)
    if outa is not None:
        assert torch.equal(outa, outb)


WIDE_CASES = [
    # (Sq, Sk, q_off, kv_off, causal): 128 query heads (GQA 16:1) over 8 KV heads, a grid
    # of 64-query waves with four query heads per workgroup.
    (1900, 2100, 2100, 2100, True),   # diagonal chunk, ragged tails on both sides
    (1900, 2100, 2100, 0, True),      # earlier chunk: every block fully visible
    (2048, 1500, 900, 1200, True),    # partly in the future: some rows see nothing
    (2000, 333, 0, 0, False),         # non-causal, short chunk
    (1900, 20, 0, 0, False),          # chunk shorter than one 32-key block of a 64-key tile
    (2048, 40, 2048, 2030, True),     # 40 keys: the tile's second block partly past the chunk end
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_fwd_step_wide_grid(case):
    """A forward step on a wide grid (GQA 16:1): comparison with the oracle on a
    subset of query heads (each head is an independent attention problem over its
    own KV head)."""
    ra = lib()
    Sq, Sk, q_off, kv_off, causal = case
    B, Hq, Hkv, d = 1, 128, 8, 128
    rng = np.random.default_rng(Sq + 7 * Sk + q_off)
    q, k, v = _qkv(rng, B, Sq, Sk, Hq, Hkv, d, "bf16")
    scale = 1 / math.sqrt(d)
    o = torch.full((B, Sq, Hq, d), float("nan"), dtype=torch.float32, device=device())
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=device())
    ra.ring_attn_fwd_step(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), o, lse,
                          q_offset=q_off, kv_offset=kv_off, causal=causal, scale=scale)
    torch.cuda.synchronize()
    on, ln = to_np(o), to_np(lse)
    assert np.all(np.isfinite(on))
    group = Hq // Hkv
    for h in (0, 17, 64, 127):
        kh = h // group
        o_ref, l_ref = oracle.attention_full(q[:, :, h:h + 1], k[:, :, kh:kh + 1], v[:, :, kh:kh + 1],
                                             q_off + np.arange(Sq), kv_off + np.arange(Sk), scale, causal)
        oh, lh = on[:, :, h:h + 1], ln[:, h:h + 1]
        err_o = max_abs(oh, o_ref)
        err_l = lse_close(lh, l_ref, 1e-3)
        report("fwd_step_wide", case=case, head=h, o_err=err_o, lse_err=err_l, o_rel=rel_to_max(oh, o_ref))
        assert err_o <= 2e-2
        assert rel_to_max(oh, o_ref) <= 2e-2
        dead = ~np.isfinite(l_ref)
        assert np.all(oh[np.transpose(dead, (0, 2, 1))] == 0)


def test_fwd_step_is_bitwise_repeatable():
    ra = lib()
    rng = np.random.default_rng(1)
    q, k, v = _qkv(rng, 1, 512, 512, 8, 2, 128, "bf16")
    qd, kd, vd = to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16)
    outs = []
    for _ in range(3):
        o = torch.empty((1, 512, 8, 128), dtype=torch.float32, device=device())
        lse = torch.empty((1, 8, 512), dtype=torch.float32, device=device())
        ra.ring_attn_fwd_step(qd, kd, vd, o, lse, q_offset=512, kv_offset=0, causal=True, scale=0.088)
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


def test_invalid_arguments_enqueue_nothing():
    ra = lib()
    q = torch.zeros((1, 64, 4, 96), dtype=torch.bfloat16, device=device())
    k = torch.zeros((1, 64, 2, 96), dtype=torch.bfloat16, device=device())
    o = torch.zeros((1, 64, 4, 96), dtype=torch.float32, device=device())
    lse = torch.zeros((1, 4, 64), dtype=torch.float32, device=device())
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd_step(q, k, k, o, lse, q_offset=0, kv_offset=0, causal=True, scale=0.1)
    assert e.value.status == 2  # RA_ERR_UNSUPPORTED: head_dim 96
    q = torch.zeros((1, 64, 3, 64), dtype=torch.bfloat16, device=device())
    k = torch.zeros((1, 64, 2, 64), dtype=torch.bfloat16, device=device())
    o = torch.zeros((1, 64, 3, 64), dtype=torch.float32, device=device())
    lse = torch.zeros((1, 3, 64), dtype=torch.float32, device=device())
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd_step(q, k, k, o, lse, q_offset=0, kv_offset=0, causal=True, scale=0.1)
    assert e.value.status == 1  # Hq % Hkv != 0
    seg = torch.zeros((1, 100), dtype=torch.int32, device=device())
    k = torch.zeros((1, 64, 3, 64), dtype=torch.bfloat16, device=device())
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd_step(q, k, k, o, lse, q_offset=64, kv_offset=0, causal=True, scale=0.1, seg_ids=seg)
    assert e.value.status == 1  # q range past seg_len
    assert torch.all(o == 0) and torch.all(lse == 0)


@pytest.mark.parametrize("shift", [1 << 31, (1 << 40) + 12345])
def test_steps_depend_only_on_offset_differences(shift):
    """The causal rule compares global positions, so adding the same amount to both
    offsets (here past 2^31, where the kernels' clamped 32-bit arithmetic must still
    give the exact rule) changes nothing: forward and backward outputs bit-identical."""
    ra = lib()
    rng = np.random.default_rng(77)
    B, Sq, Sk, Hq, Hkv, d = 1, 300, 260, 4, 2, 128
    q, k, v = _qkv(rng, B, Sq, Sk, Hq, Hkv, d, "bf16")
    do = bf16_round(rng.standard_normal((B, Sq, Hq, d), dtype=np.float32))
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    lse_f = to_dev(rng.uniform(4.0, 6.0, (B, Hq, Sq)).astype(np.float32), torch.float32)
    delta = to_dev(0.1 * rng.standard_normal((B, Hq, Sq), dtype=np.float32), torch.float32)
    outs = []
    for base in (0, shift):
        o = torch.empty((B, Sq, Hq, d), dtype=torch.float32, device=device())
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=device())
        ra.ring_attn_fwd_step(qd, kd, vd, o, lse, q_offset=base + 200, kv_offset=base + 100, causal=True,
                              scale=0.088)
        dq = torch.zeros((B, Sq, Hq, d), dtype=torch.float32, device=device())
        dk = torch.zeros((B, Sk, Hkv, d), dtype=torch.float32, device=device())
        dv = torch.zeros_like(dk)
        ra.ring_attn_bwd_step(qd, kd, vd, dod, lse_f, delta, dq, dk, dv, q_offset=base + 200, kv_offset=base + 100,
                              causal=True, scale=0.088)
        outs.append([t.cpu().numpy() for t in (o, lse, dq, dk, dv)])
    for a_, b_ in zip(outs[0], outs[1]):
        assert np.array_equal(a_, b_)
