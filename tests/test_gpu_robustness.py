"""Robustness of the C-ABI entry points on the GPU (no fault is provoked; every input is
valid):

* guard bands: every output is placed inside a larger buffer filled with a sentinel
  pattern, at ragged sizes; the bytes around each output, and every input buffer,
  must be unchanged after the call;
* non-finite inputs: a NaN or Inf in Q, K, V or dO must not crash or hang, must
  reach the outputs that depend on it, and must leave the outputs that do not
  depend on it bit-identical to a clean run (a NaN must never be reported as a row
  that sees no key);
* merge order: the partial results of the ring steps merged in every order agree
  within fp32 rounding, and with the oracle (the merge is exact up to rounding, so
  the order of arrival around the ring must not matter).
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
from synthetic import LLAMA3_8K_FWD, bf16_round, make_workload
from tests.gpu_util import device, lib, lse_close, max_abs, report, to_dev, to_np

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of sentinel on each side of an output
SENTINEL = {torch.float32: 0x7FA5A5A5, torch.bfloat16: 0x7FA5, torch.int32: 0x5A5A5A5A}


class Guarded:
    """A tensor of `shape` placed GUARD bytes into a sentinel-filled buffer."""

    def __init__(self, shape, dtype):
        es = torch.tensor([], dtype=dtype).element_size()
        self.pad = GUARD // es
        self.n = int(np.prod(shape))
        self.buf = torch.empty(self.n + 2 * self.pad, dtype=dtype, device=device())
        ibits = {4: torch.int32, 2: torch.int16}[es]
        self.buf.view(ibits).fill_(SENTINEL[dtype] if SENTINEL[dtype] < 2 ** (8 * es - 1)
                                   else SENTINEL[dtype] - 2 ** (8 * es))
        self.ibits = ibits
        self.t = self.buf[self.pad:self.pad + self.n].view(shape)
        assert self.t.data_ptr() % 256 == 0 or GUARD % 256 == 0

    def guards_intact(self):
        b = self.buf.view(self.ibits)
        ref = b[:1].clone()
        return bool(torch.all(b[:self.pad] == ref)) and bool(torch.all(b[self.pad + self.n:] == ref))


def _bf(x):
    return to_dev(bf16_round(x), torch.bfloat16)


CASES = [
    # B, Sq, Sk, Hq, Hkv, d, dtype, q_offset, kv_offset, packed
    (2, 333, 517, 8, 2, 128, "bf16", 300, 0, False),
    (1, 1000, 777, 4, 4, 128, "bf16", 777, 0, True),
    (2, 97, 130, 2, 1, 64, "f32", 40, 0, False),
]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,d,dt,q_off,kv_off,packed", CASES)
def test_outputs_stay_inside_their_buffers(B, Sq, Sk, Hq, Hkv, d, dt, q_off, kv_off, packed):
    ra = lib()
    rng = np.random.default_rng(Sq * 7 + Sk)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32

    def inp(shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        g = Guarded(shape, tdt)
        g.t.copy_(to_dev(bf16_round(x) if dt == "bf16" else x, tdt))
        return g

    q, k, v, do = inp((B, Sq, Hq, d)), inp((B, Sk, Hkv, d)), inp((B, Sk, Hkv, d)), inp((B, Sq, Hq, d))
    inputs = [q, k, v, do]
    snap = [x.buf.clone() for x in inputs]
    seg = None
    outs = []
    scale = 1.0 / np.sqrt(d)
    S = max(q_off + Sq, kv_off + Sk)
    if packed:
        pos = np.concatenate([np.arange(n) for n in (150, 400, 333, 2000)])[:S].astype(np.int32)
        pos_g = Guarded((B, S), torch.int32)
        pos_g.t.copy_(torch.from_numpy(np.tile(pos, (B, 1))).to(device()))
        seg_g = Guarded((B, S), torch.int32)
        ra.segment_mask_from_pos(pos_g.t, seg_g.t)
        outs.append(("seg", seg_g))
        inputs.append(pos_g)
        snap.append(pos_g.buf.clone())
        seg = seg_g.t
    kw = dict(q_offset=q_off, kv_offset=kv_off, causal=True, scale=scale, seg_ids=seg)
    o_s, l_s = Guarded((B, Sq, Hq, d), torch.float32), Guarded((B, Hq, Sq), torch.float32)
    ra.ring_attn_fwd_step(q.t, k.t, v.t, o_s.t, l_s.t, **kw)
    outs += [("o_step", o_s), ("lse_step", l_s)]
    # fused step + merge into a running result, writing the output dtype
    o_a, l_a = Guarded((B, Sq, Hq, d), torch.float32), Guarded((B, Hq, Sq), torch.float32)
    o_a.t.copy_(o_s.t)
    l_a.t.copy_(l_s.t)
    o_out = Guarded((B, Sq, Hq, d), tdt)
    ra.ring_attn_fwd_step_merge(q.t, k.t, v.t, o_a.t, l_a.t, o_out=o_out.t, **kw)
    outs += [("o_acc", o_a), ("lse_acc", l_a), ("o_out", o_out)]
    # the merge entry point on its own
    o_m, l_m = Guarded((B, Sq, Hq, d), torch.float32), Guarded((B, Hq, Sq), torch.float32)
    o_m.t.copy_(o_s.t)
    l_m.t.copy_(l_s.t)
    o_out2 = Guarded((B, Sq, Hq, d), tdt)
    ra.lse_merge(o_m.t, l_m.t, o_s.t, l_s.t, o_out=o_out2.t)
    outs += [("merge_o", o_m), ("merge_lse", l_m), ("merge_out", o_out2)]
    # backward: delta, then one step into zeroed accumulators
    delta = Guarded((B, Hq, Sq), torch.float32)
    ra.ring_attn_bwd_preprocess(o_out.t, do.t, delta.t)
    dq, dk, dv = (Guarded((B, Sq, Hq, d), torch.float32), Guarded((B, Sk, Hkv, d), torch.float32),
                  Guarded((B, Sk, Hkv, d), torch.float32))
    for g in (dq, dk, dv):
        g.t.zero_()
    ra.ring_attn_bwd_step(q.t, k.t, v.t, do.t, l_a.t, delta.t, dq.t, dk.t, dv.t, **kw)
    outs += [("delta", delta), ("dq", dq), ("dk", dk), ("dv", dv)]
    # the receive copy
    dst = Guarded((B, Sk, Hkv, d), tdt)
    ra.ring_recv_copy(dst.t, k.t)
    outs.append(("recv", dst))
    torch.cuda.synchronize()
    bad = [name for name, g in outs if not g.guards_intact()]
    assert not bad, f"guard bytes overwritten around {bad}"
    for x, s0 in zip(inputs, snap):
        assert torch.equal(x.buf.view(x.ibits), s0.view(x.ibits)), "an input buffer was written"
    assert torch.equal(dst.t, k.t)
    for name, g in outs:
        if name in ("seg", "lse_step", "lse_acc", "merge_lse"):
            continue  # -inf is a legal LSE for rows that see no key in this step
        assert bool(torch.isfinite(g.t.float()).all()), name
    # and the values are right: the step's partial against the oracle
    seg_ref = None if seg is None else seg.cpu().numpy()
    o_ref, l_ref = oracle.attention_full(to_np(q.t), to_np(k.t), to_np(v.t), q_off + np.arange(Sq),
                                         kv_off + np.arange(Sk), scale, True,
                                         None if seg_ref is None else seg_ref[:, q_off:q_off + Sq],
                                         None if seg_ref is None else seg_ref[:, kv_off:kv_off + Sk])
    tol = 1e-4 if dt == "f32" else 2e-2
    assert max_abs(to_np(o_s.t), o_ref) <= tol
    lse_close(to_np(l_s.t), l_ref, 1e-4 if dt == "f32" else 1e-3)


def _nan_inputs(rng, Sq, Sk, Hq, Hkv, d):
    q = bf16_round(rng.standard_normal((1, Sq, Hq, d), dtype=np.float32))
    k = bf16_round(rng.standard_normal((1, Sk, Hkv, d), dtype=np.float32))
    v = bf16_round(rng.standard_normal((1, Sk, Hkv, d), dtype=np.float32))
    do = bf16_round(rng.standard_normal((1, Sq, Hq, d), dtype=np.float32))
    return q, k, v, do


def _fwd(ra, q, k, v):
    Sq, Hq, d = q.shape[1], q.shape[2], q.shape[3]
    o = torch.empty((1, Sq, Hq, d), dtype=torch.float32, device=device())
    lse = torch.empty((1, Hq, Sq), dtype=torch.float32, device=device())
    ra.ring_attn_fwd_step(_bf(q), _bf(k), _bf(v), o, lse, q_offset=0, kv_offset=0, causal=True,
                          scale=1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


SQ = SK = 640
HQ, HKV, D = 8, 2, 128


def test_nan_in_k_reaches_exactly_the_rows_that_see_it():
    ra = lib()
    rng = np.random.default_rng(41)
    q, k, v, _ = _nan_inputs(rng, SQ, SK, HQ, HKV, D)
    o0, l0 = _fwd(ra, q, k, v)
    j, g = 300, 1
    k2 = k.copy()
    k2[0, j, g, 5] = np.nan
    o1, l1 = _fwd(ra, q, k2, v)
    grp = [h for h in range(HQ) if h // (HQ // HKV) == g]
    other = [h for h in range(HQ) if h not in grp]
    # rows i >= j of the group's heads see key j: their LSE and O are NaN
    assert np.all(np.isnan(l1[0][np.ix_(grp, range(j, SQ))]))
    assert np.all(np.isnan(o1[0, j:, grp]))
    # rows before j never see it (masked before the exponent): bit-identical
    assert np.array_equal(l1[0][np.ix_(grp, range(j))], l0[0][np.ix_(grp, range(j))])
    assert np.array_equal(o1[0, :j][:, grp], o0[0, :j][:, grp])
    # other KV groups are untouched
    assert np.array_equal(l1[0, other], l0[0, other]) and np.array_equal(o1[0][:, other], o0[0][:, other])


def test_inf_in_q_and_nan_in_v():
    ra = lib()
    rng = np.random.default_rng(42)
    q, k, v, _ = _nan_inputs(rng, SQ, SK, HQ, HKV, D)
    o0, l0 = _fwd(ra, q, k, v)
    i, h = 500, 6
    q2 = q.copy()
    q2[0, i, h, 3] = np.inf
    o1, l1 = _fwd(ra, q2, k, v)
    assert not np.isfinite(l1[0, h, i]) and not np.all(np.isfinite(o1[0, i, h]))
    mask = np.ones_like(l0, dtype=bool)
    mask[0, h, i] = False
    assert np.array_equal(l1[mask], l0[mask])
    omask = np.ones(o0.shape[:3], dtype=bool)
    omask[0, i, h] = False
    assert np.array_equal(o1[omask], o0[omask])
    # NaN in V row j: the output of every row that sees key j is NaN, the LSE is not
    # affected at all (V does not enter it); rows of workgroups whose key range ends
    # before j's tile, and other KV groups, are bit-identical
    j, g = 400, 0
    v2 = v.copy()
    v2[0, j, g, 77] = np.nan
    o2, l2 = _fwd(ra, q, k, v2)
    grp = [x for x in range(HQ) if x // (HQ // HKV) == g]
    other = [x for x in range(HQ) if x not in grp]
    assert np.array_equal(l2, l0)
    assert np.all(np.isnan(o2[0, j:][:, grp, 77]))
    assert np.array_equal(o2[0, :j - 256][:, grp], o0[0, :j - 256][:, grp])
    assert np.array_equal(o2[0][:, other], o0[0][:, other])


def test_nan_in_do_backward_and_merge():
    ra = lib()
    rng = np.random.default_rng(43)
    q, k, v, do = _nan_inputs(rng, SQ, SK, HQ, HKV, D)
    o, lse = _fwd(ra, q, k, v)
    ob = _bf(o)
    lse_d = torch.from_numpy(lse).to(device())

    def bwd(do_np):
        delta = torch.empty((1, HQ, SQ), dtype=torch.float32, device=device())
        ra.ring_attn_bwd_preprocess(ob, _bf(do_np), delta)
        dq = torch.zeros((1, SQ, HQ, D), dtype=torch.float32, device=device())
        dk = torch.zeros((1, SK, HKV, D), dtype=torch.float32, device=device())
        dv = torch.zeros_like(dk)
        ra.ring_attn_bwd_step(_bf(q), _bf(k), _bf(v), _bf(do_np), lse_d, delta, dq, dk, dv, q_offset=0,
                              kv_offset=0, causal=True, scale=1.0 / np.sqrt(D))
        torch.cuda.synchronize()
        return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()

    dq0, dk0, dv0 = bwd(do)
    i, h = 450, 5
    g = h // (HQ // HKV)
    do2 = do.copy()
    do2[0, i, h, 9] = np.nan
    dq1, dk1, dv1 = bwd(do2)
    assert np.all(np.isnan(dq1[0, i, h]))
    rows = np.ones(SQ, dtype=bool)
    rows[i] = False
    assert np.array_equal(dq1[0, rows], dq0[0, rows])          # every other row of every head
    assert np.array_equal(dq1[0, :, [x for x in range(HQ) if x != h]], dq0[0, :, [x for x in range(HQ) if x != h]])
    assert np.all(np.isnan(dv1[0, :i + 1, g, 9]))               # keys that row i sees
    assert np.all(np.isnan(dk1[0, :i + 1, g]).any(axis=-1))
    og = [x for x in range(HKV) if x != g]
    assert np.array_equal(dk1[0][:, og], dk0[0][:, og]) and np.array_equal(dv1[0][:, og], dv0[0][:, og])

    # merge: a NaN log-sum-exp is never taken for the identity (-inf)
    o_acc = torch.zeros((1, 4, 1, 8), dtype=torch.float32, device=device())
    l_acc = torch.tensor([[[-np.inf, 1.0, np.nan, -np.inf]]], dtype=torch.float32, device=device())
    o_s = torch.ones((1, 4, 1, 8), dtype=torch.float32, device=device())
    l_s = torch.tensor([[[np.nan, np.nan, 2.0, -np.inf]]], dtype=torch.float32, device=device())
    ra.lse_merge(o_acc, l_acc, o_s, l_s)
    torch.cuda.synchronize()
    la, oa = l_acc.cpu().numpy()[0, 0], o_acc.cpu().numpy()[0, :, 0]
    assert np.all(np.isnan(la[:3])) and np.all(np.isnan(oa[:3]))
    assert la[3] == -np.inf and np.all(oa[3] == 0)              # both -inf: left unchanged


def test_merge_order_does_not_matter():
    """The 8K Llama-3-8B-shaped share (rank 3 of 4): its four ring-step partials merged
    in all 24 orders agree with one another within fp32 rounding and with the oracle."""
    ra = lib()
    cfg = LLAMA3_8K_FWD
    wl = make_workload(cfg, q_chunks=[cfg.rank])
    C = cfg.C
    q = _bf(wl.q_local)
    parts = []
    for c in range(cfg.CP):
        o_s = torch.empty((1, C, cfg.Hq, cfg.d), dtype=torch.float32, device=device())
        l_s = torch.empty((1, cfg.Hq, C), dtype=torch.float32, device=device())
        ra.ring_attn_fwd_step(q, _bf(wl.k_chunks[c]), _bf(wl.v_chunks[c]), o_s, l_s, q_offset=cfg.rank * C,
                              kv_offset=c * C, causal=True, scale=cfg.scale)
        parts.append((o_s, l_s))
    results = []
    for order in itertools.permutations(range(cfg.CP)):
        o_acc = torch.zeros_like(parts[0][0])
        l_acc = torch.full_like(parts[0][1], -np.inf)
        for c in order:
            ra.lse_merge(o_acc, l_acc, parts[c][0], parts[c][1])
        results.append((order, o_acc, l_acc))
    torch.cuda.synchronize()
    o0, l0 = results[0][1], results[0][2]
    worst_o = max(float((o - o0).abs().max()) for _, o, _ in results)
    worst_l = max(float((lse - l0).abs().max()) for _, _, lse in results)
    o_ref, l_ref = oracle.ring_forward(wl.q_local, wl.k_chunks, wl.v_chunks, cfg.rank, cfg.CP, cfg.scale, True)
    err_ref = max_abs(to_np(o0), o_ref)
    report("merge_orders", orders=len(results), o_spread=worst_o, lse_spread=worst_l, o_vs_oracle=err_ref)
    assert worst_o <= 1e-6 and worst_l <= 1e-5
    assert err_ref <= 2e-2
    lse_close(to_np(l0), l_ref, 1e-3)
