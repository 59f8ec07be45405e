"""GPU parity of the whole ring share on the five workloads (and the 64K forward +
backward measurement workload) against the fp64 oracle, at full size.

Tolerances: fp32 O and LSE <= 1e-4 max-abs; bf16 O <= 2e-2 and LSE <= 1e-3 max-abs
(N(0,1) inputs); gradients <= 3e-2 relative to the reference's max-abs.  Because
|O| shrinks like sqrt(e/n) on long contexts, O is also held to 2e-2 relative to
its max so that the absolute bound cannot hide a gross error.
"""

import numpy as np
import pytest
import torch

import oracle
from synthetic import CONFIGS, LLAMA3_8K_BWD, PACKED16K_FWD, make_workload
from tests.gpu_util import device, lib, lse_close, max_abs, rel_to_max, report, to_dev, to_np

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _device_inputs(wl):
    cfg = wl.cfg
    dt = TD[cfg.dtype]
    q = to_dev(wl.q_local, dt)
    ks = [to_dev(k, dt) for k in wl.k_chunks]
    vs = [to_dev(v, dt) for v in wl.v_chunks]
    return q, ks, vs


def _seg(wl):
    if not wl.cfg.packed:
        return None, None
    ra = lib()
    pos = to_dev(wl.position_ids, torch.int32)
    seg = torch.empty_like(pos)
    ra.segment_mask_from_pos(pos, seg)
    return seg, oracle.segment_ids(wl.position_ids)


def _tols(cfg):
    return (1e-4, 1e-4) if cfg.dtype == "f32" else (2e-2, 1e-3)


@pytest.mark.parametrize("name", ["tiny_ring_fp32_S1k_cp4_r3", "llama3_8b_S8k_cp4_r3_fwd", "packed16k_cp4_r2_fwd"])
def test_forward_config_full(name):
    ra = lib()
    cfg = CONFIGS[name]
    wl = make_workload(cfg, q_chunks=[cfg.rank])
    q, ks, vs = _device_inputs(wl)
    seg_d, seg_ref = _seg(wl)
    if seg_d is not None:
        np.testing.assert_array_equal(seg_d.cpu().numpy(), seg_ref)
    partials_gpu = []

    o, lse = ra.ring_forward(q, ks, vs, cfg.rank, cfg.CP, causal=cfg.causal, seg_ids=seg_d)
    torch.cuda.synchronize()
    partials = []
    o_ref, l_ref = oracle.ring_forward(wl.q_local, wl.k_chunks, wl.v_chunks, cfg.rank, cfg.CP, cfg.scale,
                                       cfg.causal, seg_ref, partials=partials)
    tol_o, tol_l = _tols(cfg)
    on = to_np(o)
    err_o, rel_o = max_abs(on, o_ref), rel_to_max(on, o_ref)
    err_l = lse_close(to_np(lse), l_ref, tol_l)
    report(cfg.name, o_maxabs=err_o, o_rel=rel_o, lse_maxabs=err_l, o_ref_max=float(np.abs(o_ref).max()))
    assert err_o <= tol_o and rel_o <= 2e-2

    # every ring step's partial on its own, including fully masked chunks (-inf / 0 exactly)
    C = cfg.C
    for step, (c, o_c, l_c) in enumerate(partials):
        o_s = torch.empty((cfg.B, C, cfg.Hq, cfg.d), dtype=torch.float32, device=device())
        l_s = torch.empty((cfg.B, cfg.Hq, C), dtype=torch.float32, device=device())
        ra.ring_attn_fwd_step(q, ks[c], vs[c], o_s, l_s, q_offset=cfg.rank * C, kv_offset=c * C,
                              causal=cfg.causal, scale=cfg.scale, seg_ids=seg_d)
        torch.cuda.synchronize()
        e = max_abs(to_np(o_s), o_c)
        el = lse_close(to_np(l_s), l_c, tol_l)
        partials_gpu.append((c, e, el))
        assert e <= tol_o, (step, c, e)
    report(cfg.name + "/steps", steps=str([(c, f"{e:.1e}", f"{el:.1e}") for c, e, el in partials_gpu]))


def test_packed_config_rank2_dead_steps_cost_nothing():
    """Packed 16K, rank 2: chunks 0 and 3 have no live pair; their steps return the merge
    identity and merging them leaves the running result bit-identical."""
    ra = lib()
    cfg = PACKED16K_FWD
    wl = make_workload(cfg, q_chunks=[cfg.rank])
    q, ks, vs = _device_inputs(wl)
    seg_d, _ = _seg(wl)
    C = cfg.C
    o_acc = torch.empty((1, C, cfg.Hq, cfg.d), dtype=torch.float32, device=device())
    l_acc = torch.empty((1, cfg.Hq, C), dtype=torch.float32, device=device())
    ra.ring_attn_fwd_step(q, ks[2], vs[2], o_acc, l_acc, q_offset=2 * C, kv_offset=2 * C, causal=True,
                          scale=cfg.scale, seg_ids=seg_d)
    snap = (o_acc.clone(), l_acc.clone())
    for c in (0, 3):
        o_s = torch.empty_like(o_acc)
        l_s = torch.empty_like(l_acc)
        ra.ring_attn_fwd_step(q, ks[c], vs[c], o_s, l_s, q_offset=2 * C, kv_offset=c * C, causal=True,
                              scale=cfg.scale, seg_ids=seg_d)
        torch.cuda.synchronize()
        assert torch.all(o_s == 0) and torch.all(torch.isneginf(l_s))
        ra.lse_merge(o_acc, l_acc, o_s, l_s)
    torch.cuda.synchronize()
    assert torch.equal(o_acc, snap[0]) and torch.equal(l_acc, snap[1])


def _grad_errors(dq, dks, dvs, dq_ref, dk_ref, dv_ref):
    e_dq = rel_to_max(to_np(dq), dq_ref)
    e_dk = rel_to_max(np.concatenate([to_np(x) for x in dks], 1), np.concatenate(dk_ref, 1))
    e_dv = rel_to_max(np.concatenate([to_np(x) for x in dvs], 1), np.concatenate(dv_ref, 1))
    return e_dq, e_dk, e_dv


def test_backward_config5_full():
    ra = lib()
    cfg = LLAMA3_8K_BWD
    wl = make_workload(cfg, q_chunks=[cfg.rank])
    q, ks, vs = _device_inputs(wl)
    do = to_dev(wl.do, torch.bfloat16)
    o, lse = ra.ring_forward(q, ks, vs, cfg.rank, cfg.CP, causal=True)
    dq, dks, dvs = ra.ring_backward(q, ks, vs, o, lse, do, cfg.rank, cfg.CP, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.ring_forward(wl.q_local, wl.k_chunks, wl.v_chunks, cfg.rank, cfg.CP, cfg.scale, True)
    dq_ref, dk_ref, dv_ref = oracle.ring_backward(wl.q_local, wl.k_chunks, wl.v_chunks, o_ref, l_ref, wl.do,
                                                  cfg.rank, cfg.CP, cfg.scale, True)
    e = _grad_errors(dq, dks, dvs, dq_ref, dk_ref, dv_ref)
    report(cfg.name, dq=e[0], dk=e[1], dv=e[2], o_maxabs=max_abs(to_np(o), o_ref))
    assert max(e) <= 3e-2, e


def test_backward_packed_config4_full():
    """Backward on the packed 16K share (its forward is config 4; dO drawn from the
    config's own seed stream)."""
    ra = lib()
    cfg = PACKED16K_FWD.with_(backward=True)
    wl = make_workload(cfg, q_chunks=[cfg.rank])
    q, ks, vs = _device_inputs(wl)
    seg_d, seg_ref = _seg(wl)
    do = to_dev(wl.do, torch.bfloat16)
    o, lse = ra.ring_forward(q, ks, vs, cfg.rank, cfg.CP, causal=True, seg_ids=seg_d)
    dq, dks, dvs = ra.ring_backward(q, ks, vs, o, lse, do, cfg.rank, cfg.CP, causal=True, seg_ids=seg_d)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.ring_forward(wl.q_local, wl.k_chunks, wl.v_chunks, cfg.rank, cfg.CP, cfg.scale, True,
                                       seg_ref)
    dq_ref, dk_ref, dv_ref = oracle.ring_backward(wl.q_local, wl.k_chunks, wl.v_chunks, o_ref, l_ref, wl.do,
                                                  cfg.rank, cfg.CP, cfg.scale, True, seg_ref)
    e = _grad_errors(dq, dks, dvs, dq_ref, dk_ref, dv_ref)
    report(cfg.name + "/bwd", dq=e[0], dk=e[1], dv=e[2])
    assert max(e) <= 3e-2, e
    for c in (0, 3):  # chunks with no live pair receive exactly zero gradient
        assert torch.all(dks[c] == 0) and torch.all(dvs[c] == 0)
