"""Parity of the two other shares of the same attention on the GPU against the oracle:
the head-sharded (Ulysses) share — all of the row for a subset of heads — and the
gathered-KV (llama3-style) share — the rank's contiguous query chunk against the
gathered row.  Both must equal plain masked attention (the definition the oracle
writes out) and its gradients; tolerances as for the ring."""

import numpy as np
import pytest
import torch

import oracle
from synthetic import LLAMA3_8K_FWD, PACKED16K_FWD, make_workload
from tests.gpu_util import lib, lse_close, max_abs, rel_to_max, report, to_dev, to_np

pytestmark = pytest.mark.gpu


def _seg(ra, wl):
    if not wl.cfg.packed:
        return None, None
    pos = to_dev(wl.position_ids, torch.int32)
    seg = torch.empty_like(pos)
    ra.segment_mask_from_pos(pos, seg)
    return seg, oracle.segment_ids(wl.position_ids)


ULYSSES = {
    "causal": LLAMA3_8K_FWD.with_(name="ulysses_S2k_h4", S=2048, CP=1, rank=0, Hq=4, Hkv=1, backward=True, seed=21),
    "packed": PACKED16K_FWD.with_(name="ulysses_packed_S4k_h4", S=4096, CP=1, rank=0, Hq=4, Hkv=1, min_len=256,
                               max_len=1024, backward=True, seed=22),
}


@pytest.mark.parametrize("case", list(ULYSSES))
def test_ulysses_share(case):
    ra = lib()
    cfg = ULYSSES[case]
    wl = make_workload(cfg)
    q, k, v = (to_dev(x, torch.bfloat16) for x in (wl.q_full(), wl.k_full(), wl.v_full()))
    do = to_dev(wl.do, torch.bfloat16)
    seg_d, seg_ref = _seg(ra, wl)
    o, lse = ra.ulysses_forward(q, k, v, causal=True, seg_ids=seg_d)
    dq, dk, dv = ra.ulysses_backward(q, k, v, o, lse, do, causal=True, seg_ids=seg_d)
    torch.cuda.synchronize()
    idx = np.arange(cfg.S)
    o_ref, l_ref = oracle.attention_full(wl.q_full(), wl.k_full(), wl.v_full(), idx, idx, cfg.scale, True,
                                         seg_ref, seg_ref)
    err_o, rel_o = max_abs(to_np(o), o_ref), rel_to_max(to_np(o), o_ref)
    err_l = lse_close(to_np(lse), l_ref, 1e-3)
    delta = oracle.bwd_delta(o_ref, wl.do)
    g_ref = oracle.attention_bwd_full(wl.q_full(), wl.k_full(), wl.v_full(), wl.do, l_ref, delta, idx, idx,
                                      cfg.scale, True, seg_ref, seg_ref)
    e = [rel_to_max(to_np(x), r) for x, r in zip((dq, dk, dv), g_ref)]
    report(cfg.name, o_maxabs=err_o, o_rel=rel_o, lse_maxabs=err_l, dq=e[0], dk=e[1], dv=e[2])
    assert err_o <= 2e-2 and rel_o <= 2e-2 and max(e) <= 3e-2, (err_o, rel_o, e)


GATHERED = {
    "causal_r3": LLAMA3_8K_FWD.with_(name="gathered_S4k_cp4_r3", S=4096, Hq=8, Hkv=2, backward=True, seed=31),
    "packed_r2": PACKED16K_FWD.with_(name="gathered_packed_S4k_cp4_r2", S=4096, Hq=8, Hkv=2, min_len=256,
                                  max_len=1024, backward=True, seed=32),
}


@pytest.mark.parametrize("case", list(GATHERED))
def test_gathered_share(case):
    ra = lib()
    cfg = GATHERED[case]
    wl = make_workload(cfg, q_chunks=[cfg.rank])
    q = to_dev(wl.q_local, torch.bfloat16)
    ks = [to_dev(x, torch.bfloat16) for x in wl.k_chunks]
    vs = [to_dev(x, torch.bfloat16) for x in wl.v_chunks]
    do = to_dev(wl.do, torch.bfloat16)
    seg_d, seg_ref = _seg(ra, wl)
    k_all, v_all = ra.gather_kv(ks, vs)
    o, lse = ra.gathered_forward(q, k_all, v_all, cfg.rank, causal=True, seg_ids=seg_d)
    dq, dk_all, dv_all = ra.gathered_backward(q, k_all, v_all, o, lse, do, cfg.rank, causal=True, seg_ids=seg_d)
    dks = [torch.empty(k.shape, dtype=torch.float32, device=q.device) for k in ks]
    dvs = [torch.empty(v.shape, dtype=torch.float32, device=q.device) for v in vs]
    ra.scatter_dkv(dk_all, dv_all, dks, dvs)
    torch.cuda.synchronize()
    assert torch.equal(k_all.cpu(), torch.cat([x.cpu() for x in ks], 1))
    o_ref, l_ref = oracle.ring_forward(wl.q_local, wl.k_chunks, wl.v_chunks, cfg.rank, cfg.CP, cfg.scale, True,
                                       seg_ref)
    err_o, rel_o = max_abs(to_np(o), o_ref), rel_to_max(to_np(o), o_ref)
    err_l = lse_close(to_np(lse), l_ref, 1e-3)
    dq_ref, dk_ref, dv_ref = oracle.ring_backward(wl.q_local, wl.k_chunks, wl.v_chunks, o_ref, l_ref, wl.do,
                                                  cfg.rank, cfg.CP, cfg.scale, True, seg_ref)
    e_dq = rel_to_max(to_np(dq), dq_ref)
    e_dk = rel_to_max(np.concatenate([to_np(x) for x in dks], 1), np.concatenate(dk_ref, 1))
    e_dv = rel_to_max(np.concatenate([to_np(x) for x in dvs], 1), np.concatenate(dv_ref, 1))
    report(cfg.name, o_maxabs=err_o, o_rel=rel_o, lse_maxabs=err_l, dq=e_dq, dk=e_dk, dv=e_dv)
    assert err_o <= 2e-2 and rel_o <= 2e-2 and max(e_dq, e_dk, e_dv) <= 3e-2
