"""Parity of the load-balanced ("zigzag") ring on the GPU against the oracle.

The rank holds query/key/value halves r and 2*cp-1-r of the row; whatever the ring
order, its final O and LSE must equal plain masked attention of those query rows
over the whole row (the definition the oracle writes out), and its backward must
give that attention's gradients: dQ for its rows and its contribution to every
rank's dK/dV rows.  Tolerances as for the contiguous ring."""

import numpy as np
import pytest
import torch

import oracle
from synthetic import LLAMA3_8K_FWD, PACKED16K_FWD, TINY_RING, make_workload, zigzag_indices, zigzag_take
from tests.gpu_util import lib, lse_close, max_abs, rel_to_max, report, to_dev, to_np

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f32": torch.float32}

CASES = {
    "bf16_cp4_r0": LLAMA3_8K_FWD.with_(name="zz_bf16_cp4_r0", S=4096, rank=0, Hq=8, Hkv=2, backward=True, seed=11),
    "bf16_cp4_r3": LLAMA3_8K_FWD.with_(name="zz_bf16_cp4_r3", S=4096, rank=3, Hq=8, Hkv=2, backward=True, seed=12),
    "bf16_cp4_r2_nocausal": LLAMA3_8K_FWD.with_(name="zz_bf16_cp4_r2_nc", S=2048, rank=2, Hq=4, Hkv=1, causal=False,
                                             backward=True, seed=13),
    "packed_cp4_r1": PACKED16K_FWD.with_(name="zz_packed_cp4_r1", S=4096, rank=1, Hq=8, Hkv=2, min_len=256,
                                      max_len=1024, backward=True, seed=14),
    "f32_d64_cp2_r1": TINY_RING.with_(name="zz_f32_d64_cp2_r1", S=1024, CP=2, rank=1, Hq=2, Hkv=1, backward=True,
                                       seed=15),
}


def _setup(cfg):
    ra = lib()
    wl = make_workload(cfg)
    S, cp, r = cfg.S, cfg.CP, cfg.rank
    dt = TD[cfg.dtype]
    qf, kf, vf = wl.q_full(), wl.k_full(), wl.v_full()
    q_idx, k_idx = zigzag_indices(S, cp, r), np.arange(S)
    q = to_dev(zigzag_take(qf, S, cp, r), dt)
    ks = [to_dev(zigzag_take(kf, S, cp, c), dt) for c in range(cp)]
    vs = [to_dev(zigzag_take(vf, S, cp, c), dt) for c in range(cp)]
    seg_d = seg_ref = None
    if cfg.packed:
        pos = to_dev(wl.position_ids, torch.int32)
        seg_d = torch.empty_like(pos)
        ra.segment_mask_from_pos(pos, seg_d)
        seg_ref = oracle.segment_ids(wl.position_ids)
    return ra, wl, q, ks, vs, seg_d, seg_ref, q_idx, k_idx


@pytest.mark.parametrize("case", list(CASES))
def test_zigzag_forward_and_backward(case):
    cfg = CASES[case]
    ra, wl, q, ks, vs, seg_d, seg_ref, q_idx, k_idx = _setup(cfg)
    S, cp, r, h = cfg.S, cfg.CP, cfg.rank, cfg.S // (2 * cfg.CP)
    o, lse = ra.ring_forward_zigzag(q, ks, vs, r, cp, causal=cfg.causal, seg_ids=seg_d)
    do = to_dev(wl.do, TD[cfg.dtype])
    dq, dks, dvs = ra.ring_backward_zigzag(q, ks, vs, o, lse, do, r, cp, causal=cfg.causal, seg_ids=seg_d)
    torch.cuda.synchronize()

    qz = zigzag_take(wl.q_full(), S, cp, r)
    sq = None if seg_ref is None else seg_ref[:, q_idx]
    o_ref, l_ref = oracle.attention_full(qz, wl.k_full(), wl.v_full(), q_idx, k_idx, cfg.scale, cfg.causal,
                                         sq, seg_ref)
    tol_o, tol_l = (1e-4, 1e-4) if cfg.dtype == "f32" else (2e-2, 1e-3)
    on = to_np(o)
    err_o, rel_o = max_abs(on, o_ref), rel_to_max(on, o_ref)
    ln = to_np(lse)  # [2, Hq, h]: row block j = query half j
    err_l = max(lse_close(ln[j], l_ref[0][:, j * h:(j + 1) * h], tol_l) for j in range(2))
    assert err_o <= tol_o and rel_o <= 2e-2, (err_o, rel_o)

    delta_ref = oracle.bwd_delta(o_ref, wl.do)
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd_full(qz, wl.k_full(), wl.v_full(), wl.do, l_ref, delta_ref, q_idx,
                                                       k_idx, cfg.scale, cfg.causal, sq, seg_ref)
    e_dq = rel_to_max(to_np(dq), dq_ref)
    e_dk = rel_to_max(np.concatenate([to_np(x) for x in dks], 1),
                      np.concatenate([zigzag_take(dk_ref, S, cp, c) for c in range(cp)], 1))
    e_dv = rel_to_max(np.concatenate([to_np(x) for x in dvs], 1),
                      np.concatenate([zigzag_take(dv_ref, S, cp, c) for c in range(cp)], 1))
    report(cfg.name, o_maxabs=err_o, o_rel=rel_o, lse_maxabs=err_l, dq=e_dq, dk=e_dk, dv=e_dv)
    assert max(e_dq, e_dk, e_dv) <= (1e-4 if cfg.dtype == "f32" else 3e-2), (e_dq, e_dk, e_dv)
