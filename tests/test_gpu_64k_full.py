"""The 64K share at full size, element by element against the fp64 oracle: rank 7 of
CP=8 over S = 65536 (8192 local queries, 32 query heads, 8 KV heads, d = 128, causal,
bf16), forward and backward through the ring loops in the launch configuration the
benchmark times.  Its forward inputs are exactly the 64K forward workload's (same
seed and draws), so the forward comparison is that workload's parity at full size.

The oracle side is the plain definition over the whole row (``attention_full`` /
``attention_bwd_full`` with global indices 0..65535), run one query head at a time
on the host cores (``oracle.parallel``); its backward uses its own fp64 O and LSE.

Tolerances: O <= 2e-2 max-abs and <= 2e-2 relative to max|O|; LSE <= 1e-3 max-abs;
dQ, dK, dV <= 3e-2 relative to the reference's max-abs (per tensor, over all rows,
all 8 chunks)."""

import time

import numpy as np
import pytest
import torch

import oracle
from oracle import parallel as opar
from synthetic import METRIC_CONFIG, make_workload
from tests.gpu_util import lib, lse_close, max_abs, rel_to_max, report, to_dev, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CFG = METRIC_CONFIG


def _log(msg):
    print(f"[64k-full] {msg}", flush=True)


@pytest.fixture(scope="module")
def wl():
    return make_workload(CFG, q_chunks=[CFG.rank])


@pytest.fixture(scope="module")
def gpu(wl):
    """The HIP ring forward + backward of the share; results copied to the host."""
    ra = lib()
    q = to_dev(wl.q_local, torch.bfloat16)
    ks = [to_dev(k, torch.bfloat16) for k in wl.k_chunks]
    vs = [to_dev(v, torch.bfloat16) for v in wl.v_chunks]
    do = to_dev(wl.do, torch.bfloat16)
    o, lse = ra.ring_forward(q, ks, vs, CFG.rank, CFG.CP, causal=True)
    dq, dks, dvs = ra.ring_backward(q, ks, vs, o, lse, do, CFG.rank, CFG.CP, causal=True)
    torch.cuda.synchronize()
    out = {"o": to_np(o), "lse": to_np(lse), "dq": to_np(dq),
           "dk": np.concatenate([to_np(x) for x in dks], 1), "dv": np.concatenate([to_np(x) for x in dvs], 1)}
    del q, ks, vs, do, o, lse, dq, dks, dvs
    torch.cuda.empty_cache()
    _log("GPU forward + backward done")
    return out


@pytest.fixture(scope="module")
def ref_fwd(wl):
    """Oracle O, LSE of every head over the whole row (the direct definition)."""
    t0 = time.perf_counter()
    q_idx = CFG.rank * CFG.C + np.arange(CFG.C)
    o, lse = opar.attention_full_heads(wl.q_local, wl.k_full(), wl.v_full(), q_idx, np.arange(CFG.S), CFG.scale,
                                       True)
    _log(f"oracle forward, 32 heads: {time.perf_counter() - t0:.1f} s on {opar.host_cores()} threads")
    return o, lse


def test_64k_forward_full_size(gpu, ref_fwd):
    o_ref, l_ref = ref_fwd
    err_o, rel_o = max_abs(gpu["o"], o_ref), rel_to_max(gpu["o"], o_ref)
    rms_rel = float(np.sqrt(np.mean((gpu["o"] - o_ref) ** 2) / np.mean(o_ref ** 2)))
    err_l = lse_close(gpu["lse"], l_ref, 1e-3)
    report(CFG.name + "/fwd", o_maxabs=err_o, o_rel=rel_o, o_rms_rel=rms_rel, lse_maxabs=err_l,
           o_ref_max=float(np.abs(o_ref).max()))
    assert err_o <= 2e-2 and rel_o <= 2e-2


@pytest.mark.parametrize("kv_heads", [(0, 1, 2, 3), (4, 5, 6, 7)])
def test_64k_backward_full_size(gpu, ref_fwd, wl, kv_heads):
    """dQ of every row of the group's 16 query heads; dK, dV of the KV heads over all
    65536 keys (all 8 chunks)."""
    o_ref, l_ref = ref_fwd
    group = CFG.Hq // CFG.Hkv
    heads = [g * group + j for g in kv_heads for j in range(group)]
    delta = np.zeros_like(l_ref)
    delta[:, heads] = oracle.bwd_delta(o_ref[:, :, heads], wl.do[:, :, heads])
    t0 = time.perf_counter()
    q_idx = CFG.rank * CFG.C + np.arange(CFG.C)
    dq_ref, dk_ref, dv_ref = opar.attention_bwd_full_heads(wl.q_local, wl.k_full(), wl.v_full(), wl.do, l_ref, delta,
                                                           q_idx, np.arange(CFG.S), CFG.scale, True,
                                                           kv_heads=kv_heads)
    _log(f"oracle backward, KV heads {kv_heads}: {time.perf_counter() - t0:.1f} s")
    e_dq = rel_to_max(gpu["dq"][:, :, heads], dq_ref)
    e_dk = rel_to_max(gpu["dk"][:, :, list(kv_heads)], dk_ref)
    e_dv = rel_to_max(gpu["dv"][:, :, list(kv_heads)], dv_ref)
    report(CFG.name + f"/bwd{kv_heads}", dq=e_dq, dk=e_dk, dv=e_dv)
    assert max(e_dq, e_dk, e_dv) <= 3e-2, (e_dq, e_dk, e_dv)
