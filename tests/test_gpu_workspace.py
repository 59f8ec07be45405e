"""Device workspace of one rank's forward + backward, and repeatability of the backward.

The pages' point is that the share never holds an S x S score tensor (archcrux,
"sequence-parallel long-context attention OOM"): what the ring loops allocate
beyond their inputs and outputs must grow like C * Hq * d.  Here it is the fp32
running O of the forward and the backward's delta rows, and nothing else: the
measured peak stays within those bytes plus the allocator's rounding, and doubling
the chunk doubles it."""

import numpy as np
import pytest
import torch

from synthetic import LLAMA3_8K_BWD, make_workload
from tests.gpu_util import device, lib, to_dev

pytestmark = pytest.mark.gpu


def _workspace_bytes(S):
    ra = lib()
    cfg = LLAMA3_8K_BWD.with_(name=f"ws_S{S}", S=S, Hq=8, Hkv=2, seed=41)
    wl = make_workload(cfg)
    dev = device()
    q = to_dev(wl.q_local, torch.bfloat16)
    ks = [to_dev(k, torch.bfloat16) for k in wl.k_chunks]
    vs = [to_dev(v, torch.bfloat16) for v in wl.v_chunks]
    do = to_dev(wl.do, torch.bfloat16)
    C = cfg.C
    o = torch.empty_like(q)
    lse = torch.empty((1, cfg.Hq, C), dtype=torch.float32, device=dev)
    dq = torch.zeros((1, C, cfg.Hq, cfg.d), dtype=torch.float32, device=dev)
    dks = [torch.zeros(k.shape, dtype=torch.float32, device=dev) for k in ks]
    dvs = [torch.zeros(v.shape, dtype=torch.float32, device=dev) for v in vs]
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ra.ring_forward(q, ks, vs, cfg.rank, cfg.CP, causal=True, out=o, lse=lse)
    ra.ring_backward(q, ks, vs, o, lse, do, cfg.rank, cfg.CP, causal=True, dq=dq, dk_chunks=dks, dv_chunks=dvs)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    expected = C * cfg.Hq * cfg.d * 4 + cfg.Hq * C * 4  # running O (fp32) + delta rows
    return peak, expected, cfg


def test_workspace_is_linear_in_the_chunk():
    p1, e1, c1 = _workspace_bytes(4096)
    p2, e2, c2 = _workspace_bytes(8192)
    for p, e, c in ((p1, e1, c1), (p2, e2, c2)):
        assert 0 < p <= e + (1 << 20), (c.name, p, e)
        assert p <= c.C * c.S * c.Hq * 4 / 16  # a small fraction of one fp32 score tensor of the share
    assert 1.8 <= p2 / p1 <= 2.2


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv,kv_off", [(320, 448, 8, 2, 0), (320, 1000, 128, 64, 0),
                                                 (1000, 1024, 128, 64, 0), (600, 448, 8, 2, 300)])
def test_bwd_step_is_bitwise_repeatable(Sq, Sk, Hq, Hkv, kv_off):
    """Both dK/dV kernels (32 keys per wave; 64 keys per wave on the wider grids) and
    both dQ kernels (32 queries per wave; 64 on the last grid) give the same bits on
    every call -- also when the key blocks of the diagonal chunk are split over two
    workgroups (last case), whose partial sums arrive in any order."""
    ra = lib()
    rng = np.random.default_rng(3)
    B, d = 1, 128

    def bf(*shape):
        return to_dev(rng.standard_normal(shape, dtype=np.float32), torch.bfloat16)

    q, k, v, do = bf(B, Sq, Hq, d), bf(B, Sk, Hkv, d), bf(B, Sk, Hkv, d), bf(B, Sq, Hq, d)
    lse = to_dev(rng.uniform(4.0, 6.0, (B, Hq, Sq)).astype(np.float32), torch.float32)
    delta = to_dev(0.1 * rng.standard_normal((B, Hq, Sq), dtype=np.float32), torch.float32)
    outs = []
    for _ in range(3):
        dq = torch.zeros((B, Sq, Hq, d), dtype=torch.float32, device=device())
        dk = torch.zeros((B, Sk, Hkv, d), dtype=torch.float32, device=device())
        dv = torch.zeros_like(dk)
        ra.ring_attn_bwd_step(q, k, v, do, lse, delta, dq, dk, dv, q_offset=448, kv_offset=kv_off, causal=True,
                              scale=0.088)
        outs.append([t.cpu().numpy() for t in (dq, dk, dv)])
    for rep in outs[1:]:
        for a, b in zip(rep, outs[0]):
            assert np.array_equal(a, b)
