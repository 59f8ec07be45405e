"""The allocation-free backward step against the allocating one: bit-identical
dQ/dK/dV on two calls in a row (the second smaller), including steps whose dK/dV key
blocks are split (diagonal chunk, packed rows) and so use the static scratch."""

import math

import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_round
from tests.gpu_util import device, lib, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Sq, Sk, Hq, Hkv, d, packed):
    rng = np.random.default_rng(seed)
    q, k, v, do = (bf16_round(rng.standard_normal(s, dtype=np.float32))
                   for s in ((B, Sq, Hq, d), (B, Sk, Hkv, d), (B, Sk, Hkv, d), (B, Sq, Hq, d)))
    lse = (rng.standard_normal((B, Hq, Sq)) + 6.0).astype(np.float32)
    delta = (rng.standard_normal((B, Hq, Sq)) * 0.1).astype(np.float32)
    seg = None
    if packed:
        pos = np.concatenate([np.arange(n) for n in rng.integers(150, 700, size=64)])[: 4 * max(Sq, Sk)]
        seg = oracle.segment_ids(np.tile(pos, (B, 1)).astype(np.int32))
    acc = [rng.standard_normal(s).astype(np.float32) for s in ((B, Sq, Hq, d), (B, Sk, Hkv, d), (B, Sk, Hkv, d))]
    return q, k, v, do, lse, delta, seg, acc


# (B, Sq, Sk, Hq, Hkv, q_offset, kv_offset, causal, packed): the first call splits its
# key blocks (diagonal chunk), the second is smaller and packed.
CALLS = [(1, 1000, 1100, 32, 8, 1100, 1100, True, False),
         (1, 300, 260, 16, 4, 400, 300, True, True)]


def test_noalloc_matches_allocating_step_twice():
    ra = lib()
    bf = torch.bfloat16
    for n, (B, Sq, Sk, Hq, Hkv, q_off, kv_off, causal, packed) in enumerate(CALLS):
        q, k, v, do, lse, delta, seg, acc = _inputs(7 + n, B, Sq, Sk, Hq, Hkv, 128, packed)
        args = [to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(do, bf), to_dev(lse, torch.float32),
                to_dev(delta, torch.float32)]
        kw = dict(q_offset=q_off, kv_offset=kv_off, causal=causal, scale=1 / math.sqrt(128),
                  seg_ids=None if seg is None else to_dev(seg, torch.int32))
        ref = [to_dev(a, torch.float32) for a in acc]
        got = [to_dev(a, torch.float32) for a in acc]
        ra.ring_attn_bwd_step(*args, *ref, **kw)
        ra.ring_attn_bwd_step_noalloc(*args, *got, **kw)
        torch.cuda.synchronize()
        print(f"[noalloc] call {n}: shape {(B, Sq, Sk, Hq, Hkv)} packed={packed}", flush=True)
        for name, r, g, a0 in zip(("dq", "dk", "dv"), ref, got, acc):
            assert torch.equal(r, g), name
            assert not torch.equal(g, to_dev(a0, torch.float32)), name  # the step did add something
