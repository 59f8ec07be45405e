"""Synthetic input generators (CPU only): rounding, packed lengths, determinism."""

import numpy as np
import torch

from synthetic import (CONFIGS, CTX64K_FWD, LLAMA3_8K_BWD, LLAMA3_8K_FWD, METRIC_CONFIG, PACKED16K_FWD, TINY_RING,
                       bf16_round, draw_packed_lengths, make_workload)


def test_bf16_round_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.0039062, 3e-39, 0.0, -0.0, 65504.0],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_round(x), ref)


def test_packed_lengths_cover_row_exactly():
    for seed in range(20):
        rng = np.random.default_rng(seed)
        lengths = draw_packed_lengths(rng, 16384, 512, 4096)
        assert lengths.sum() == 16384
        assert np.all(lengths[:-1] >= 512) and np.all(lengths <= 4096)
        assert lengths[-1] >= 1


def test_packed_workload_position_ids_restart_per_sample():
    wl = make_workload(PACKED16K_FWD)
    pos = wl.position_ids[0]
    starts = np.concatenate([[0], np.cumsum(wl.lengths)[:-1]])
    assert np.all(pos[starts] == 0)
    assert int((pos == 0).sum()) == len(wl.lengths)
    assert wl.position_ids.dtype == np.int32


def test_workloads_are_deterministic_and_bf16_exact():
    a = make_workload(LLAMA3_8K_FWD)
    b = make_workload(LLAMA3_8K_FWD, q_chunks=[3])
    np.testing.assert_array_equal(a.q_local, b.q_local)
    np.testing.assert_array_equal(a.k_chunks[1], b.k_chunks[1])
    assert b.q_chunks[0] is None
    np.testing.assert_array_equal(bf16_round(a.v_chunks[0]), a.v_chunks[0])
    assert a.q_local.shape == (1, 2048, 32, 128) and a.k_chunks[0].shape == (1, 2048, 8, 128)


def test_config_shapes():
    t, x = TINY_RING, CTX64K_FWD
    assert (t.S, t.CP, t.rank, t.C, t.d, t.dtype) == (1024, 4, 3, 256, 64, "f32")
    assert (x.S, x.CP, x.rank, x.C) == (65536, 8, 7, 8192)
    assert LLAMA3_8K_BWD.backward and not LLAMA3_8K_FWD.backward
    assert PACKED16K_FWD.packed and len(CONFIGS) == 5 and all(CONFIGS[k].name == k for k in CONFIGS)
    assert METRIC_CONFIG.backward and METRIC_CONFIG.S == 65536
