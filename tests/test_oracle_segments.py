"""Pins of the oracle's segment ids (CPU only): the packed-row generator's own sample
boundaries are an independent ground truth for the sample index of every token."""

import numpy as np
import pytest

import oracle
from synthetic import PACKED16K_FWD, make_workload
from tests._brute import brute_segment_ids


def test_segment_ids_equal_generator_sample_index_full_size():
    wl = make_workload(PACKED16K_FWD)
    seg = oracle.segment_ids(wl.position_ids)
    np.testing.assert_array_equal(seg, wl.sample_index)
    assert seg.dtype == np.int32


@pytest.mark.parametrize("seed", range(6))
def test_segment_ids_brute_force_random_rows(seed):
    rng = np.random.default_rng(seed)
    B, S = 3, 300
    rows = []
    for _ in range(B):
        row = []
        if seed % 2:                       # a row that starts mid-sample
            row.extend(range(5, 5 + int(rng.integers(1, 20))))
        while len(row) < S:
            row.extend(range(int(rng.integers(1, 40))))
        rows.append(row[:S])
    pos = np.asarray(rows, dtype=np.int32)
    seg = oracle.segment_ids(pos)
    for b in range(B):
        assert seg[b].tolist() == brute_segment_ids(pos[b].tolist())


def test_chunk_that_starts_mid_sample_keeps_sample_id():
    pos = np.array([[0, 1, 2, 3, 0, 1, 2, 3, 4, 5, 0, 1]], dtype=np.int32)
    seg = oracle.segment_ids(pos)
    # chunks of 3: chunk 2 = tokens 6..8 start inside sample 1
    assert seg[0, 6:9].tolist() == [1, 1, 1]
    assert seg[0].tolist() == [0, 0, 0, 0, 1, 1, 1, 1, 1, 1, 2, 2]


def test_packed_rank2_structure():
    """Samples are at most 4096 = one chunk long, so for rank 2 of the 16K row chunk 0
    never shares a sample with a local query, and chunk 3 lies in the future: two of the
    four ring steps have no live pair."""
    cfg = PACKED16K_FWD
    wl = make_workload(cfg)
    seg = oracle.segment_ids(wl.position_ids)
    C, r = cfg.C, cfg.rank
    q_idx = r * C + np.arange(C)
    counts = {}
    for c in range(cfg.CP):
        counts[c] = oracle.live_pairs(q_idx, c * C + np.arange(C), True, seg[0, q_idx], seg[0, c * C:(c + 1) * C])
    assert counts[0] == 0 and counts[3] == 0
    assert counts[2] > 0
    # exact count = sum over the samples overlapping the shard of the causal triangle part
    total = 0
    starts = np.concatenate([[0], np.cumsum(wl.lengths)])
    for s0, s1 in zip(starts[:-1], starts[1:]):
        lo, hi = max(s0, r * C), min(s1, (r + 1) * C)
        for i in range(lo, hi):
            total += i - s0 + 1
    assert sum(counts.values()) == total
