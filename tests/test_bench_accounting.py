"""CPU checks of the benchmark's pair and buffer accounting: the closed forms it
divides by (live causal pairs, live packed pairs), the executed-pair count of the
packed forward's tile ranges, and the accumulator views of one flat buffer."""

import numpy as np
import torch

import bench
import oracle


def _brute_live(seg, C, rank, cp):
    q = np.arange(rank * C, (rank + 1) * C)
    k = np.arange(cp * C)
    vis = (k[None, :] <= q[:, None])
    if seg is not None:
        vis &= seg[k][None, :] == seg[q][:, None]
    return int(vis.sum())


def test_live_pairs_causal_closed_form():
    for C, rank in ((1, 0), (5, 0), (5, 3), (64, 7), (33, 2)):
        assert bench.live_pairs_causal(C, rank) == _brute_live(None, C, rank, rank + 1)


def test_packed_live_pairs_match_brute_force():
    rng = np.random.default_rng(4)
    for _ in range(20):
        cp = int(rng.integers(2, 5))
        C = int(rng.integers(8, 60))
        lengths = []
        while sum(lengths) < cp * C:
            lengths.append(int(rng.integers(1, 3 * C)))
        pos = np.concatenate([np.arange(n) for n in lengths])[: cp * C]
        seg = oracle.segment_ids(pos[None, :].astype(np.int32))[0]
        for rank in range(cp):
            assert bench.packed_live_pairs(lengths, C, rank) == _brute_live(seg, C, rank, cp)


def _brute_executed(seg, C, rank, cp, qb, kt):
    total = 0
    for c in range(cp):
        for q0 in range(0, C, qb):
            qs = np.arange(rank * C + q0, rank * C + min(q0 + qb, C))
            live_tiles = []
            for t0 in range(0, C, kt):
                ks = np.arange(c * C + t0, c * C + min(t0 + kt, C))
                causal = ks[0] <= qs[-1]  # some key of the tile is not after every query
                shares = bool(np.intersect1d(seg[ks], seg[qs]).size) or (
                    seg[ks[-1]] >= seg[qs[0]] and seg[ks[0]] <= seg[qs[-1]])
                if causal and shares:
                    live_tiles.append(t0 // kt)
            if live_tiles:
                total += qb * kt * (live_tiles[-1] - live_tiles[0] + 1)
    return total


def test_packed_executed_pairs_follow_the_tile_ranges():
    rng = np.random.default_rng(9)
    for _ in range(10):
        cp, C = 3, 96
        lengths = []
        while sum(lengths) < cp * C:
            lengths.append(int(rng.integers(10, 150)))
        pos = np.concatenate([np.arange(n) for n in lengths])[: cp * C]
        seg = oracle.segment_ids(pos[None, :].astype(np.int32))[0]
        for rank in range(cp):
            e = bench.packed_executed_pairs(np, seg, C, rank, cp, qblock=16, ktile=8)
            assert e == _brute_executed(seg, C, rank, cp, 16, 8)
            assert e >= bench.packed_live_pairs(lengths, C, rank)


def test_flat_grads_are_disjoint_views_of_one_buffer():
    g = bench.flat_grads(torch, torch.device("cpu"), (1, 5, 2, 3), [(1, 4, 1, 3), (1, 4, 1, 3), (1, 2, 1, 3)])
    views = [g["dq"]] + g["dk_chunks"] + g["dv_chunks"]
    assert sum(v.numel() for v in views) == g["flat"].numel()
    for i, v in enumerate(views):
        g["flat"].zero_()
        v.fill_(1.0)
        assert float(g["flat"].sum()) == v.numel()
        assert v.is_contiguous() and v.data_ptr() >= g["flat"].data_ptr()
