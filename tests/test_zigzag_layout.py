"""Host logic of the load-balanced causal layout (CPU): the data placement, the
pair schedule of the ring loop, and the balance it exists for.

Pins: every token is held by exactly one rank; the schedule keeps exactly the
(query half, key half) pairs that have a visible pair (brute force over the
index sets with the oracle's mask); every rank's visible-pair count equals the
closed form 2*cp*h^2 + h, against (r + 1/2) C^2 + C/2 for contiguous chunks
(aicassindra, "Transformer math: SP math": the causal load-balance problem)."""

import numpy as np
import pytest

import oracle
from context_long_sequence_amd.ring import ring_schedule, zigzag_halves, zigzag_pairs
from synthetic import zigzag_indices


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_every_token_held_once(cp):
    S = 2 * cp * 16
    held = np.concatenate([zigzag_indices(S, cp, r) for r in range(cp)])
    np.testing.assert_array_equal(np.sort(held), np.arange(S))


@pytest.mark.parametrize("cp", [2, 4, 8])
def test_host_halves_match_the_placement(cp):
    S, h = 2 * cp * 8, 8
    for r in range(cp):
        idx = zigzag_indices(S, cp, r)
        lo, hi = zigzag_halves(r, cp)
        np.testing.assert_array_equal(idx[:h], np.arange(lo * h, lo * h + h))
        np.testing.assert_array_equal(idx[h:], np.arange(hi * h, hi * h + h))


@pytest.mark.parametrize("cp,h", [(2, 4), (4, 3), (8, 2), (3, 5)])
@pytest.mark.parametrize("causal", [True, False])
def test_pair_schedule_is_exactly_the_live_pairs(cp, h, causal):
    S = 2 * cp * h
    for r in range(cp):
        q_idx = zigzag_indices(S, cp, r)
        expect = []
        for i, c in enumerate(ring_schedule(r, cp)):
            k_idx = zigzag_indices(S, cp, c)
            for j in range(2):
                for k in range(2):
                    if oracle.live_pairs(q_idx[j * h:(j + 1) * h], k_idx[k * h:(k + 1) * h], causal) > 0:
                        expect.append((i, c, j, k))
        assert zigzag_pairs(r, cp, h, causal) == expect


@pytest.mark.parametrize("cp,h", [(2, 8), (4, 8), (8, 4)])
def test_balanced_work(cp, h):
    S, C = 2 * cp * h, 2 * h
    k_idx = np.arange(S)
    zig = [oracle.live_pairs(zigzag_indices(S, cp, r), k_idx, True) for r in range(cp)]
    assert zig == [2 * cp * h * h + h] * cp
    contig = [oracle.live_pairs(np.arange(r * C, (r + 1) * C), k_idx, True) for r in range(cp)]
    assert contig == [r * C * C + C * (C + 1) // 2 for r in range(cp)]
    assert sum(zig) == sum(contig) == S * (S + 1) // 2
