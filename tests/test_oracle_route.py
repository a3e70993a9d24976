"""Pins of the oracle's token->expert permutation (stable counting sort).

The pages have the GPU route 32-token decode blocks to experts (minnow README,
section "Quantization"); the permutation groups the slots s = t*K + k by expert
so each expert's rows are contiguous.  Checked against brute force (Python's
sort on (expert, slot)) and the permutation's invariants.
"""
import numpy as np
import pytest

import oracle


def _brute(ids, E):
    S = ids.size
    flat = ids.reshape(-1)
    valid = [s for s in range(S) if 0 <= flat[s] < E]
    order = sorted(valid, key=lambda s: (flat[s], s))
    counts = np.bincount(flat[valid], minlength=E) if valid else np.zeros(E, int)
    return order, counts


@pytest.mark.parametrize("T,K,E,seed", [(37, 3, 11, 0), (32, 8, 256, 1), (5, 1, 3, 2), (64, 4, 4, 3)])
def test_route_matches_brute_force(T, K, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)     # duplicates within a token allowed
    counts, offsets, sorted_slot, slot_row, nbad = oracle.route(ids, E)
    order, c_ref = _brute(ids, E)
    assert nbad == 0
    np.testing.assert_array_equal(counts, c_ref)
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(c_ref)]))
    np.testing.assert_array_equal(sorted_slot, order)
    S = T * K
    np.testing.assert_array_equal(sorted_slot[slot_row], np.arange(S))   # inverse permutation
    assert np.all(np.diff(offsets) >= 0) and offsets[-1] == S
    # each expert's segment holds exactly its slots, ascending
    for e in range(E):
        seg = sorted_slot[offsets[e]:offsets[e + 1]]
        assert np.all(ids.reshape(-1)[seg] == e) and np.all(np.diff(seg) > 0)


def test_route_drops_out_of_range_ids():
    ids = np.array([[0, 5], [-1, 2], [2, 99], [1, 0]], np.int32)
    E = 3
    counts, offsets, sorted_slot, slot_row, nbad = oracle.route(ids, E)
    assert nbad == 3
    np.testing.assert_array_equal(counts, [2, 1, 2])
    assert offsets[-1] == 5
    np.testing.assert_array_equal(sorted_slot[:5], [0, 7, 6, 3, 4])
    np.testing.assert_array_equal(sorted_slot[5:], -1)
    np.testing.assert_array_equal(slot_row, [0, -1, -1, 3, 4, -1, 2, 1])


def test_route_empty():
    ids = np.zeros((0, 4), np.int32)
    counts, offsets, sorted_slot, slot_row, nbad = oracle.route(ids, 7)
    assert nbad == 0 and counts.sum() == 0 and np.all(offsets == 0)
