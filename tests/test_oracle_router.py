"""Pins of the oracle's router (top-K selection + softmax weights) against
definitions that do not go through the oracle's code: a brute-force sort
with an explicit tie rule, closed-form softmax values, exact invariances, and
the independent NumPy routing of the input generator."""
import math

import numpy as np
import pytest

import oracle
from harness.inputs import topk_softmax as np_topk_softmax

U = 2.0 ** -24   # FP32 unit roundoff


def brute_ids(l, K):
    """Order experts by (-logit, id) and keep the first K."""
    return [e for e in sorted(range(len(l)), key=lambda e: (-float(l[e]), e))[:K]]


@pytest.mark.parametrize("T,E,K,seed", [(7, 8, 2, 0), (5, 64, 8, 1), (3, 256, 8, 2), (4, 100, 100, 3),
                                        (6, 1024, 16, 4), (2, 17, 1, 5)])
def test_selection_matches_brute_force(T, E, K, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.topk_softmax(l, K)
    for t in range(T):
        assert list(ids[t]) == brute_ids(l[t], K)


def test_ties_go_to_lower_id():
    # logits from a three-value set: long runs of equal values
    rng = np.random.default_rng(11)
    l = rng.choice(np.array([-1.0, 0.0, 2.5], dtype=np.float32), size=(20, 48))
    l[3, :] = 1.0                                     # every logit equal
    l[4, 10] = np.float32(-np.inf)                    # -inf entries are never preferred
    ids, w = oracle.topk_softmax(l, 6)
    for t in range(20):
        assert list(ids[t]) == brute_ids(l[t], 6)
    assert list(ids[3]) == [0, 1, 2, 3, 4, 5]
    np.testing.assert_array_equal(w[3], np.float32(1.0 / 6.0))


def test_softmax_closed_forms():
    # K = 1: the single weight is exactly one
    l = np.array([[0.3, -2.0, 7.0, 1.0]], dtype=np.float32)
    ids, w = oracle.topk_softmax(l, 1)
    assert ids[0, 0] == 2 and w[0, 0] == np.float32(1.0)
    # two selected logits ln 3 and 0: weights 3/4 and 1/4
    l = np.array([[0.0, -5.0, math.log(3.0), -9.0]], dtype=np.float32)
    ids, w = oracle.topk_softmax(l, 2)
    assert list(ids[0]) == [2, 0]
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=4 * U)
    # equal spacing by ln 2: weights 4/7, 2/7, 1/7
    l = np.array([[-math.log(2.0), 0.0, -2 * math.log(2.0)]], dtype=np.float32)
    ids, w = oracle.topk_softmax(l, 3)
    assert list(ids[0]) == [1, 0, 2]
    np.testing.assert_allclose(w[0], [4 / 7, 2 / 7, 1 / 7], rtol=8 * U)


def test_invariants_and_shift():
    rng = np.random.default_rng(7)
    T, E, K = 64, 256, 8
    # multiples of 2^-10 within (-8, 8): adding 16 is exact, and so are the
    # differences of shifted logits, so the weights must not change at all
    l = (np.round(rng.standard_normal((T, E)) * 1024) / 1024).clip(-7.9, 7.9).astype(np.float32)
    ids, w = oracle.topk_softmax(l, K)
    assert np.all(w > 0)
    assert np.all(np.diff(w, axis=1) <= 0)            # descending logits give non-increasing weights
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=K * U)
    for t in range(T):
        assert len(set(ids[t])) == K and ids[t].min() >= 0 and ids[t].max() < E
    ids2, w2 = oracle.topk_softmax(l + np.float32(16.0), K)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_array_equal(w2, w)


def test_matches_numpy_routing():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((200, 256)).astype(np.float32)
    ids, w = oracle.topk_softmax(l, 8)
    ids_np, w_np = np_topk_softmax(l, 8)
    np.testing.assert_array_equal(ids, ids_np)
    np.testing.assert_allclose(w, w_np, rtol=16 * U, atol=0)


def test_rejects_bad_k():
    l = np.zeros((2, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.topk_softmax(l, 5)
    with pytest.raises(ValueError):
        oracle.topk_softmax(l, 0)
