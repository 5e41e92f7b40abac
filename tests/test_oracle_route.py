"""Pins of oracle.route_topk against facts that do not come from the oracle."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle import route_topk


def test_distinct_values_all_orderings_small_e():
    # For distinct values 0..E-1 placed by a permutation p, position j of the
    # top-K list must be the expert holding value E-1-j (inverse permutation).
    for E in range(1, 6):
        for p in itertools.permutations(range(E)):
            logits = np.array([p], dtype=np.float32)
            for K in range(1, E + 1):
                idx, _ = route_topk(logits, K)
                expect = [p.index(E - 1 - j) for j in range(K)]
                assert idx[0].tolist() == expect, (p, K)


def test_ties_lower_index_first_exhaustive():
    # Values from {0, 1}: experts holding 1 come first in ascending index,
    # then those holding 0 in ascending index.
    for E in range(1, 6):
        for vals in itertools.product([0.0, 1.0], repeat=E):
            logits = np.array([vals], dtype=np.float32)
            expect = [e for e in range(E) if vals[e] == 1.0] + [e for e in range(E) if vals[e] == 0.0]
            for K in range(1, E + 1):
                idx, _ = route_topk(logits, K)
                assert idx[0].tolist() == expect[:K], (vals, K)


def test_three_level_ties():
    for vals in itertools.product([-1.5, 0.25, 2.0], repeat=4):
        logits = np.array([vals], dtype=np.float32)
        expect = [e for lvl in (2.0, 0.25, -1.5) for e in range(4) if vals[e] == lvl]
        idx, _ = route_topk(logits, 4)
        assert idx[0].tolist() == expect


def test_matches_lexsort_with_forced_ties():
    rng = np.random.default_rng(7)
    for E, K in [(16, 2), (256, 8), (384, 8), (64, 16)]:
        z = rng.standard_normal((300, E)).astype(np.float32)
        z[::3] = np.round(z[::3] * 2) / 2  # many exact ties
        idx, _ = route_topk(z, K)
        ids = np.broadcast_to(np.arange(E), z.shape)
        ref = np.lexsort((ids, -z), axis=-1)[:, :K]
        np.testing.assert_array_equal(idx, ref)


def test_k_equals_e_gives_full_softmax():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((50, 16)).astype(np.float32)
    idx, w = route_topk(z, 16)
    p = scipy.special.softmax(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), axis=1), rtol=1e-12, atol=0)


def test_k1_weight_is_exactly_one():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((40, 256)).astype(np.float32)
    idx, w = route_topk(z, 1)
    assert np.all(w == 1.0)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(z, axis=1))


def test_renormalised_equals_softmax_of_selected_logits():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((64, 256)).astype(np.float32)
    idx, w = route_topk(z, 8)
    sel = np.take_along_axis(z.astype(np.float64), idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-12)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # descending logits give non-increasing weights
    assert np.all(np.diff(w, axis=1) <= 0)


def test_unnormalised_weights_are_softmax_entries():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((20, 64)).astype(np.float32)
    idx, w = route_topk(z, 4, renormalize=False)
    p = scipy.special.softmax(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), axis=1), rtol=1e-12)
    assert np.all(w.sum(axis=1) < 1.0)


def test_large_logits_do_not_overflow():
    z = np.array([[1000.0, 999.0, -1000.0, 998.0]], dtype=np.float32)
    idx, w = route_topk(z, 2)
    assert idx[0].tolist() == [0, 1]
    e = np.exp(-1.0)
    np.testing.assert_allclose(w[0], [1 / (1 + e), e / (1 + e)], rtol=1e-14)


def test_rejects_non_finite():
    with pytest.raises(AssertionError):
        route_topk(np.array([[0.0, np.nan]], dtype=np.float32), 1)
