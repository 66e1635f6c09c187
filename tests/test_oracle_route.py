"""Pins of the routing oracle: brute-force sorting, constructed ties, special cases that reduce to
the plain softmax, and a brute-force stable counting sort."""

import math

import numpy as np
import pytest
import scipy.special

from oracle import route as R


def brute_route(logits, k, renormalize):
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        lt = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-lt[e], e))[:k]
        ex = [math.exp(v - max(lt)) for v in lt]
        den = math.fsum(ex[e] for e in order) if renormalize else math.fsum(ex)
        ids[t] = order
        w[t] = [ex[e] / den for e in order]
    return ids, w


@pytest.mark.parametrize("T,E,k,ren", [(7, 5, 2, True), (9, 16, 4, False), (5, 3, 3, True), (20, 32, 8, True)])
def test_route_matches_brute_force(T, E, k, ren):
    g = np.random.default_rng(T * E + k)
    logits = g.standard_normal((T, E)).astype(np.float32)
    ids, w = R.route_ref(logits, k, ren)
    bi, bw = brute_route(logits, k, ren)
    np.testing.assert_array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-14, atol=0)


def test_ties_go_to_lower_expert_index():
    logits = np.array([[0.5, 1.0, 1.0, 0.5, 1.0, -0.0, 0.0]], np.float32)
    ids, w = R.route_ref(logits, 5, True)
    assert ids[0].tolist() == [1, 2, 4, 0, 3]
    ids, _ = R.route_ref(logits, 7, True)
    assert ids[0].tolist() == [1, 2, 4, 0, 3, 5, 6]  # -0.0 and 0.0 compare equal


def test_k_equals_E_is_the_softmax():
    g = np.random.default_rng(4)
    logits = g.standard_normal((6, 9)).astype(np.float32)
    ids, w = R.route_ref(logits, 9, True)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)
    ids2, w2 = R.route_ref(logits, 3, False)
    np.testing.assert_allclose(w2, np.take_along_axis(p, ids2.astype(np.int64), 1), rtol=1e-13)


def test_k1_renormalized_weight_is_one_and_sums():
    g = np.random.default_rng(5)
    logits = g.standard_normal((50, 12)).astype(np.float32)
    _, w = R.route_ref(logits, 1, True)
    assert np.all(w == 1.0)
    _, w = R.route_ref(logits, 4, True)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending logits give descending weights
    _, w = R.route_ref(logits, 4, False)
    assert np.all(w.sum(1) < 1.0)
    with pytest.raises(ValueError):
        R.route_ref(logits, 13, True)


def test_sort_pairs_matches_brute_force():
    g = np.random.default_rng(6)
    T, E, k = 40, 7, 3
    logits = g.standard_normal((T, E)).astype(np.float32)
    ids, _ = R.route_ref(logits, k, True)
    offsets, sp = R.sort_pairs_ref(ids, E)
    flat = ids.reshape(-1).tolist()
    want, want_off = [], [0]
    for e in range(E):
        want += [p for p in range(T * k) if flat[p] == e]
        want_off.append(len(want))
    assert sp.tolist() == want
    assert offsets.tolist() == want_off
    assert offsets[-1] == T * k
