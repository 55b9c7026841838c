"""Pins for routing: top-k selection and softmax weights.

Selection is pinned by brute-force enumeration of every k-subset on tiny inputs (random
and tie-heavy), the weights by the literal fp64 "softmax over all experts -> take top-k
-> renormalise" and by closed forms (k = E, equal logits).
"""
import itertools

import numpy as np
import pytest

import oracle


def brute_topk(l, k):
    """Best k-subset by enumeration: the subset whose (logit desc, id asc) sequence is
    lexicographically largest.  Returns ids in slot order."""
    E = len(l)
    best = None
    for sub in itertools.combinations(range(E), k):
        seq = sorted(((float(l[e]), -e) for e in sub), reverse=True)
        if best is None or seq > best:
            best = seq
    return [-e for _, e in best]


def softmax64(l):
    l = np.asarray(l, np.float64)
    p = np.exp(l - l.max(axis=-1, keepdims=True))
    return p / p.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("tie_heavy", [False, True])
def test_selection_brute_force(seed, tie_heavy):
    rng = np.random.default_rng(seed)
    for E in range(1, 6):
        for k in range(1, min(3, E) + 1):
            T = 6
            if tie_heavy:
                l = rng.integers(0, 3, size=(T, E)).astype(np.float32)
            else:
                l = rng.standard_normal((T, E)).astype(np.float32)
            ids, w = oracle.route(l, k)
            for t in range(T):
                assert list(ids[t]) == brute_topk(l[t], k), (l[t], ids[t])


def test_signed_zero_ties_go_to_lower_index():
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    ids, w = oracle.route(l, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]
    assert np.all(w == np.float32(0.5))


@pytest.mark.parametrize("E,k", [(8, 2), (64, 4), (128, 8), (256, 8)])
def test_weights_match_literal_softmax(E, k):
    rng = np.random.default_rng(E * 31 + k)
    l = (rng.standard_normal((300, E)) * 2.0).astype(np.float32)
    ids, w = oracle.route(l, k)
    p = softmax64(l)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    # error budget of the fp32 arithmetic: two exps (<= 1 ulp each, pinned exhaustively),
    # k-1 additions (1/2 ulp each) and one division (1/2 ulp), all relative to 2^-24
    assert (np.abs(w - ref) / ref).max() <= (k + 4) * 2.0 ** -24
    # the renormalised weights sum to one
    assert np.abs(w.astype(np.float64).sum(axis=1) - 1.0).max() <= 4 * k * 2.0 ** -24
    # slots are in non-increasing weight order
    assert np.all(np.diff(w, axis=1) <= 0)


def test_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((50, 6)).astype(np.float32)
    ids, w = oracle.route(l, 6)
    full = softmax64(l)
    got = np.zeros_like(full)
    np.put_along_axis(got, ids.astype(np.int64), w.astype(np.float64), axis=1)
    assert (np.abs(got - full) / full).max() <= (6 + 4) * 2.0 ** -24


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_equal_logits(k):
    l = np.full((5, 16), 0.375, np.float32)
    ids, w = oracle.route(l, k)
    assert np.all(ids == np.arange(k)[None, :])
    assert np.all(w == np.float32(1.0 / k))


def test_without_renormalisation_is_plain_softmax_of_the_selected():
    rng = np.random.default_rng(11)
    E, k = 32, 4
    l = rng.standard_normal((100, E)).astype(np.float32)
    ids, w = oracle.route(l, k, renormalize=0)
    ref = np.take_along_axis(softmax64(l), ids.astype(np.int64), axis=1)
    # the divisor is a left-to-right fp32 sum of E terms
    assert (np.abs(w - ref) / ref).max() <= E * 2.0 ** -23
    ids2, _ = oracle.route(l, k, renormalize=1)
    assert np.array_equal(ids, ids2)


def test_weights_depend_only_on_logit_differences():
    # shifting all logits of a token by an integer changes nothing exactly (x - m is exact
    # for these small integer-spaced values)
    l = np.array([[3.0, 1.0, 2.0, 0.0]], np.float32)
    a = oracle.route(l, 3)
    b = oracle.route(l + 8.0, 3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
