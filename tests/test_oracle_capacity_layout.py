"""Pins for the per-expert capacity rule and the expert-contiguous layout.

Capacity (docs.axolotl.ai expert-parallel args, `expert_parallel_token_capacity`): at most
C assignments per expert; the lowest-weight excess is dropped, ties to the lower token
index.  Pinned by enumerating every C-subset on tiny tie-heavy inputs.

Layout (LightLLM PR #1687, expert prefix-sum layout): pinned by a stable sort of the
kept (expert, token) pairs and by the invariants every layout must satisfy.
"""
import itertools

import numpy as np
import pytest

import oracle


def brute_keep(ids, w, E, C):
    T, k = ids.shape
    keep = np.ones((T, k), np.uint8)
    for e in range(E):
        cands = [(t, j) for t in range(T) for j in range(k) if ids[t, j] == e]
        if len(cands) <= C:
            continue
        best, best_seq = None, None
        for sub in itertools.combinations(cands, C):
            seq = sorted(((float(w[t, j]), -t) for t, j in sub), reverse=True)
            if best_seq is None or seq > best_seq:
                best, best_seq = sub, seq
        for t, j in cands:
            if (t, j) not in best:
                keep[t, j] = 0
    return keep


@pytest.mark.parametrize("seed", range(8))
def test_capacity_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    for E, k in [(3, 1), (3, 2), (4, 2), (4, 3)]:
        for C in (1, 2, 3):
            T = 6
            l = rng.integers(0, 2, size=(T, E)).astype(np.float32)  # many equal weights
            if seed % 2:
                l = l + rng.standard_normal((T, E)).astype(np.float32) * 0.1
            ids, w = oracle.route(l, k)
            keep = oracle.capacity(ids, w, E, C)
            assert np.array_equal(keep, brute_keep(ids, w, E, C)), (E, k, C)


def test_equal_weights_keep_lowest_tokens():
    T, E, k, C = 20, 4, 2, 3
    l = np.zeros((T, E), np.float32)  # every token picks experts 0, 1 with w = 1/2
    ids, w = oracle.route(l, k)
    keep = oracle.capacity(ids, w, E, C)
    assert keep[:C].all() and not keep[C:].any()


def test_cap_at_or_above_T_is_no_cap():
    rng = np.random.default_rng(5)
    T, E, k = 40, 5, 2
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    assert oracle.capacity(ids, w, E, T).all()
    assert oracle.capacity(ids, w, E, 0).all()


def check_layout(ids, keep, E, lay, C=0):
    T, k = ids.shape
    counts, offsets, rt, s2r, N = (lay[n] for n in ("counts", "offsets", "row_token", "slot_to_row", "N"))
    kept = keep.astype(bool) if keep is not None else np.ones_like(ids, bool)
    # offsets is the exclusive scan of counts, and counts count kept assignments
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert N == offsets[-1] == kept.sum()
    assert np.array_equal(counts, np.bincount(ids[kept], minlength=E))
    if C > 0:
        assert counts.max(initial=0) <= C
    # every kept slot appears exactly once, dropped slots are -1, maps are inverse
    assert np.all(s2r[~kept] == -1)
    rows = s2r[kept]
    assert np.array_equal(np.sort(rows), np.arange(N))
    tt = np.nonzero(kept)[0]
    assert np.array_equal(rt[rows], tt)
    # each row lies in its expert's segment; tokens strictly increase inside a segment
    ee = ids[kept]
    assert np.all((offsets[ee] <= rows) & (rows < offsets[ee + 1]))
    for e in range(E):
        seg = rt[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


@pytest.mark.parametrize("T,E,k,C", [(1, 1, 1, 0), (7, 3, 2, 0), (64, 8, 2, 0), (300, 16, 4, 0),
                                     (300, 16, 4, 40), (257, 32, 8, 0), (500, 8, 3, 100)])
def test_layout_invariants_and_stable_sort(T, E, k, C):
    rng = np.random.default_rng(T + E + k + C)
    l = rng.standard_normal((T, E)).astype(np.float32) + np.linspace(0, 2, E, dtype=np.float32)
    ids, w = oracle.route(l, k)
    keep = oracle.capacity(ids, w, E, C)
    lay = oracle.layout(ids, keep, E)
    check_layout(ids, keep, E, lay, C)
    # the permutation is the stable sort of the kept slots by expert id
    tt, jj = np.nonzero(keep.astype(bool))
    order = sorted(range(len(tt)), key=lambda i: (ids[tt[i], jj[i]], tt[i]))
    assert np.array_equal(lay["row_token"][:lay["N"]], tt[order])


def test_dropped_set_is_the_lowest_key_excess():
    # skewed routing with a cap: several experts overflow
    rng = np.random.default_rng(3)
    T, E, k, C = 512, 16, 4, 64
    bias = -1.2 * np.log(rng.permutation(E) + 1.0)
    l = (rng.standard_normal((T, E)) + bias).astype(np.float32)
    ids, w = oracle.route(l, k)
    keep = oracle.capacity(ids, w, E, C)
    n_over = 0
    for e in range(E):
        m = ids == e
        cand = np.nonzero(m)
        keys = [(float(w[t, j]), -t) for t, j in zip(*cand)]
        kept = [kk for kk, (t, j) in zip(keys, zip(*cand)) if keep[t, j]]
        drop = [kk for kk, (t, j) in zip(keys, zip(*cand)) if not keep[t, j]]
        if len(keys) <= C:
            assert not drop
            continue
        n_over += 1
        assert len(kept) == C
        assert max(drop) < min(kept)
    assert n_over >= 2
    check_layout(ids, keep, E, oracle.layout(ids, keep, E), C)


def test_all_tokens_to_one_expert():
    T, E, k, C = 100, 4, 2, 10
    l = np.zeros((T, E), np.float32)
    l[:, 0] = 5.0
    ids, w = oracle.route(l, k)
    keep = oracle.capacity(ids, w, E, C)
    lay = oracle.layout(ids, keep, E)
    assert lay["counts"].tolist() == [10, 10, 0, 0]
    check_layout(ids, keep, E, lay, C)


def test_gather_is_row_copy():
    rng = np.random.default_rng(9)
    x = rng.integers(0, 65535, size=(10, 8)).astype(np.uint16)
    rt = np.array([3, 3, 0, 9, 1], np.int32)
    xp = oracle.gather(x, rt, 5)
    assert np.array_equal(xp, x[rt])
