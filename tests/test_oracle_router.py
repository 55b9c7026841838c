"""Pins of the oracle's routing front-end: group-limited top-k and the router logits.

Group-limited selection is pinned by the hand-worked fixture in tests/golden/, by the
special cases that reduce to plain top-k (one group; every group taken; one expert per
group), by brute force over every choice of groups on tiny inputs (the taken groups are the
unique set whose worst (score, -index) beats the best left out), and by invariants.  The
router logits are pinned by one-hot gate rows (exact copies of x's columns), linearity and
numpy's fp64 matrix product.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "grouped_route_handworked.json")


def test_grouped_handworked_example():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        l = np.array(case["logits"], np.float32)
        ids, w = oracle.route_grouped(l, case["k"], case["n_group"], case["topk_group"],
                                      case["renormalize"])
        assert ids.tolist() == case["topk_ids"], case["derivation"]
        ref = np.array(case["topk_w"])
        # the routing weights' error bound of the specified fp32 arithmetic (k + 4 ulp;
        # without renormalisation the sum runs over E terms: E + 4)
        n = case["k"] if case["renormalize"] else l.shape[1]
        assert (np.abs(w - ref) / ref).max() <= (n + 4) * 2.0 ** -24


def logits_sets(T, E, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, E)).astype(np.float32),
            rng.integers(0, 3, (T, E)).astype(np.float32)]  # tie-heavy


@pytest.mark.parametrize("renorm", [1, 0])
def test_grouped_reduces_to_plain_top_k(renorm):
    for E, k in ((8, 2), (64, 6), (256, 8)):
        for l in logits_sets(97, E, E + renorm):
            ids0, w0 = oracle.route(l, k, renorm)
            for n_group, topk_group in ((1, 1), (4, 4), (E, E)):
                ids, w = oracle.route_grouped(l, k, n_group, topk_group, renorm)
                assert np.array_equal(ids, ids0) and np.array_equal(w.view(np.uint32), w0.view(np.uint32))
            # one expert per group, k groups: the k best experts
            ids, w = oracle.route_grouped(l, k, E, k, renorm)
            assert np.array_equal(ids, ids0) and np.array_equal(w.view(np.uint32), w0.view(np.uint32))


def brute_force(l, k, n_group, topk_group):
    """The taken groups are the unique set S of topk_group groups with
    min over S of (score, -g) > max over the rest of (score, -g); then the k best experts
    of S by (logit, -e), best first."""
    E = l.size
    gs = E // n_group
    key = [(float(l[g * gs:(g + 1) * gs].max()), -g) for g in range(n_group)]
    found = []
    for S in itertools.combinations(range(n_group), topk_group):
        rest = [g for g in range(n_group) if g not in S]
        if not rest or min(key[g] for g in S) > max(key[g] for g in rest):
            found.append(S)
    assert len(found) == 1
    cand = [e for g in found[0] for e in range(g * gs, (g + 1) * gs)]
    return sorted(cand, key=lambda e: (-float(l[e]), e))[:k]


def test_grouped_brute_force_on_tiny_inputs():
    rng = np.random.default_rng(11)
    for E, n_group in ((4, 2), (6, 3), (8, 4), (8, 2), (9, 3)):
        gs = E // n_group
        for topk_group in range(1, n_group + 1):
            for k in range(1, min(topk_group * gs, 4) + 1):
                for trial in range(40):
                    l = (rng.integers(0, 3, E) if trial % 2 else rng.standard_normal(E))
                    l = l.astype(np.float32)[None, :]
                    ids, _ = oracle.route_grouped(l, k, n_group, topk_group)
                    assert ids[0].tolist() == brute_force(l[0], k, n_group, topk_group)


def test_grouped_invariants():
    rng = np.random.default_rng(5)
    T, E, k, n_group, topk_group = 500, 256, 8, 8, 4
    l = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route_grouped(l, k, n_group, topk_group)
    gs = E // n_group
    for t in range(T):
        groups = set(int(e) // gs for e in ids[t])
        assert len(groups) <= topk_group
        assert len(set(ids[t].tolist())) == k
        sel = l[t, ids[t]]
        assert np.all(np.diff(sel) <= 0)                   # slot order: logit descending
        assert ids[t, 0] == int(np.argmax(l[t]))           # the best expert is always taken
    assert np.allclose(w.sum(axis=1), 1.0, atol=(k + 4) * 2.0 ** -24 * 2)
    # the first slot is the overall best expert with or without groups
    ids0, _ = oracle.route(l, k)
    assert np.all(ids[:, 0] == ids0[:, 0])


def test_router_logits_pins():
    rng = np.random.default_rng(3)
    T, H, E = 37, 96, 12
    x = rng.standard_normal((T, H)).astype(np.float32)
    # one-hot gate rows copy columns of x exactly
    cols = rng.integers(0, H, E)
    onehot = np.zeros((E, H), np.float32)
    onehot[np.arange(E), cols] = 1.0
    assert np.array_equal(oracle.router_logits(x, onehot), x[:, cols].astype(np.float64))
    w = rng.standard_normal((E, H)).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    got = oracle.router_logits(x, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.router_logits(2 * x, w), 2 * got)   # exact scaling
    # bf16 inputs are upcast exactly
    import torch
    xb = torch.from_numpy(x).to(torch.bfloat16)
    wb = torch.from_numpy(w).to(torch.bfloat16)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    got_b = oracle.router_logits(bits(xb), bits(wb))
    ref_b = xb.double().numpy() @ wb.double().numpy().T
    assert np.allclose(got_b, ref_b, rtol=1e-12, atol=1e-12)


def test_combine_with_shared_expert():
    """y = routed combine + shared expert output: zero shared output leaves the combine
    unchanged; a token with every slot dropped gets exactly the shared output; the shared
    expert is the one-expert dense SwiGLU MLP (numpy fp64)."""
    rng = np.random.default_rng(21)
    T, H, k, Is = 6, 16, 2, 24
    yp = rng.standard_normal((T * k, H))
    w = rng.random((T, k)).astype(np.float32)
    s2r = np.arange(T * k, dtype=np.int32).reshape(T, k)
    s2r[2] = -1                                            # token 2: every slot dropped
    toks = np.arange(T, dtype=np.int32)
    base = oracle.combine(toks, w, s2r, yp)
    assert np.array_equal(oracle.combine(toks, w, s2r, yp, np.zeros((T, H))), base)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu = (rng.standard_normal((1, H, Is)).astype(np.float32) for _ in range(2))
    wd = rng.standard_normal((1, Is, H)).astype(np.float32)
    sh = oracle.shared_expert(x, wg, wu, wd)
    g, u = x.astype(np.float64) @ wg[0].astype(np.float64), x.astype(np.float64) @ wu[0].astype(np.float64)
    ref = (g / (1.0 + np.exp(-g)) * u) @ wd[0].astype(np.float64)
    assert np.allclose(sh, ref, rtol=1e-12, atol=1e-12)
    y = oracle.combine(toks, w, s2r, yp, sh)
    assert np.array_equal(y[2], sh[2])
    assert np.allclose(y - sh, base, rtol=0, atol=1e-12)
