"""Pins of the oracle's backward pass (oracle/backward.py).

Two independent checks of every gradient: central finite differences of the oracle's own
forward (oracle.layer, the C implementation), and torch autograd in fp64 on a dense
restatement of the forward (every token times every expert, masked by the oracle's
selection, which is piecewise constant).  Cases: renormalised and plain softmax weights,
a capacity that drops assignments, and a router in front (logits = x W_r^T).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import backward as ob


def make(T, H, E, k, I, seed, router=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (rng.standard_normal((E, H, I)) / np.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, H, I)) / np.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, I, H)) / np.sqrt(I)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32) if router else None
    lg = rng.standard_normal((T, E)).astype(np.float32)
    dy = rng.standard_normal((T, H))
    return x, lg, wg, wu, wd, wr, dy


def logits_of(x, lg, wr):
    return (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32) if wr is not None else lg


def objective(x, lg, wg, wu, wd, wr, dy, k, cap, renorm):
    out = oracle.layer(x, logits_of(x, lg, wr), wg, wu, wd, k, cap, renorm)
    return float(np.sum(out["y"] * dy))


CASES = [dict(renorm=1, cap=0, router=False), dict(renorm=0, cap=0, router=False),
         dict(renorm=1, cap=3, router=False), dict(renorm=1, cap=0, router=True)]


@pytest.mark.parametrize("case", CASES, ids=["renorm", "plain_softmax", "capacity", "router"])
def test_backward_matches_finite_differences(case):
    T, H, E, k, I = 7, 8, 4, 2, 6
    x, lg, wg, wu, wd, wr, dy = make(T, H, E, k, I, seed=5 + case["cap"] + case["renorm"], router=case["router"])
    args = (k, case["cap"], case["renorm"])
    g = ob.layer_backward(x, logits_of(x, lg, wr), wg, wu, wd, k, dy, case["cap"], case["renorm"],
                          w_router=wr)
    if case["cap"]:
        assert np.any(g["keep"] == 0)  # the cap drops something
    rng = np.random.default_rng(1)
    h = 1e-2

    def fd(arr, idx, build):
        a0 = arr.copy()
        ap, am = a0.copy(), a0.copy()
        ap[idx] += h
        am[idx] -= h
        fp, fm = objective(*build(ap), dy, *args), objective(*build(am), dy, *args)
        dh = float(ap[idx]) - float(am[idx])  # the step actually taken in f32
        return (fp - fm) / dh

    tensors = {
        "dx": (x, lambda v: (v, lg, wg, wu, wd, wr)),
        "dw_gate": (wg, lambda v: (x, lg, v, wu, wd, wr)),
        "dw_up": (wu, lambda v: (x, lg, wg, v, wd, wr)),
        "dw_down": (wd, lambda v: (x, lg, wg, wu, v, wr)),
    }
    if case["router"]:
        tensors["dw_router"] = (wr, lambda v: (x, lg, wg, wu, wd, v))
    else:
        tensors["dlogits"] = (lg, lambda v: (x, v, wg, wu, wd, wr))
    for name, (arr, build) in tensors.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            num = fd(arr, idx, build)
            ana = g[name][idx]
            assert abs(num - ana) <= 2e-3 * max(1.0, abs(ana)), (name, idx, num, ana)


@pytest.mark.parametrize("case", CASES, ids=["renorm", "plain_softmax", "capacity", "router"])
def test_backward_matches_torch_autograd(case):
    T, H, E, k, I = 11, 16, 5, 2, 12
    x, lg, wg, wu, wd, wr, dy = make(T, H, E, k, I, seed=9, router=case["router"])
    logits = logits_of(x, lg, wr)
    g = ob.layer_backward(x, logits, wg, wu, wd, k, dy, case["cap"], case["renorm"], w_router=wr)
    ids, keep = g["topk_ids"], g["keep"]
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    Wg = torch.tensor(wg, dtype=torch.float64, requires_grad=True)
    Wu = torch.tensor(wu, dtype=torch.float64, requires_grad=True)
    Wd = torch.tensor(wd, dtype=torch.float64, requires_grad=True)
    if case["router"]:
        Wr = torch.tensor(wr, dtype=torch.float64, requires_grad=True)
        L = X @ Wr.T
    else:
        L = torch.tensor(lg, dtype=torch.float64, requires_grad=True)
    sel = torch.zeros(T, E, dtype=torch.float64)
    kept = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            sel[t, ids[t, j]] = 1.0
            kept[t, ids[t, j]] = float(keep[t, j])
    if case["renorm"]:
        ex = torch.exp(L - L.max(dim=1, keepdim=True).values) * sel
        wts = ex / ex.sum(dim=1, keepdim=True)
    else:
        wts = torch.softmax(L, dim=1) * sel
    G = torch.einsum("th,ehi->tei", X, Wg)
    U = torch.einsum("th,ehi->tei", X, Wu)
    A = G * torch.sigmoid(G) * U
    Yp = torch.einsum("tei,eih->teh", A, Wd)
    Y = torch.einsum("te,teh->th", wts * kept, Yp)
    (Y * torch.tensor(dy)).sum().backward()
    pairs = [("dx", X), ("dw_gate", Wg), ("dw_up", Wu), ("dw_down", Wd)]
    pairs.append(("dw_router", Wr) if case["router"] else ("dlogits", L))
    # the oracle's routing weights are the specified fp32 values (torch's are fp64): agree
    # to fp32 rounding, 2^-24 relative per weight
    for name, t in pairs:
        ref = t.grad.numpy()
        assert np.allclose(g[name], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max()), name


def test_backward_expert_subset_and_zero_upstream():
    x, lg, wg, wu, wd, _, dy = make(9, 8, 4, 2, 6, seed=3)
    full = ob.layer_backward(x, lg, wg, wu, wd, 2, dy)
    sub = ob.layer_backward(x, lg, wg, wu, wd, 2, dy, experts=np.array([3, 1]))
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(sub[n], full[n][[3, 1]])
    assert np.array_equal(sub["dx"], full["dx"]) and np.array_equal(sub["dlogits"], full["dlogits"])
    zero = ob.layer_backward(x, lg, wg, wu, wd, 2, np.zeros_like(dy))
    for n in ("dx", "dw_gate", "dw_up", "dw_down", "dlogits"):
        assert not np.any(zero[n])


def test_backward_token_subset():
    x, lg, wg, wu, wd, _, dy = make(12, 8, 4, 2, 6, seed=4)
    full = ob.layer_backward(x, lg, wg, wu, wd, 2, dy)
    toks = np.array([0, 5, 11])
    sub = ob.layer_backward(x, lg, wg, wu, wd, 2, dy, experts=np.array([2]), tokens=toks)
    for n in ("dx", "dlogits", "dtopk_w"):
        assert np.allclose(sub[n][toks], full[n][toks], rtol=1e-13, atol=1e-13), n
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert np.allclose(sub[n][0], full[n][2], rtol=1e-13, atol=1e-13), n


def test_gate_up_rows_gives_the_ffn_activation():
    """silu(g) * u from the backward's pre-activations (numpy) equals the activation a of
    the C oracle's expert FFN on the same rows, and rows of experts left out stay zero."""
    rng = np.random.default_rng(11)
    T, H, E, k, I = 40, 64, 5, 2, 96
    x = synth.bf16_bits(torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16))
    wg, wu = (synth.bf16_bits(torch.from_numpy(rng.standard_normal((E, H, I), dtype=np.float32) * 0.1)
                              .to(torch.bfloat16)) for _ in range(2))
    wd = synth.bf16_bits(torch.from_numpy(rng.standard_normal((E, I, H), dtype=np.float32) * 0.1)
                         .to(torch.bfloat16))
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    lay = oracle.layout(ids, None, E)
    N = lay["N"]
    g, u = ob.gate_up_rows(x, lay["row_token"], lay["offsets"], wg, wu)
    rexp = (np.searchsorted(lay["offsets"], np.arange(N), side="right") - 1).astype(np.int32)
    _, a = oracle.ffn_rows(oracle.gather(x, lay["row_token"], N), rexp, wg, wu, wd, want_a=True)
    ref = g / (1.0 + np.exp(-g)) * u
    assert np.abs(ref - a).max() <= 1e-12 * np.abs(a).max()
    g2, u2 = ob.gate_up_rows(x, lay["row_token"], lay["offsets"], wg, wu, experts=[1, 3])
    mine = np.isin(rexp, [1, 3])
    assert np.array_equal(g2[mine], g[mine]) and np.array_equal(u2[mine], u[mine])
    assert not g2[~mine].any() and not u2[~mine].any()
