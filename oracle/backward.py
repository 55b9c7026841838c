"""Backward pass of the MoE layer -- TEST INFRASTRUCTURE ONLY (part of the oracle).

docs.axolotl.ai "integrations.expert_parallel.args", attribute table, row
`expert_parallel_save_dispatch`: the backward reuses the forward's routing (top-k and the
split counts are always saved) and either the saved dispatch rows or rows recomputed from
x.  The gradients are those of the forward this oracle defines (route -> capacity ->
layout -> SwiGLU experts -> combine), written out from the chain rule in fp64, one expert
at a time (numpy matrix products as the primitive):

  y[t]  = sum_{kept j} w[t,j] * yp[r(t,j)],   yp = a Wd[e],  a = silu(g) * u,
  g = x[t] Wg[e],  u = x[t] Wu[e],  silu(z) = z sigma(z)

  dyp[r]   = w[t,j] dy[t]                      dw[t,j] = <yp[r], dy[t]>  (0 if dropped)
  da       = dyp Wd[e]^T                       dWd[e]  = a^T dyp
  du       = da * silu(g)                      dg      = da * u * sigma(g) (1 + g (1 - sigma(g)))
  dx[t]   += dg Wg[e]^T + du Wu[e]^T           dWg[e]  = x_e^T dg,  dWu[e] = x_e^T du
  router:  with renormalisation w_j = e_j / sum_{i in S} e_i over the k selected:
             dl_j = w_j (dw_j - sum_{i in S} w_i dw_i) for j in S, 0 elsewhere;
           without: w_j = p_j, p = softmax over all E:
             dl_e = p_e ([e in S] dw_e - sum_{i in S} w_i dw_i)
  the selection itself is piecewise constant (no gradient through it); with a router
  (logits = x W_r^T): dW_r = dl^T x, dx += dl W_r.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import capacity, layout, route


def _f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gate_up_rows(x, row_token, offsets, w_gate, w_up, experts: Optional[np.ndarray] = None):
    """The pre-activations the backward reuses, per layout row r of expert e (token
    t = row_token[r]): g[r] = x[t] Wg[e] and u[r] = x[t] Wu[e] in fp64 (the forward's
    definition above; LightLLM PR #1687 walkthrough: the gate/up GEMM that silu_and_mul
    follows).  Only the rows of `experts` (default: all) are filled.  Returns (g, u), each
    [offsets[E], I]."""
    offsets = np.asarray(offsets, np.int64)
    E, I = w_gate.shape[0], w_gate.shape[2]
    N = int(offsets[-1])
    g = np.zeros((N, I))
    u = np.zeros((N, I))
    xd = _f64(x)
    for e in (range(E) if experts is None else experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            xe = xd[np.asarray(row_token[r0:r1], np.int64)]
            g[r0:r1] = xe @ _f64(w_gate[e])
            u[r0:r1] = xe @ _f64(w_up[e])
    return g, u


def layer_backward(x, logits, w_gate, w_up, w_down, k: int, dy, capacity_: int = 0,
                   renormalize: int = 1, w_router: Optional[np.ndarray] = None,
                   experts: Optional[np.ndarray] = None, tokens: Optional[np.ndarray] = None):
    """Gradients of the layer for upstream gradient dy [T, H].

    x [T, H], w_gate/w_up [E, H, I], w_down [E, I, H] (f32/f64, or bf16 as uint16);
    logits [T, E] f32 (the routing is recomputed from them exactly as in the forward).
    experts: if given, the weight gradients are computed for these experts only and
    dw_gate / dw_up / dw_down hold just them, in that order ([len(experts), ...]); tokens: if given, dx, dlogits and dtopk_w are computed
    for these tokens only (rows of other tokens are evaluated only where a listed expert's
    weight gradient needs them; the other tokens' entries are left at zero).
    Returns dict(dx [T,H], dw_gate, dw_up [E,H,I], dw_down [E,I,H], dlogits [T,E],
    dtopk_w [T,k], yp [N,H], and dw_router [E,H] if w_router is given), fp64."""
    X = _f64(np.asarray(x))
    # weights stay in their storage type; each expert's are widened when it is evaluated
    Wg_s, Wu_s, Wd_s = np.asarray(w_gate), np.asarray(w_up), np.asarray(w_down)
    dY = _f64(np.asarray(dy))
    T, H = X.shape
    E, _, I = Wg_s.shape
    ids, w = route(np.asarray(logits, np.float32), k, renormalize)
    keep = capacity(ids, w, E, capacity_)
    lay = layout(ids, keep, E)
    N = lay["N"]
    rt, off = lay["row_token"][:N], lay["offsets"]
    s2r = lay["slot_to_row"]
    wsel = np.asarray(experts) if experts is not None else np.arange(E)
    tsel = np.zeros(T, bool)
    tsel[np.asarray(tokens) if tokens is not None else np.arange(T)] = True

    # row -> (token, slot)
    row_t = np.empty(N, np.int64)
    row_w = np.empty(N, np.float64)
    tt, jj = np.nonzero(s2r >= 0)
    row_t[s2r[tt, jj]] = tt
    row_w[s2r[tt, jj]] = w[tt, jj].astype(np.float64)

    dX = np.zeros((T, H))
    slot = {int(e): i for i, e in enumerate(wsel)}  # weight-gradient slot of each expert
    dWg = np.zeros((len(wsel), H, I))
    dWu = np.zeros((len(wsel), H, I))
    dWd = np.zeros((len(wsel), I, H))
    yp = np.zeros((N, H))
    dW = np.zeros((T, k))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        if e in slot:
            rows = np.arange(r0, r1)
        else:
            rows = np.arange(r0, r1)[tsel[rt[r0:r1]]]
            if rows.size == 0:
                continue
        xe = X[rt[rows]]
        Wge, Wue, Wde = _f64(Wg_s[e]), _f64(Wu_s[e]), _f64(Wd_s[e])
        g = xe @ Wge
        u = xe @ Wue
        sg = _sigmoid(g)
        a = g * sg * u
        ype = a @ Wde
        yp[rows] = ype
        dyt = dY[row_t[rows]]
        dyp = row_w[rows, None] * dyt
        dwr = np.sum(ype * dyt, axis=1)
        for q, r in enumerate(rows):
            t = row_t[r]
            j = int(np.nonzero(s2r[t] == r)[0][0])
            dW[t, j] = dwr[q]
        da = dyp @ Wde.T
        du = da * g * sg
        dg = da * u * sg * (1.0 + g * (1.0 - sg))
        tok = rt[rows]
        mine = tsel[tok]
        np.add.at(dX, tok[mine], (dg @ Wge.T + du @ Wue.T)[mine])
        if e in slot:
            dWd[slot[e]] = a.T @ dyp
            dWg[slot[e]] = xe.T @ dg
            dWu[slot[e]] = xe.T @ du

    # router: d logits from d w (dropped slots carry no gradient: dW is 0 there)
    dW[~tsel] = 0.0
    L = np.asarray(logits, np.float64)
    wf = w.astype(np.float64)
    dL = np.zeros((T, E))
    inner = np.sum(wf * dW, axis=1)
    if renormalize:
        for j in range(k):
            dL[np.arange(T), ids[:, j]] += wf[:, j] * (dW[:, j] - inner)
    else:
        m = L.max(axis=1, keepdims=True)
        p = np.exp(L - m)
        p /= p.sum(axis=1, keepdims=True)
        dsel = np.zeros((T, E))
        dsel[np.arange(T)[:, None], ids] = dW
        dL = p * (dsel - inner[:, None])
    out = dict(dx=dX, dw_gate=dWg, dw_up=dWu, dw_down=dWd, dlogits=dL, dtopk_w=dW, yp=yp,
               topk_ids=ids, topk_w=w, keep=keep, **lay)
    if w_router is not None:
        Wr = _f64(np.asarray(w_router))
        out["dw_router"] = dL.T @ X
        out["dx"] = dX + dL @ Wr
    return out
