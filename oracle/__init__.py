"""CPU oracle for the MoE layer hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the cpu_baseline leg of bench.py may
import this package.  The product path (expert_ffn_moe_amd) never does: it runs the HIP
library or fails.

Every function wraps one function of moe_oracle.c (plain C, built without fast-math or
fp contraction) and works on host numpy arrays.  bf16 data travels as uint16 bit
patterns.  The passage each step follows is cited in moe_oracle.c.

Parity status: every function is pinned by tests/test_oracle_*.py (brute force on tiny
inputs, closed forms, special cases and invariants).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32 = 0
BF16 = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b

        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.orc_exp.restype = ctypes.c_float
    lib.orc_exp.argtypes = [ctypes.c_float]
    lib.orc_exp_max_ulp.restype = ctypes.c_double
    lib.orc_exp_max_ulp.argtypes = [ctypes.c_float, ctypes.c_float, P]
    lib.orc_exp_vec.restype = None
    lib.orc_exp_vec.argtypes = [ctypes.c_int64, P, P]
    lib.orc_route.restype = None
    lib.orc_route.argtypes = [i32, i32, i32, i32, P, P, P]
    lib.orc_capacity.restype = None
    lib.orc_capacity.argtypes = [i32, i32, i32, i32, P, P, P]
    lib.orc_layout.restype = i32
    lib.orc_layout.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    lib.orc_gather.restype = None
    lib.orc_gather.argtypes = [i32, i32, i32, P, P, P]
    lib.orc_ffn_rows.restype = None
    lib.orc_ffn_rows.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32]
    lib.orc_combine.restype = None
    lib.orc_combine.argtypes = [i32, P, i32, i32, P, P, P, P]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [i32]
    lib.orc_e4m3_encode.restype = i32
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_ue8m0.restype = i32
    lib.orc_ue8m0.argtypes = [ctypes.c_double]
    for name in ("orc_e4m3_encode_vec", "orc_e4m3_value_vec", "orc_ue8m0_vec"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [ctypes.c_int64, P, P]
    lib.orc_quant_rows.restype = None
    lib.orc_quant_rows.argtypes = [ctypes.c_int64, i32, i32, P, P, P]
    lib.orc_route_grouped.restype = None
    lib.orc_route_grouped.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P]
    lib.orc_router_logits.restype = None
    lib.orc_router_logits.argtypes = [i32, i32, i32, i32, P, P, P]
    lib.orc_ffn_rows_fp8.restype = None
    lib.orc_ffn_rows_fp8.argtypes = [i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, i32]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


def exp32(x) -> np.ndarray:
    """The specified fp32 exponential, element-wise."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    y = np.empty_like(x)
    _load().orc_exp_vec(x.size, _p(x), _p(y))
    return y


def exp_max_ulp(lo: float, hi: float):
    """(max ulp error vs fp64 exp, worst x) over every fp32 in [lo, hi]."""
    wx = ctypes.c_float(0.0)
    err = _load().orc_exp_max_ulp(lo, hi, ctypes.byref(wx))
    return err, wx.value


def route(logits: np.ndarray, k: int, renormalize: int = 1):
    """Top-k ids [T,k] int32 (slot order: logit desc, ties to lower id) and weights [T,k] f32."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not (1 <= k <= min(E, 64)):
        raise ValueError("need 1 <= k <= min(E, 64)")
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().orc_route(T, E, k, int(renormalize), _p(logits), _p(ids), _p(w))
    return ids, w


def route_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int,
                  renormalize: int = 1):
    """Group-limited top-k (groups of E / n_group consecutive experts, group score = its
    largest logit, the topk_group best groups, then top-k inside them): ids, weights."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if n_group < 1 or E % n_group or not (1 <= topk_group <= n_group):
        raise ValueError("need E % n_group == 0 and 1 <= topk_group <= n_group")
    if not (1 <= k <= min(topk_group * (E // n_group), 64)):
        raise ValueError("need 1 <= k <= min(topk_group * E / n_group, 64)")
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().orc_route_grouped(T, E, k, int(renormalize), n_group, topk_group, _p(logits),
                              _p(ids), _p(w))
    return ids, w


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits [T, E] f64 = x [T, H] times W_r [E, H] transposed (f32, or bf16 as uint16)."""
    x = np.ascontiguousarray(x)
    w_router = np.ascontiguousarray(w_router)
    assert x.dtype == w_router.dtype and x.shape[1] == w_router.shape[1]
    T, H = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), np.float64)
    _load().orc_router_logits(T, H, E, _dtype_code(x), _p(x), _p(w_router), _p(out))
    return out


def capacity(ids: np.ndarray, w: np.ndarray, E: int, C: int) -> np.ndarray:
    """keep [T,k] uint8: 0 for the lowest-weight excess assignments of each expert over C."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = ids.shape
    keep = np.empty((T, k), np.uint8)
    _load().orc_capacity(T, E, k, int(C), _p(ids), _p(w), _p(keep))
    return keep


def layout(ids: np.ndarray, keep: Optional[np.ndarray], E: int):
    """Expert-contiguous layout: dict(counts, offsets, row_token, slot_to_row, N)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_token = np.full(T * k, -1, np.int32)
    slot_to_row = np.empty((T, k), np.int32)
    kp = None
    if keep is not None:
        kp = np.ascontiguousarray(keep, dtype=np.uint8)
    n = _load().orc_layout(T, E, k, _p(ids), _p(kp) if kp is not None else None, _p(counts),
                           _p(offsets), _p(row_token), _p(slot_to_row))
    return dict(counts=counts, offsets=offsets, row_token=row_token, slot_to_row=slot_to_row, N=int(n))


def gather(x: np.ndarray, row_token: np.ndarray, N: int) -> np.ndarray:
    """xp[r] = x[row_token[r]] for r < N (byte copy)."""
    x = np.ascontiguousarray(x)
    rt = np.ascontiguousarray(row_token[:N], dtype=np.int32)
    xp = np.empty((N,) + x.shape[1:], x.dtype)
    _load().orc_gather(N, x.shape[1], x.dtype.itemsize, _p(x), _p(rt), _p(xp))
    return xp


def ffn_rows(xrows: np.ndarray, row_expert: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
             w_down: np.ndarray, want_a: bool = False, nthreads: int = 0):
    """SwiGLU expert FFN per row in fp64.  Returns yp [n,H] f64 (and a [n,I] f64)."""
    xrows = np.ascontiguousarray(xrows)
    row_expert = np.ascontiguousarray(row_expert, dtype=np.int32)
    w_gate = np.ascontiguousarray(w_gate)
    w_up = np.ascontiguousarray(w_up)
    w_down = np.ascontiguousarray(w_down)
    n, H = xrows.shape
    Ew, H2, I = w_gate.shape
    assert H2 == H and w_up.shape == w_gate.shape and w_down.shape == (Ew, I, H)
    if n:
        assert 0 <= row_expert.min() and row_expert.max() < Ew
    xd, wd = _dtype_code(xrows), _dtype_code(w_gate)
    assert _dtype_code(w_up) == wd and _dtype_code(w_down) == wd
    yp = np.zeros((n, H), np.float64)
    a = np.zeros((n, I), np.float64) if want_a else None
    if n:
        _load().orc_ffn_rows(H, I, xd, wd, n, _p(row_expert), _p(xrows), _p(w_gate), _p(w_up),
                             _p(w_down), _p(yp), _p(a) if a is not None else None, int(nthreads))
    return (yp, a) if want_a else yp


def combine(tokens: np.ndarray, topk_w: np.ndarray, slot_to_row: np.ndarray, yp: np.ndarray,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """y[i] = sum over kept slots j of token tokens[i]: w[t,j] * yp[slot_to_row[t,j]], fp64;
    plus shared[i] (the shared expert's output for that token, [LightLLM] PR body: the
    combine adds the shared expert's output) if given."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    yp = np.ascontiguousarray(yp, dtype=np.float64)
    T, k = topk_w.shape
    H = yp.shape[1]
    y = np.zeros((tokens.size, H), np.float64)
    _load().orc_combine(tokens.size, _p(tokens), H, k, _p(topk_w), _p(s2r), _p(yp), _p(y))
    if shared is not None:
        y = y + np.asarray(shared, dtype=np.float64)
    return y


def shared_expert(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
                  nthreads: int = 0) -> np.ndarray:
    """The shared expert: the SwiGLU MLP of one expert ([1, H, Is] / [1, Is, H] weights)
    applied to every row of x, fp64 (ffn_rows with every row on expert 0)."""
    rows = np.zeros(x.shape[0], np.int32)
    return ffn_rows(x, rows, w_gate, w_up, w_down, nthreads=nthreads)


def layer(x: np.ndarray, logits: np.ndarray, w_gate, w_up, w_down, k: int, capacity_: int = 0,
          renormalize: int = 1, nthreads: int = 0):
    """The whole path on the CPU: route -> capacity -> layout -> gather -> FFN -> combine."""
    T, E = logits.shape
    ids, w = route(logits, k, renormalize)
    keep = capacity(ids, w, E, capacity_)
    lay = layout(ids, keep, E)
    N = lay["N"]
    xp = gather(x, lay["row_token"], N)
    row_expert = np.repeat(np.arange(E, dtype=np.int32), lay["counts"])
    yp, a = ffn_rows(xp, row_expert, w_gate, w_up, w_down, want_a=True, nthreads=nthreads)
    y = combine(np.arange(T, dtype=np.int32), w, lay["slot_to_row"], yp)
    return dict(topk_ids=ids, topk_w=w, keep=keep, xp=xp, a=a, yp=yp, y=y, **lay)


# ---------------------------------------------------------------------------------------
# FP8 (E4M3 codes with UE8M0 power-of-two block scales, blocks of 32 along the reduction
# dimension; the readings are recorded in moe_oracle.c)
# ---------------------------------------------------------------------------------------
QBLOCK = 32


def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 code (NaN for 0x7F / 0xFF), fp64."""
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8).ravel())
    out = np.empty(codes.size, np.float64)
    _load().orc_e4m3_value_vec(codes.size, _p(codes), _p(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    """Nearest E4M3 code of each value (|v| <= 448), ties to even, sign kept at zero."""
    vals = np.ascontiguousarray(np.asarray(values, dtype=np.float64).ravel())
    out = np.empty(vals.size, np.uint8)
    _load().orc_e4m3_encode_vec(vals.size, _p(vals), _p(out))
    return out


def ue8m0(amax) -> np.ndarray:
    """E8M0 scale byte 127 + e, e the smallest integer with amax <= 448 * 2^e."""
    vals = np.ascontiguousarray(np.asarray(amax, dtype=np.float64).ravel())
    out = np.empty(vals.size, np.uint8)
    _load().orc_ue8m0_vec(vals.size, _p(vals), _p(out))
    return out


def quant_rows(x: np.ndarray):
    """Quantise each row of x [n, m] (m % 32 == 0; f32, bf16-as-uint16 or f64) in blocks of
    32: returns (codes [n, m] uint8, scales [n, m / 32] uint8)."""
    x = np.ascontiguousarray(x)
    n, m = x.shape
    assert m % QBLOCK == 0
    code = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}[x.dtype]
    codes = np.empty((n, m), np.uint8)
    scales = np.empty((n, m // QBLOCK), np.uint8)
    _load().orc_quant_rows(n, m, code, _p(x), _p(codes), _p(scales))
    return codes, scales


def quant_weights(w: np.ndarray):
    """Quantise expert weights w [E, K, N] (K the reduction dimension) in blocks of 32 along
    K: returns (codes [E, K, N], scales [E, K / 32, N])."""
    E, K, N = w.shape
    wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1))).reshape(E * N, K)
    c, s = quant_rows(wt)
    codes = np.ascontiguousarray(np.transpose(c.reshape(E, N, K), (0, 2, 1)))
    scales = np.ascontiguousarray(np.transpose(s.reshape(E, N, K // QBLOCK), (0, 2, 1)))
    return codes, scales


def dequant(codes: np.ndarray, scales: np.ndarray, axis: int) -> np.ndarray:
    """codes * 2^(scale - 127), the scale of element i along `axis` being scales[i // 32]."""
    v = e4m3_value(codes).reshape(codes.shape)
    s = np.repeat(scales.astype(np.int64) - 127, QBLOCK, axis=axis)
    return np.ldexp(v, s)


def ffn_rows_fp8(xq, xs, row_expert, wg, wu, wd, want_a: bool = False, nthreads: int = 0):
    """FP8 SwiGLU FFN per row.  xq/xs: quantised rows; wg, wu, wd: (codes, scales) pairs from
    quant_weights of W_gate, W_up [E,H,I] and W_down [E,I,H].  g, u and yp accumulate in
    fp64; a is quantised per row (blocks of 32) before the down projection.  Returns yp
    [n,H] f64, and with want_a (a before quantisation f64, a codes, a scales)."""
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    xs = np.ascontiguousarray(xs, dtype=np.uint8)
    row_expert = np.ascontiguousarray(row_expert, dtype=np.int32)
    (gq, gs), (uq, us), (dq, ds) = [(np.ascontiguousarray(c), np.ascontiguousarray(s))
                                    for c, s in (wg, wu, wd)]
    n, H = xq.shape
    E, H2, I = gq.shape
    assert H2 == H and dq.shape == (E, I, H) and xs.shape == (n, H // QBLOCK)
    yp = np.zeros((n, H), np.float64)
    a = np.zeros((n, I), np.float64)
    ac = np.zeros((n, I), np.uint8)
    asc = np.zeros((n, I // QBLOCK), np.uint8)
    if n:
        _load().orc_ffn_rows_fp8(H, I, n, _p(row_expert), _p(xq), _p(xs), _p(gq), _p(gs), _p(uq),
                                 _p(us), _p(dq), _p(ds), _p(yp), _p(a), _p(ac), _p(asc),
                                 int(nthreads))
    return (yp, a, ac, asc) if want_a else yp
