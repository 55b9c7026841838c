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


def combine(tokens: np.ndarray, topk_w: np.ndarray, slot_to_row: np.ndarray, yp: np.ndarray) -> np.ndarray:
    """y[i] = sum over kept slots j of token tokens[i]: w[t,j] * yp[slot_to_row[t,j]], fp64."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    s2r = np.ascontiguousarray(slot_to_row, dtype=np.int32)
    yp = np.ascontiguousarray(yp, dtype=np.float64)
    T, k = topk_w.shape
    H = yp.shape[1]
    y = np.zeros((tokens.size, H), np.float64)
    _load().orc_combine(tokens.size, _p(tokens), H, k, _p(topk_w), _p(s2r), _p(yp), _p(y))
    return y


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
