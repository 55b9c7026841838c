"""Python binding of libmoe, the MI355X (gfx950) MoE-layer hot path.

Argument marshalling only: every function checks shapes/dtypes/devices of torch tensors,
allocates outputs with torch (device memory and streams are all torch is used for) and
calls the C ABI declared in include/moe.h on torch's current HIP stream.  All compute runs
in the library's HIP kernels; if libmoe.so is missing or fails to load, importing this
package raises -- there is no other implementation.

Call names follow the C ABI: route, dispatch, expert_gate_up, expert_gate_up_gather,
expert_down, expert_ffn, combine, layer, quantize_fp8, plus pack_weights for the one-time
weight packing.

Problem.dtype "fp8" means FP8 (E4M3, UE8M0 block scales) expert weights with bf16
activations: pack_weights then takes bf16 weights and quantises them, and the intermediate
activation `a` is a uint8 buffer of E4M3 codes followed by scale bytes (split_quantized).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8 = 0, 1, 2
QBLOCK = 32  # elements per UE8M0 scale
OP_ROUTE, OP_DISPATCH, OP_FFN, OP_COMBINE, OP_LAYER, OP_ROUTER, OP_BACKWARD = range(7)
W_GATE_UP, W_DOWN = 0, 1

EXPORTS = ("moe_status_str", "moe_problem_check", "moe_workspace_bytes", "moe_packed_bytes",
           "moe_pack_weights", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_gate_up",
           "moe_expert_gate_up_gather",
           "moe_expert_down", "moe_combine", "moe_layer", "moe_quantize_fp8",
           "moe_route_grouped", "moe_router", "moe_layer_chunked_workspace_bytes",
           "moe_layer_chunked", "moe_pack_weights_backward", "moe_expert_gate_up_gather_gu",
           "moe_layer_backward", "moe_debug_status", "moe_layer_static",
           "moe_layer_static_max_bytes")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")


class MoeSharedExpert(ctypes.Structure):
    _fields_ = [("I", ctypes.c_int32), ("packed_gate_up", ctypes.c_void_p),
                ("packed_down", ctypes.c_void_p)]


class MoeSavedRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_ids", "topk_w", "offsets", "row_token", "slot_to_row")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_gate", "dw_up", "dw_down", "dlogits", "dtopk_w", "dw_router")]


class MoeProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "k", "I", "capacity", "renormalize", "act_dtype", "w_dtype")]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python expert_ffn_moe_amd/build.py` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(MoeProblem)
    sz = ctypes.c_size_t
    sigs = {
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_problem_check": (ctypes.c_int, [PP]),
        "moe_workspace_bytes": (sz, [PP, ctypes.c_int]),
        "moe_packed_bytes": (sz, [PP, ctypes.c_int]),
        "moe_pack_weights": (ctypes.c_int, [PP, P, P, P, P, P, P]),
        "moe_route": (ctypes.c_int, [PP, P, P, P, P, P, sz, P]),
        "moe_dispatch": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, sz, P]),
        "moe_expert_ffn": (ctypes.c_int, [PP, P, P, P, P, P, P, sz, P]),
        "moe_expert_gate_up": (ctypes.c_int, [PP, P, P, P, P, P, sz, P]),
        "moe_expert_gate_up_gather": (ctypes.c_int, [PP, P, P, P, P, P, P, sz, P]),
        "moe_expert_down": (ctypes.c_int, [PP, P, P, P, P, P, sz, P]),
        "moe_combine": (ctypes.c_int, [PP, P, P, P, P, P]),
        "moe_layer": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "moe_quantize_fp8": (ctypes.c_int, [P, ctypes.c_int64, ctypes.c_int32, P, P, P]),
        "moe_route_grouped": (ctypes.c_int, [PP, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P,
                                             sz, P]),
        "moe_router": (ctypes.c_int, [PP, P, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P,
                                      sz, P]),
        "moe_layer_chunked_workspace_bytes": (sz, [PP, ctypes.c_int32, ctypes.c_int32]),
        "moe_pack_weights_backward": (ctypes.c_int, [PP, P, P, P, P, P, P]),
        "moe_expert_gate_up_gather_gu": (ctypes.c_int, [PP, P, P, P, P, P, P, P]),
        "moe_layer_backward": (ctypes.c_int, [PP, P, P, P, P, P, P, P,
                                              ctypes.POINTER(MoeSavedRouting), P, P, P,
                                              ctypes.POINTER(MoeGrads), P, sz, P]),
        "moe_layer_chunked": (ctypes.c_int, [PP, P, P, P, P, ctypes.POINTER(MoeSharedExpert),
                                             ctypes.c_int32, P, P, sz, P, P]),
        "moe_debug_status": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32)]),
        "moe_layer_static": (ctypes.c_int, [PP, P, P, P, P, P, P, P, P, P, P, P, P, P]),
        "moe_layer_static_max_bytes": (ctypes.c_size_t, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
LIB_DEBUG_PATH = os.path.join(_HERE, "libmoe_debug.so")
_debug_lib = None


def debug_lib() -> ctypes.CDLL:
    """The debug build of the library (device-side precondition checks, moe_debug_status),
    loaded on first use; same entry points and signatures as `lib`."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(LIB_DEBUG_PATH)
    return _debug_lib


def debug_status(dlib=None) -> int:
    """moe_debug_status of the debug library: the precondition-check bits since the last
    read (waits for the device)."""
    v = ctypes.c_uint32(0)
    _call_on(dlib or debug_lib(), "moe_debug_status", ctypes.byref(v))
    return int(v.value)


def status_str(status: int) -> str:
    return lib.moe_status_str(int(status)).decode()


@dataclasses.dataclass(frozen=True)
class Problem:
    """Shapes of one layer call (see moe_problem in include/moe.h)."""
    T: int
    H: int
    E: int
    k: int
    I: int
    capacity: int = 0
    renormalize: int = 1
    dtype: str = "bf16"  # "bf16" or "f32" (activations and weights), "fp8" (FP8 weights)

    @property
    def torch_dtype(self) -> torch.dtype:
        """Activation dtype."""
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def fp8(self) -> bool:
        return self.dtype == "fp8"

    def c(self) -> MoeProblem:
        act = MOE_F32 if self.dtype == "f32" else MOE_BF16
        w = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8}.get(self.dtype, -1)
        return MoeProblem(self.T, self.H, self.E, self.k, self.I, self.capacity, self.renormalize,
                          act, w)

    def a_shape(self):
        """Shape and dtype of the intermediate activation buffer `a`."""
        tk = self.T * self.k
        if self.fp8:
            return (_align256(tk * self.I) + tk * (self.I // QBLOCK),), torch.uint8
        return (tk, self.I), self.torch_dtype

    def check(self) -> int:
        c = self.c()
        return lib.moe_problem_check(ctypes.byref(c))

    def workspace_bytes(self, op: int) -> int:
        c = self.c()
        return int(lib.moe_workspace_bytes(ctypes.byref(c), op))

    def packed_bytes(self, which: int) -> int:
        c = self.c()
        return int(lib.moe_packed_bytes(ctypes.byref(c), which))

    @classmethod
    def of(cls, wl) -> "Problem":
        """From a workload description with T, H, E, k, I, capacity, renormalize, dtype."""
        return cls(wl.T, wl.H, wl.E, wl.k, wl.I, wl.capacity, wl.renormalize, wl.dtype)


def _align256(n: int) -> int:
    return (n + 255) & ~255


def split_quantized(p: Problem, a: torch.Tensor):
    """Views of an FP8 intermediate buffer: (codes [T*k, I] u8, scales [T*k, I/32] u8)."""
    tk = p.T * p.k
    off = _align256(tk * p.I)
    return a[:tk * p.I].view(tk, p.I), a[off:off + tk * (p.I // QBLOCK)].view(tk, p.I // QBLOCK)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _call(name: str, *args):
    _call_on(lib, name, *args)


def _call_on(which: ctypes.CDLL, name: str, *args):
    st = getattr(which, name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def workspace(p: Problem, op: int, device="cuda") -> torch.Tensor:
    """A workspace buffer for `op` (torch's allocator returns 256-byte aligned blocks)."""
    return torch.empty(max(p.workspace_bytes(op), 256), dtype=torch.uint8, device=device)


def pack_weights(p: Problem, w_gate, w_up, w_down, packed_gate_up=None, packed_down=None):
    """One-time packing of [E,H,I], [E,H,I], [E,I,H] weights into the kernels' layout
    (fp8 problems: bf16 weights, quantised while packing)."""
    dt = p.torch_dtype
    _need(w_gate, "w_gate", (p.E, p.H, p.I), dt)
    _need(w_up, "w_up", (p.E, p.H, p.I), dt)
    _need(w_down, "w_down", (p.E, p.I, p.H), dt)
    dev = w_gate.device
    if packed_gate_up is None:
        packed_gate_up = _empty((p.packed_bytes(W_GATE_UP),), torch.uint8, dev)
    if packed_down is None:
        packed_down = _empty((p.packed_bytes(W_DOWN),), torch.uint8, dev)
    c = p.c()
    _call("moe_pack_weights", ctypes.byref(c), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
          _ptr(packed_gate_up), _ptr(packed_down), _stream())
    return packed_gate_up, packed_down


def route(p: Problem, logits, out=None, ws=None):
    """Top-k + capacity: returns (topk_ids [T,k] i32, topk_w [T,k] f32, keep [T,k] u8)."""
    _need(logits, "logits", (p.T, p.E), torch.float32)
    dev = logits.device
    ids, w, keep = out if out is not None else (
        _empty((p.T, p.k), torch.int32, dev), _empty((p.T, p.k), torch.float32, dev),
        _empty((p.T, p.k), torch.uint8, dev))
    ws = workspace(p, OP_ROUTE, dev) if ws is None else ws
    c = p.c()
    _call("moe_route", ctypes.byref(c), _ptr(logits), _ptr(ids), _ptr(w), _ptr(keep), _ptr(ws),
          ws.numel(), _stream())
    return ids, w, keep


def route_grouped(p: Problem, logits, n_group: int, topk_group: int, out=None, ws=None):
    """Group-limited top-k + capacity: returns (topk_ids, topk_w, keep) as route()."""
    _need(logits, "logits", (p.T, p.E), torch.float32)
    dev = logits.device
    ids, w, keep = out if out is not None else (
        _empty((p.T, p.k), torch.int32, dev), _empty((p.T, p.k), torch.float32, dev),
        _empty((p.T, p.k), torch.uint8, dev))
    ws = workspace(p, OP_ROUTE, dev) if ws is None else ws
    c = p.c()
    _call("moe_route_grouped", ctypes.byref(c), _ptr(logits), ctypes.c_int32(n_group),
          ctypes.c_int32(topk_group), _ptr(ids), _ptr(w), _ptr(keep), _ptr(ws), ws.numel(),
          _stream())
    return ids, w, keep


def router(p: Problem, x, w_router, n_group: int = 1, topk_group: int = 1, logits=None,
           want_logits: bool = False, out=None, ws=None):
    """Router GEMM (logits = x W_r^T, W_r [E, H]) + (grouped) top-k + capacity.  Returns
    (topk_ids, topk_w, keep, logits) -- logits None unless asked for (or passed in)."""
    _need(x, "x", (p.T, p.H), torch.bfloat16)
    _need(w_router, "w_router", (p.E, p.H), torch.bfloat16)
    dev = x.device
    if logits is None and want_logits:
        logits = _empty((p.T, p.E), torch.float32, dev)
    if logits is not None:
        _need(logits, "logits", (p.T, p.E), torch.float32)
    ids, w, keep = out if out is not None else (
        _empty((p.T, p.k), torch.int32, dev), _empty((p.T, p.k), torch.float32, dev),
        _empty((p.T, p.k), torch.uint8, dev))
    ws = workspace(p, OP_ROUTER, dev) if ws is None else ws
    c = p.c()
    _call("moe_router", ctypes.byref(c), _ptr(x), _ptr(w_router), ctypes.c_int32(n_group),
          ctypes.c_int32(topk_group), _ptr(logits), _ptr(ids), _ptr(w), _ptr(keep), _ptr(ws),
          ws.numel(), _stream())
    return ids, w, keep, logits


def dispatch(p: Problem, x, topk_ids, keep=None, out=None, ws=None, rows=True):
    """Expert-contiguous layout + row gather (rows=False: the layout only, xp is None).
    Returns dict(counts, offsets, row_token, slot_to_row, xp)."""
    dt = p.torch_dtype
    _need(x, "x", (p.T, p.H), dt)
    _need(topk_ids, "topk_ids", (p.T, p.k), torch.int32)
    if keep is not None:
        _need(keep, "keep", (p.T, p.k), torch.uint8)
    dev = x.device
    tk = p.T * p.k
    if out is None:
        out = dict(counts=_empty((p.E,), torch.int32, dev), offsets=_empty((p.E + 1,), torch.int32, dev),
                   row_token=_empty((tk,), torch.int32, dev),
                   slot_to_row=_empty((p.T, p.k), torch.int32, dev),
                   xp=_empty((tk, p.H), dt, dev) if rows else None)
    elif not rows:
        out = dict(out, xp=None)
    ws = workspace(p, OP_DISPATCH, dev) if ws is None else ws
    c = p.c()
    _call("moe_dispatch", ctypes.byref(c), _ptr(x), _ptr(topk_ids), _ptr(keep), _ptr(out["counts"]),
          _ptr(out["offsets"]), _ptr(out["row_token"]), _ptr(out["slot_to_row"]), _ptr(out["xp"]),
          _ptr(ws), ws.numel(), _stream())
    return out


def expert_gate_up(p: Problem, xp, offsets, packed_gate_up, out=None, ws=None):
    """a = silu(xp Wg) * (xp Wu) per expert segment; returns a [T*k, I]."""
    dt = p.torch_dtype
    tk = p.T * p.k
    _need(xp, "xp", (tk, p.H), dt)
    _need(offsets, "offsets", (p.E + 1,), torch.int32)
    a = _empty(*p.a_shape(), xp.device) if out is None else out
    _need(a, "a", *p.a_shape())
    ws = workspace(p, OP_FFN, xp.device) if ws is None else ws
    c = p.c()
    _call("moe_expert_gate_up", ctypes.byref(c), _ptr(xp), _ptr(offsets), _ptr(packed_gate_up),
          _ptr(a), _ptr(ws), ws.numel(), _stream())
    return a


def expert_gate_up_gather(p: Problem, x, row_token, offsets, packed_gate_up, out=None, ws=None):
    """expert_gate_up with the rows read as x[row_token[r]] (no xp); returns a [T*k, I]."""
    dt = p.torch_dtype
    tk = p.T * p.k
    _need(x, "x", (p.T, p.H), dt)
    _need(row_token, "row_token", (tk,), torch.int32)
    _need(offsets, "offsets", (p.E + 1,), torch.int32)
    a = _empty(*p.a_shape(), x.device) if out is None else out
    _need(a, "a", *p.a_shape())
    if ws is None and p.fp8:
        ws = workspace(p, OP_FFN, x.device)
    c = p.c()
    _call("moe_expert_gate_up_gather", ctypes.byref(c), _ptr(x), _ptr(row_token), _ptr(offsets),
          _ptr(packed_gate_up), _ptr(a), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    return a


def expert_down(p: Problem, a, offsets, packed_down, out=None, ws=None):
    """yp = a Wd per expert segment; returns yp [T*k, H]."""
    dt = p.torch_dtype
    tk = p.T * p.k
    _need(a, "a", *p.a_shape())
    _need(offsets, "offsets", (p.E + 1,), torch.int32)
    yp = _empty((tk, p.H), dt, a.device) if out is None else out
    ws = workspace(p, OP_FFN, a.device) if ws is None else ws
    c = p.c()
    _call("moe_expert_down", ctypes.byref(c), _ptr(a), _ptr(offsets), _ptr(packed_down), _ptr(yp),
          _ptr(ws), ws.numel(), _stream())
    return yp


def expert_ffn(p: Problem, xp, offsets, packed_gate_up, packed_down, out=None, ws=None):
    """Grouped SwiGLU FFN; returns yp [T*k, H]."""
    dt = p.torch_dtype
    tk = p.T * p.k
    _need(xp, "xp", (tk, p.H), dt)
    _need(offsets, "offsets", (p.E + 1,), torch.int32)
    yp = _empty((tk, p.H), dt, xp.device) if out is None else out
    ws = workspace(p, OP_FFN, xp.device) if ws is None else ws
    c = p.c()
    _call("moe_expert_ffn", ctypes.byref(c), _ptr(xp), _ptr(offsets), _ptr(packed_gate_up),
          _ptr(packed_down), _ptr(yp), _ptr(ws), ws.numel(), _stream())
    return yp


def combine(p: Problem, yp, topk_w, slot_to_row, out=None):
    """y[t] = sum of kept w[t,j] * yp[slot_to_row[t,j]] in slot order; returns y [T, H]."""
    dt = p.torch_dtype
    _need(yp, "yp", (p.T * p.k, p.H), dt)
    _need(topk_w, "topk_w", (p.T, p.k), torch.float32)
    _need(slot_to_row, "slot_to_row", (p.T, p.k), torch.int32)
    y = _empty((p.T, p.H), dt, yp.device) if out is None else out
    c = p.c()
    _call("moe_combine", ctypes.byref(c), _ptr(yp), _ptr(topk_w), _ptr(slot_to_row), _ptr(y),
          _stream())
    return y


def layer(p: Problem, x, logits, packed_gate_up, packed_down, out=None, routing=None, ws=None):
    """The whole layer.  `routing` may be a dict of preallocated buffers (topk_ids, topk_w,
    keep, counts, offsets, row_token, slot_to_row) that receive the routing results."""
    dt = p.torch_dtype
    _need(x, "x", (p.T, p.H), dt)
    _need(logits, "logits", (p.T, p.E), torch.float32)
    y = _empty((p.T, p.H), dt, x.device) if out is None else out
    r = routing or {}
    ws = workspace(p, OP_LAYER, x.device) if ws is None else ws
    c = p.c()
    _call("moe_layer", ctypes.byref(c), _ptr(x), _ptr(logits), _ptr(packed_gate_up), _ptr(packed_down),
          _ptr(y), _ptr(r.get("topk_ids")), _ptr(r.get("topk_w")), _ptr(r.get("keep")),
          _ptr(r.get("counts")), _ptr(r.get("offsets")), _ptr(r.get("row_token")),
          _ptr(r.get("slot_to_row")), _ptr(ws), ws.numel(), _stream())
    return y


def quantize_fp8(x, codes=None, scales=None):
    """Per-row FP8 quantisation of bf16 x [rows, cols] (cols a multiple of 32): returns
    (codes [rows, cols] u8 E4M3, scales [rows, cols/32] u8 UE8M0)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    _need(x, "x", (rows, cols), torch.bfloat16)
    codes = _empty((rows, cols), torch.uint8, x.device) if codes is None else codes
    scales = _empty((rows, cols // QBLOCK), torch.uint8, x.device) if scales is None else scales
    _need(codes, "codes", (rows, cols), torch.uint8)
    _need(scales, "scales", (rows, cols // QBLOCK), torch.uint8)
    _call("moe_quantize_fp8", _ptr(x), ctypes.c_int64(rows), ctypes.c_int32(cols), _ptr(codes),
          _ptr(scales), _stream())
    return codes, scales


def shared_problem(p: Problem, I: int) -> Problem:
    """The one-expert problem whose packed weights a shared expert of width I uses."""
    return dataclasses.replace(p, E=1, k=1, I=I, capacity=0)


def layer_chunked(p: Problem, x, logits, packed_gate_up, packed_down, chunk_tokens: int,
                  shared=None, aux_stream=None, out=None, ws=None):
    """The layer over chunks of tokens (see moe_layer_chunked).  shared: None or
    (I, packed_gate_up, packed_down) of the shared expert; aux_stream: a torch stream for
    the layouts (and the shared expert), or None."""
    dt = p.torch_dtype
    _need(x, "x", (p.T, p.H), dt)
    _need(logits, "logits", (p.T, p.E), torch.float32)
    y = _empty((p.T, p.H), dt, x.device) if out is None else out
    sI = 0 if shared is None else int(shared[0])
    c = p.c()
    need = int(lib.moe_layer_chunked_workspace_bytes(ctypes.byref(c), int(chunk_tokens), sI))
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    sh = None
    if shared is not None:
        sh = MoeSharedExpert(sI, shared[1].data_ptr(), shared[2].data_ptr())
    aux = None if aux_stream is None else ctypes.c_void_p(aux_stream.cuda_stream)
    _call("moe_layer_chunked", ctypes.byref(c), _ptr(x), _ptr(logits), _ptr(packed_gate_up),
          _ptr(packed_down), None if sh is None else ctypes.byref(sh), int(chunk_tokens), _ptr(y),
          _ptr(ws), ws.numel(), _stream(), aux)
    return y


def pack_weights_backward(p: Problem, w_gate, w_up, w_down):
    """One-time packing of the backward operands ([W_gate | W_up]^T, W_down^T) from the
    natural bf16 weights; returns (packed_bwd_gate_up, packed_bwd_down)."""
    _need(w_gate, "w_gate", (p.E, p.H, p.I), torch.bfloat16)
    _need(w_up, "w_up", (p.E, p.H, p.I), torch.bfloat16)
    _need(w_down, "w_down", (p.E, p.I, p.H), torch.bfloat16)
    dev = w_gate.device
    pgu = _empty((p.packed_bytes(W_GATE_UP),), torch.uint8, dev)
    pd = _empty((p.packed_bytes(W_DOWN),), torch.uint8, dev)
    c = p.c()
    _call("moe_pack_weights_backward", ctypes.byref(c), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
          _ptr(pgu), _ptr(pd), _stream())
    return pgu, pd


def expert_gate_up_gather_gu(p: Problem, x, row_token, offsets, packed_gate_up, out=None,
                             gu=None):
    """expert_gate_up_gather (bf16) that also stores the pre-activations g|u for the
    backward; returns (a [T*k, I], gu [T*k, 2I])."""
    tk = p.T * p.k
    _need(x, "x", (p.T, p.H), torch.bfloat16)
    _need(row_token, "row_token", (tk,), torch.int32)
    _need(offsets, "offsets", (p.E + 1,), torch.int32)
    a = _empty((tk, p.I), torch.bfloat16, x.device) if out is None else out
    _need(a, "a", (tk, p.I), torch.bfloat16)
    gu = _empty((tk, 2 * p.I), torch.bfloat16, x.device) if gu is None else gu
    _need(gu, "gu", (tk, 2 * p.I), torch.bfloat16)
    c = p.c()
    _call("moe_expert_gate_up_gather_gu", ctypes.byref(c), _ptr(x), _ptr(row_token),
          _ptr(offsets), _ptr(packed_gate_up), _ptr(a), _ptr(gu), _stream())
    return a, gu


def layer_backward(p: Problem, x, logits, packed_gate_up, packed_down, packed_bwd_gate_up,
                   packed_bwd_down, routing, dy, yp=None, w_router=None, ws=None, gu=None):
    """Gradients of the layer (see moe_layer_backward).  routing: the forward's topk_ids,
    topk_w, offsets, row_token, slot_to_row (a dict); yp: the forward's expert outputs or
    None (recomputed); gu: the forward's pre-activations (expert_gate_up_gather_gu) or None
    (recomputed).  Returns dict(dx, dw_gate, dw_up, dw_down, dlogits, dtopk_w[,
    dw_router])."""
    _need(x, "x", (p.T, p.H), torch.bfloat16)
    _need(dy, "dy", (p.T, p.H), torch.bfloat16)
    if yp is not None:
        _need(yp, "yp", (p.T * p.k, p.H), torch.bfloat16)
    if gu is not None:
        _need(gu, "gu", (p.T * p.k, 2 * p.I), torch.bfloat16)
    dev = x.device
    f32 = torch.float32
    g = dict(dx=_empty((p.T, p.H), torch.bfloat16, dev),
             dw_gate=_empty((p.E, p.H, p.I), f32, dev), dw_up=_empty((p.E, p.H, p.I), f32, dev),
             dw_down=_empty((p.E, p.I, p.H), f32, dev), dlogits=_empty((p.T, p.E), f32, dev),
             dtopk_w=_empty((p.T, p.k), f32, dev))
    if w_router is not None:
        _need(w_router, "w_router", (p.E, p.H), torch.bfloat16)
        g["dw_router"] = _empty((p.E, p.H), f32, dev)
    sv = MoeSavedRouting(*(routing[n].data_ptr() for n in
                           ("topk_ids", "topk_w", "offsets", "row_token", "slot_to_row")))
    gr = MoeGrads(*((g[n].data_ptr() if n in g else None) for n in
                    ("dx", "dw_gate", "dw_up", "dw_down", "dlogits", "dtopk_w", "dw_router")))
    ws = workspace(p, OP_BACKWARD, dev) if ws is None else ws
    c = p.c()
    _call("moe_layer_backward", ctypes.byref(c), _ptr(x), _ptr(logits), _ptr(w_router),
          _ptr(packed_gate_up), _ptr(packed_down), _ptr(packed_bwd_gate_up), _ptr(packed_bwd_down),
          ctypes.byref(sv), _ptr(yp), _ptr(gu), _ptr(dy), ctypes.byref(gr), _ptr(ws), ws.numel(),
          _stream())
    return g


def routing_buffers(p: Problem, device="cuda"):
    """Preallocated routing outputs for layer(..., routing=...)."""
    tk = p.T * p.k
    return dict(topk_ids=_empty((p.T, p.k), torch.int32, device),
                topk_w=_empty((p.T, p.k), torch.float32, device),
                keep=_empty((p.T, p.k), torch.uint8, device),
                counts=_empty((p.E,), torch.int32, device),
                offsets=_empty((p.E + 1,), torch.int32, device),
                row_token=_empty((tk,), torch.int32, device),
                slot_to_row=_empty((p.T, p.k), torch.int32, device))
