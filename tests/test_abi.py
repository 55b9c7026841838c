"""The C-ABI library: it loads, exports every entry point include/moe.h declares, and its
host-side checks (problem validation, workspace and packed sizes) behave as documented.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def fake_ptrs(n, base=1 << 44):
    """n distinct 256-aligned host-side stand-ins for device pointers, 64 GiB apart (so no
    two of the buffers a call sizes from its problem overlap).  Only calls that return before
    launching anything may receive them."""
    return [ctypes.c_void_p(base + (i << 36)) for i in range(n)]


@pytest.fixture(scope="module")
def moe():
    import expert_ffn_moe_amd

    return expert_ffn_moe_amd


def test_library_exports_every_declared_symbol(moe):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(moe.lib, n), n
    assert set(names) == set(moe.EXPORTS)


def test_library_is_built_for_gfx950():
    # the device code objects embedded in the library name their target
    lib = os.path.join(ROOT, "expert_ffn_moe_amd", "libmoe.so")
    data = open(lib, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings(moe):
    assert moe.status_str(0) == "ok"
    assert "workspace" in moe.status_str(3)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), 1), (dict(k=9, E=8), 1), (dict(H=-1), 1), (dict(E=2000), 2), (dict(k=33, E=64), 2),
    (dict(H=100), 2), (dict(I=96), 2), (dict(renormalize=2), 1),
])
def test_problem_check(moe, kw, status):
    base = dict(T=64, H=128, E=8, k=2, I=128, capacity=0, renormalize=1, dtype="bf16")
    base.update(kw)
    assert moe.Problem(**base).check() == status


def test_problem_check_dtype_pairs(moe):
    p = moe.Problem(64, 128, 8, 2, 128)
    c = p.c()
    c.w_dtype = 0  # bf16 activations with fp32 weights: not handled
    assert moe.lib.moe_problem_check(ctypes.byref(c)) == moe.MOE_ERR_UNSUPPORTED
    c.w_dtype = 7
    assert moe.lib.moe_problem_check(ctypes.byref(c)) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib.moe_problem_check(None) == moe.MOE_ERR_INVALID_ARG
    # fp32 accepts multiples of 8
    assert moe.Problem(64, 136, 8, 2, 24, dtype="f32").check() == 0


def test_workspace_and_packed_sizes(moe):
    p = moe.Problem(T=4096, H=2048, E=128, k=8, I=768)
    assert p.workspace_bytes(moe.OP_ROUTE) == 0  # no cap: routing needs no scratch
    assert p.workspace_bytes(moe.OP_COMBINE) == 0
    assert p.workspace_bytes(moe.OP_DISPATCH) > 0
    ffn = p.workspace_bytes(moe.OP_FFN)
    assert ffn >= 4096 * 8 * 768 * 2  # the intermediate activation
    # the layer keeps yp and the intermediate activation; the rows are gathered by the
    # gate/up kernel itself, so there is no xp in it
    layer = p.workspace_bytes(moe.OP_LAYER)
    assert 4096 * 8 * 2048 * 2 + ffn <= layer < 2 * 4096 * 8 * 2048 * 2 + ffn
    capped = moe.Problem(T=4096, H=2048, E=128, k=8, I=768, capacity=1024)
    assert capped.workspace_bytes(moe.OP_ROUTE) >= 4096 * 8 * 4
    assert p.packed_bytes(moe.W_GATE_UP) == 2 * 128 * 2048 * 768 * 2
    assert p.packed_bytes(moe.W_DOWN) == 128 * 2048 * 768 * 2
    bad = moe.Problem(T=0, H=2048, E=128, k=8, I=768)
    assert bad.workspace_bytes(moe.OP_LAYER) == 0 and bad.packed_bytes(0) == 0


def test_calls_reject_bad_arguments_before_touching_the_device(moe):
    # NULL pointers and a missing workspace are refused on the host
    p = moe.Problem(T=64, H=128, E=8, k=2, I=128, capacity=4)
    c = p.c()
    st = moe.lib.moe_route(ctypes.byref(c), None, None, None, None, None, 0, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    f = fake_ptrs(6)
    st = moe.lib.moe_route(ctypes.byref(c), f[0], f[1], f[2], f[3], None, 0, None)
    assert st == moe.MOE_ERR_WORKSPACE
    st = moe.lib.moe_combine(ctypes.byref(c), ctypes.c_void_p(8), f[1], f[2], f[3], None)
    assert st == moe.MOE_ERR_INVALID_ARG  # misaligned yp
    st = moe.lib.moe_expert_gate_up_gather(ctypes.byref(c), f[0], None, f[1], f[2], f[3], None, 0,
                                           None)
    assert st == moe.MOE_ERR_INVALID_ARG  # gather without row_token
    bad = moe.Problem(T=64, H=100, E=8, k=2, I=128).c()
    st = moe.lib.moe_layer(ctypes.byref(bad), f[0], f[1], f[2], f[3], f[4], None, None, None, None,
                           None, None, None, None, 0, None)
    assert st == moe.MOE_ERR_UNSUPPORTED


def test_fp8_problem_check_and_sizes(moe):
    # FP8 weights go with bf16 activations and need H, I multiples of 128
    assert moe.Problem(64, 256, 8, 2, 384, dtype="fp8").check() == 0
    assert moe.Problem(64, 192, 8, 2, 384, dtype="fp8").check() == moe.MOE_ERR_UNSUPPORTED
    assert moe.Problem(64, 256, 8, 2, 320, dtype="fp8").check() == moe.MOE_ERR_UNSUPPORTED
    c = moe.Problem(64, 256, 8, 2, 384, dtype="fp8").c()
    c.act_dtype = moe.MOE_F32
    assert moe.lib.moe_problem_check(ctypes.byref(c)) == moe.MOE_ERR_UNSUPPORTED
    c.act_dtype = moe.MOE_FP8  # FP8 is a weight format only
    assert moe.lib.moe_problem_check(ctypes.byref(c)) == moe.MOE_ERR_INVALID_ARG
    p = moe.Problem(T=4096, H=2048, E=128, k=8, I=768, dtype="fp8")
    align = lambda n: (n + 255) & ~255
    # codes (one byte per weight) then one scale byte per 32 along K, grouped 4 k-steps of
    # 64 per 4-byte word
    gu_codes = 128 * 2 * 2048 * 768
    assert p.packed_bytes(moe.W_GATE_UP) == align(gu_codes) + 128 * (768 // 32) * 2 * 8 * 256
    assert p.packed_bytes(moe.W_DOWN) == align(128 * 768 * 2048) + 128 * (2048 // 32) * 3 * 256
    # the FFN workspace holds the quantised intermediate and the quantised input rows
    tk = 4096 * 8
    q = lambda cols: align(tk * cols) + tk * cols // 32
    assert p.workspace_bytes(moe.OP_FFN) == align(q(768)) + align(q(2048))
    assert p.a_shape() == ((q(768),), moe.torch.uint8)


def test_quantize_fp8_rejects_bad_arguments(moe):
    fake = ctypes.c_void_p(256)
    q = moe.lib.moe_quantize_fp8
    assert q(fake, ctypes.c_int64(4), ctypes.c_int32(48), fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert q(fake, ctypes.c_int64(-1), ctypes.c_int32(64), fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert q(None, ctypes.c_int64(4), ctypes.c_int32(64), fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert q(ctypes.c_void_p(8), ctypes.c_int64(4), ctypes.c_int32(64), fake, fake,
             None) == moe.MOE_ERR_INVALID_ARG
    assert q(None, ctypes.c_int64(0), ctypes.c_int32(64), None, None, None) == moe.MOE_OK


def test_router_workspace_holds_the_partial_logits(moe):
    # split-K partial planes [S][T][E] f32 with S >= 1, plus the capacity scratch with a cap
    p = moe.Problem(T=16384, H=7168, E=256, k=8, I=2048)
    base = p.workspace_bytes(moe.OP_ROUTER)
    assert base >= 16384 * 256 * 4 and base % (16384 * 256 * 4) == 0
    capped = moe.Problem(T=16384, H=7168, E=256, k=8, I=2048, capacity=4096)
    assert capped.workspace_bytes(moe.OP_ROUTER) > base
    assert moe.Problem(T=8, H=64, E=320, k=2, I=64).workspace_bytes(moe.OP_ROUTER) == 0
    # grouped routing from logits needs no scratch without a cap
    assert p.workspace_bytes(moe.OP_ROUTE) == 0


def test_router_and_grouped_route_reject_bad_arguments(moe):
    lg, ids, w, keep, x, wr = fake_ptrs(6)
    p = moe.Problem(T=64, H=128, E=64, k=4, I=128).c()
    P = ctypes.byref(p)
    gr = moe.lib.moe_route_grouped
    assert gr(P, lg, 3, 1, ids, w, keep, None, 0, None) == moe.MOE_ERR_INVALID_ARG  # 64 % 3
    assert gr(P, lg, 8, 9, ids, w, keep, None, 0, None) == moe.MOE_ERR_INVALID_ARG  # 9 > 8
    assert gr(P, lg, 64, 2, ids, w, keep, None, 0, None) == moe.MOE_ERR_INVALID_ARG  # k > 2
    assert gr(P, lg, 128, 1, ids, w, keep, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    r = moe.lib.moe_router
    assert r(P, x, wr, 1, 1, None, ids, w, keep, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert r(P, ctypes.c_void_p(8), wr, 1, 1, None, ids, w, keep, None, 0,
             None) == moe.MOE_ERR_INVALID_ARG
    f32 = moe.Problem(T=64, H=128, E=64, k=4, I=128, dtype="f32").c()
    assert r(ctypes.byref(f32), x, wr, 1, 1, None, ids, w, keep, None, 0,
             None) == moe.MOE_ERR_UNSUPPORTED


def test_overlapping_buffers_are_rejected(moe):
    """An output overlapping an input, another output or the workspace is refused on the
    host (MOE_ERR_INVALID_ARG) before anything is enqueued; buffers that only touch are
    not overlapping.  With distinct buffers the calls below go on to their next host check
    (the missing workspace)."""
    INV, WS = moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_WORKSPACE
    T, H, E, k, I = 64, 128, 8, 2, 128
    c = moe.Problem(T=T, H=H, E=E, k=k, I=I, capacity=4).c()
    P = ctypes.byref(c)
    lg, ids, w, keep, x, xp, cnt, off, rt, s2r, ws = fake_ptrs(11)
    at = lambda ptr, nbytes: ctypes.c_void_p(ptr.value + nbytes)
    route = moe.lib.moe_route
    assert route(P, lg, ids, w, keep, None, 0, None) == WS
    assert route(P, lg, at(lg, 64), w, keep, None, 0, None) == INV        # ids inside logits
    assert route(P, lg, ids, at(ids, T * k * 4 - 4), keep, None, 0, None) == INV  # w over ids' end
    assert route(P, lg, ids, at(ids, T * k * 4), keep, None, 0, None) == WS  # w right after ids
    assert route(P, lg, ids, w, keep, at(keep, 8), 1 << 20, None) == INV  # workspace over keep
    disp = moe.lib.moe_dispatch
    args = lambda **kw: [kw.get(n, v) for n, v in (("x", x), ("ids", ids), ("keep", keep),
                                                     ("cnt", cnt), ("off", off), ("rt", rt),
                                                     ("s2r", s2r), ("xp", xp))]
    ok = args()
    assert disp(P, *ok, None, 0, None) == WS
    assert disp(P, *args(xp=at(x, 16 * H * 2)), None, 0, None) == INV    # xp over x
    assert disp(P, *args(s2r=rt), None, 0, None) == INV                   # two outputs alike
    assert disp(P, *args(off=at(ids, 4)), None, 0, None) == INV           # offsets over ids
    # inputs may share memory (keep inside the ids buffer is only read)
    assert disp(P, *args(keep=at(ids, 8)), None, 0, None) == WS
    # calls without a workspace check: only the refusals can be exercised off the GPU
    import torch
    buf = torch.empty(4 << 20, dtype=torch.uint8)  # host bytes; nothing is launched
    yp, y = buf[: T * k * H * 2], buf[T * H * 2:]  # aliased views: y starts inside yp
    assert moe.lib.moe_combine(P, ctypes.c_void_p(yp.data_ptr()), w, s2r,
                               ctypes.c_void_p(y.data_ptr()), None) == INV
    pb = moe.Problem(T=T, H=H, E=E, k=k, I=I).c()
    PB = ctypes.byref(pb)
    assert moe.lib.moe_expert_down(PB, xp, off, x, at(xp, 256), None, 0, None) == INV  # yp over a
    assert moe.lib.moe_layer(PB, x, lg, keep, cnt, at(x, 512), None, None, None, None, None,
                             None, None, ws, 1 << 30, None) == INV        # y over x
    assert moe.lib.moe_layer(PB, x, lg, keep, cnt, xp, ids, at(ids, 4), None, None, None,
                             None, None, ws, 1 << 30, None) == INV        # topk_w over topk_ids
