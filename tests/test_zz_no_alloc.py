"""moe_layer_static, the layer entry point that allocates nothing: its workspace is a
file-scope device array of the library (moe_layer_static_max_bytes), so callers that cannot
allocate (graph capture, tight serving loops) can run the layer.  Checked through the C ABI
against moe_layer on the same inputs, bit for bit: two calls in a row, the second on a
smaller problem (the array keeps the first call's contents), on the decode- and the
prefill-shaped kernels; a problem whose workspace exceeds the array is refused."""
import ctypes

import pytest
import torch

import synth
from synth import Workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def moe():
    import expert_ffn_moe_amd

    return expert_ffn_moe_amd


def static_fn(m):
    m.lib.moe_layer_static_max_bytes.restype = ctypes.c_size_t
    f = m.lib.moe_layer_static
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.POINTER(m.MoeProblem)] + [ctypes.c_void_p] * 13
    return f


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_static(m, p, inp, pgu, pd):
    y = torch.empty(p.T, p.H, dtype=p.torch_dtype, device=DEV)
    r = m.routing_buffers(p, DEV)
    c = p.c()
    st = static_fn(m)(ctypes.byref(c), ptr(inp["x"]), ptr(inp["logits"]), ptr(pgu), ptr(pd),
                      ptr(y), *(ptr(r[n]) for n in ("topk_ids", "topk_w", "keep", "counts",
                                                   "offsets", "row_token", "slot_to_row")),
                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == m.MOE_OK, m.status_str(st)
    return y, r


CASES = [
    # decode-shaped (T*k <= 24 E): larger first, then smaller
    (Workload("static_decode", T=128, H=1024, E=64, k=8, I=512, capacity=0, dtype="bf16",
              logits="normal", seed=91),
     Workload("static_decode_small", T=40, H=1024, E=64, k=8, I=512, capacity=0, dtype="bf16",
              logits="normal+bias0.5", seed=92)),
    # prefill-shaped kernels, with a cap (capacity scratch in the array too)
    (Workload("static_prefill", T=900, H=512, E=8, k=2, I=256, capacity=200, dtype="bf16",
              logits="normal+zipf1.2", seed=93),
     Workload("static_prefill_small", T=300, H=512, E=8, k=2, I=256, capacity=0, dtype="bf16",
              logits="normal", seed=94)),
]


@pytest.mark.parametrize("first,second", CASES, ids=[c[0].name for c in CASES])
def test_static_layer_equals_moe_layer_twice(first, second):
    m = moe()
    for wl in (first, second):
        print(f"case {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity}",
              flush=True)
        p = m.Problem.of(wl)
        assert p.workspace_bytes(m.OP_LAYER) <= m.lib.moe_layer_static_max_bytes()
        inp = synth.make_inputs(wl, DEV)
        pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
        r_ref = m.routing_buffers(p, DEV)
        y_ref = m.layer(p, inp["x"], inp["logits"], pgu, pd, routing=r_ref)
        y, r = run_static(m, p, inp, pgu, pd)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        N = int(r_ref["offsets"][-1])
        for n in ("topk_ids", "topk_w", "keep", "counts", "offsets", "slot_to_row"):
            assert torch.equal(r[n], r_ref[n]), n
        assert torch.equal(r["row_token"][:N], r_ref["row_token"][:N])


def test_static_layer_refuses_a_workspace_beyond_the_array():
    m = moe()
    m.lib.moe_layer_static_max_bytes.restype = ctypes.c_size_t
    cap = m.lib.moe_layer_static_max_bytes()
    p = m.Problem(T=4096, H=2048, E=128, k=8, I=768)  # 128 MiB of expert outputs alone
    assert p.workspace_bytes(m.OP_LAYER) > cap
    c = p.c()
    f = static_fn(m)
    null = ctypes.c_void_p(None)
    # refused on the host before anything is enqueued
    assert f(ctypes.byref(c), *([null] * 13)) == m.MOE_ERR_WORKSPACE
