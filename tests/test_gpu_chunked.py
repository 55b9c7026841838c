"""GPU: the chunked layer (moe_layer_chunked) against moe_layer and the oracle.

Without a shared expert the chunked layer must equal moe_layer bit for bit (routing and
capacity are taken over all tokens first; every row's GEMM result and every token's
combine are independent of which other rows share its chunk), with or without the
auxiliary stream, for ragged and degenerate chunkings, bf16 / fp32 / FP8.  With a shared
expert, y is compared with the oracle: the routed combine plus the shared expert's SwiGLU
MLP of each token, fp64 (max|gpu - ref| <= 2e-2 max|ref| for bf16, 1e-5 for fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def moe():
    import expert_ffn_moe_amd

    return expert_ffn_moe_amd


def host(t):
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits(t)
    return t.detach().cpu().numpy()


def as_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


CASES = [
    (Workload("chk_cap", T=700, H=256, E=8, k=3, I=192, capacity=200, dtype="bf16",
              logits="normal+zipf1.2", seed=61), (1, 64, 300, 699, 700, 5000)),
    (Workload("chk_ragged", T=1000, H=576, E=4, k=2, I=320, capacity=0, dtype="bf16",
              logits="normal", seed=62), (128, 333)),
    (Workload("chk_decode", T=40, H=512, E=64, k=4, I=256, capacity=0, dtype="bf16",
              logits="normal+bias0.5", seed=63), (7, 40)),
    (Workload("chk_f32", T=256, H=128, E=8, k=2, I=256, capacity=30, dtype="f32",
              logits="ties012", seed=64), (50, 256)),
    (Workload("chk_fp8", T=1000, H=640, E=4, k=2, I=384, capacity=0, dtype="fp8",
              logits="normal", seed=65), (256, 999)),
]


@pytest.mark.parametrize("wl,chunks", CASES, ids=[c[0].name for c in CASES])
def test_chunked_equals_layer(wl, chunks):
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    ref = m.layer(p, inp["x"], inp["logits"], pgu, pd)
    torch.cuda.synchronize()
    aux = torch.cuda.Stream()
    for c in chunks:
        for stream in (None, aux):
            say(f"case {wl.name} chunk_tokens={c} aux={'yes' if stream else 'no'}")
            y = m.layer_chunked(p, inp["x"], inp["logits"], pgu, pd, c, aux_stream=stream)
            torch.cuda.synchronize()
            assert torch.equal(y, ref), (c, stream)


def shared_weights(wl, I, device):
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 131 + 7)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    wg = (torch.randn(1, wl.H, I, generator=g, device=device) / wl.H ** 0.5).to(dt)
    wu = (torch.randn(1, wl.H, I, generator=g, device=device) / wl.H ** 0.5).to(dt)
    wd = (torch.randn(1, I, wl.H, generator=g, device=device) / I ** 0.5).to(dt)
    return wg, wu, wd


def check_shared(wl, I, chunk, tokens=None):
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    swg, swu, swd = shared_weights(wl, I, DEV)
    ps = m.shared_problem(p, I)
    spgu, spd = m.pack_weights(ps, swg, swu, swd)
    aux = torch.cuda.Stream()
    y = m.layer_chunked(p, inp["x"], inp["logits"], pgu, pd, chunk, shared=(I, spgu, spd),
                        aux_stream=aux)
    y2 = m.layer_chunked(p, inp["x"], inp["logits"], pgu, pd, chunk, shared=(I, spgu, spd))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)  # the auxiliary stream changes nothing
    # oracle: routed rows of the checked tokens, their combine, plus the shared MLP
    logits = host(inp["logits"])
    ids, w = oracle.route(logits, p.k, p.renormalize)
    keep = oracle.capacity(ids, w, p.E, p.capacity)
    lay = oracle.layout(ids, keep, p.E)
    tokens = np.arange(p.T) if tokens is None else np.asarray(tokens)
    s2r = lay["slot_to_row"][tokens]
    rows = np.unique(s2r[s2r >= 0])
    rexp = (np.searchsorted(lay["offsets"], rows, side="right") - 1).astype(np.int32)
    experts = np.unique(rexp)
    idx = torch.as_tensor(experts, device=DEV)
    wg, wu, wd = (host(inp[n].index_select(0, idx)) for n in ("w_gate", "w_up", "w_down"))
    xh = host(inp["x"])
    yp = oracle.ffn_rows(xh[lay["row_token"][rows]], np.searchsorted(experts, rexp).astype(np.int32),
                         wg, wu, wd, nthreads=16)
    pos = {int(r): i for i, r in enumerate(rows)}
    s2r_sub = np.array([[pos[int(r)] if r >= 0 else -1 for r in row] for row in s2r], np.int32)
    sh = oracle.shared_expert(xh[tokens], host(swg), host(swu), host(swd), nthreads=16)
    ref = oracle.combine(np.arange(tokens.size, dtype=np.int32), w[tokens], s2r_sub, yp, sh)
    got = as_f64(host(y.index_select(0, torch.as_tensor(tokens, device=DEV))))
    err, scale = np.abs(got - ref).max(), np.abs(ref).max()
    tol = 1e-5 if wl.dtype == "f32" else 2e-2
    say(f"  y with shared expert: max err {err:.3e} of max|ref| {scale:.3e}")
    assert err <= tol * scale


@pytest.mark.parametrize("wl,I,chunk", [(CASES[0][0], 128, 300), (CASES[2][0], 192, 16),
                                        (CASES[3][0], 64, 50)], ids=["cap", "decode", "f32"])
def test_chunked_with_shared_expert(wl, I, chunk):
    say(f"case shared {wl.name} I={I} chunk={chunk}")
    check_shared(wl, I, chunk)


def test_chunked_rejects_bad_arguments():
    m = moe()
    p = m.Problem(T=64, H=128, E=8, k=2, I=128)
    c = p.c()
    import ctypes
    assert m.lib.moe_layer_chunked_workspace_bytes(ctypes.byref(c), 0, 0) == 0
    assert m.lib.moe_layer_chunked_workspace_bytes(ctypes.byref(c), 16, 100) == 0  # 100 % 64
    assert m.lib.moe_layer_chunked_workspace_bytes(ctypes.byref(c), 16, 0) > 0
    x = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros(64, 8, dtype=torch.float32, device=DEV)
    w = torch.zeros(8, 128, 128, dtype=torch.bfloat16, device=DEV)
    pgu, pd = m.pack_weights(p, w, w, w)
    with pytest.raises(m.MoeError) as ei:
        m.layer_chunked(p, x, lg, pgu, pd, 16, ws=torch.empty(256, dtype=torch.uint8, device=DEV))
    assert ei.value.status == m.MOE_ERR_WORKSPACE


def test_chunked_full_size_dsv3_prefill():
    """DeepSeek-V3-shaped prefill in chunks of 4096 tokens (32K rows), layouts on the
    auxiliary stream: equal to the unchunked layer bit for bit."""
    wl = synth.WORKLOADS["dsv3_prefill"]
    say(f"case chunked {wl.name} chunk 4096")
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    del inp["w_gate"], inp["w_up"], inp["w_down"]
    ref = m.layer(p, inp["x"], inp["logits"], pgu, pd)
    y = m.layer_chunked(p, inp["x"], inp["logits"], pgu, pd, 4096,
                        aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    del pgu, pd
    torch.cuda.empty_cache()


def test_chunked_full_size_qwen3_with_shared_expert():
    wl = synth.WORKLOADS["qwen3_30b_a3b"]
    say(f"case chunked {wl.name} chunk 1024, shared expert I=1536")
    rng = np.random.default_rng(7)
    tokens = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 30, replace=False)]))
    check_shared(wl, 1536, 1024, tokens=tokens)


def test_chunked_fp8_with_shared_expert():
    """FP8 weights for the routed and the shared expert: y against the FP8 oracle (the
    routed rows and the shared rows quantised exactly as the path does), normwise 2e-2."""
    wl = Workload("chk_fp8_shared", T=300, H=256, E=8, k=2, I=128, capacity=0, dtype="fp8",
                  logits="normal", seed=66)
    I = 256
    say(f"case {wl.name} shared I={I}")
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    swg, swu, swd = shared_weights(wl, I, DEV)
    spgu, spd = m.pack_weights(m.shared_problem(p, I), swg, swu, swd)
    y = m.layer_chunked(p, inp["x"], inp["logits"], pgu, pd, 128, shared=(I, spgu, spd),
                        aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    ids, w = oracle.route(host(inp["logits"]), p.k, p.renormalize)
    lay = oracle.layout(ids, None, p.E)
    N = lay["N"]
    xh = host(inp["x"])
    rexp = (np.searchsorted(lay["offsets"], np.arange(N), side="right") - 1).astype(np.int32)
    xq, xs = oracle.quant_rows(xh[lay["row_token"][:N]])
    wq = [oracle.quant_weights(host(inp[n])) for n in ("w_gate", "w_up", "w_down")]
    yp = oracle.ffn_rows_fp8(xq, xs, rexp, *wq)
    sq, ss = oracle.quant_rows(xh)
    swq = [oracle.quant_weights(host(t)) for t in (swg, swu, swd)]
    sh = oracle.ffn_rows_fp8(sq, ss, np.zeros(p.T, np.int32), *swq)
    ref = oracle.combine(np.arange(p.T, dtype=np.int32), w, lay["slot_to_row"], yp, sh)
    got = as_f64(host(y))
    err, scale = np.abs(got - ref).max(), np.abs(ref).max()
    say(f"  y: max err {err:.3e} of max|ref| {scale:.3e}")
    assert err <= 2e-2 * scale
