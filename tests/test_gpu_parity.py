"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: indices, weights' bits, keep flags, counts, offsets, the permutation and gathered rows
are bit-exact; floats within the tolerance of their dtype:
  fp32 problems : max|gpu - ref| <= 1e-5 * max|ref|   (normwise)
  bf16 problems : max|gpu - ref| <= 2e-2 * max|ref|   (against the fp64 oracle)
Small problems are compared element by element; the five full-size workloads on sampled
rows/tokens (all routing and layout outputs are still compared in full).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Workload

pytestmark = pytest.mark.gpu

DEV = "cuda"
ORACLE_THREADS = 16


def say(*a):
    print(*a, flush=True)


def moe():
    import expert_ffn_moe_amd

    return expert_ffn_moe_amd


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits(t)
    return t.detach().cpu().numpy()


def as_f32(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def tol_ok(got: np.ndarray, ref: np.ndarray, dtype: str):
    got = as_f32(got).astype(np.float64)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max() if ref.size else 0.0
    bound = (1e-5 if dtype == "f32" else 2e-2) * scale
    return err <= bound, err, scale


def problem_of(wl):
    return moe().Problem.of(wl)


def gpu_staged(p, inp):
    m = moe()
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    ids, w, keep = m.route(p, inp["logits"])
    d = m.dispatch(p, inp["x"], ids, keep)
    a = m.expert_gate_up(p, d["xp"], d["offsets"], pgu)
    yp = m.expert_down(p, a, d["offsets"], pd)
    y = m.combine(p, yp, w, d["slot_to_row"])
    torch.cuda.synchronize()
    return dict(topk_ids=ids, topk_w=w, keep=keep, a=a, yp=yp, y=y, pgu=pgu, pd=pd, **d)


def check_routing(p, logits_np, g):
    """Bit-exact routing, capacity and layout; returns the oracle's results."""
    ids, w = oracle.route(logits_np, p.k, p.renormalize)
    keep = oracle.capacity(ids, w, p.E, p.capacity)
    assert np.array_equal(host(g["topk_ids"]), ids), "topk_ids"
    assert np.array_equal(host(g["topk_w"]).view(np.uint32), w.view(np.uint32)), "topk_w bits"
    assert np.array_equal(host(g["keep"]), keep), "keep (dropped set)"
    lay = oracle.layout(ids, keep, p.E)
    N = lay["N"]
    assert np.array_equal(host(g["counts"]), lay["counts"]), "counts"
    assert np.array_equal(host(g["offsets"]), lay["offsets"]), "offsets"
    assert np.array_equal(host(g["row_token"])[:N], lay["row_token"][:N]), "row_token"
    assert np.array_equal(host(g["slot_to_row"]), lay["slot_to_row"]), "slot_to_row"
    return ids, w, keep, lay


def row_experts(offsets, rows):
    return (np.searchsorted(offsets, rows, side="right") - 1).astype(np.int32)


def check_ffn_and_combine(p, wl, inp, g, lay, w, rows=None, tokens=None):
    """yp on `rows` and y on `tokens` (None: all) against the fp64 oracle."""
    N = lay["N"]
    xh = host(inp["x"])
    rows = np.arange(N) if rows is None else np.asarray(rows)
    tokens = np.arange(p.T) if tokens is None else np.asarray(tokens)
    s2r = lay["slot_to_row"]
    # every row that a checked token needs
    need = s2r[tokens].ravel()
    rows = np.unique(np.concatenate([rows, need[need >= 0]])).astype(np.int64)
    rexp = row_experts(lay["offsets"], rows)
    experts = np.unique(rexp)
    local = np.searchsorted(experts, rexp).astype(np.int32)
    idx = torch.as_tensor(experts, device=inp["w_gate"].device)
    wg, wu, wd = (host(inp[n].index_select(0, idx)) for n in ("w_gate", "w_up", "w_down"))
    xrows = xh[lay["row_token"][rows]]
    # the gathered rows are exact copies
    assert np.array_equal(host(g["xp"][torch.as_tensor(rows, device=DEV)]), xrows), "xp rows"
    yp_ref = oracle.ffn_rows(xrows, local, wg, wu, wd, nthreads=ORACLE_THREADS)
    yp_gpu = host(g["yp"][torch.as_tensor(rows, device=DEV)])
    ok, err, scale = tol_ok(yp_gpu, yp_ref, p.dtype)
    say(f"  yp: {rows.size} rows, max err {err:.3e} of max|ref| {scale:.3e}")
    assert ok, ("yp", err, scale)
    # combine over the checked tokens, from the oracle's rows
    pos = {int(r): i for i, r in enumerate(rows)}
    s2r_sub = np.array([[pos[int(r)] if r >= 0 else -1 for r in s2r[t]] for t in tokens], np.int32)
    y_ref = oracle.combine(np.arange(tokens.size, dtype=np.int32), w[tokens], s2r_sub, yp_ref)
    y_gpu = host(g["y"][torch.as_tensor(tokens, device=DEV)])
    ok, err, scale = tol_ok(y_gpu, y_ref, p.dtype)
    say(f"  y : {tokens.size} tokens, max err {err:.3e} of max|ref| {scale:.3e}")
    assert ok, ("y", err, scale)
    # tokens whose every slot was dropped output exactly 0
    dead = tokens[(s2r[tokens] < 0).all(axis=1)]
    if dead.size:
        assert np.all(as_f32(host(g["y"][torch.as_tensor(dead, device=DEV)])) == 0.0)


def sampled_rows_and_tokens(lay, T, rng, tile=128, n_tokens=64):
    """Rows and tokens for a full-size check: the first and the last row of every non-empty
    expert and of every `tile`-row block inside it (the blocks of the grouped GEMM's M tiles,
    so every work item of the persistent kernels, on whichever XCD range it falls, has rows
    checked in all its columns), plus n_tokens random tokens (and the first and last)."""
    offs = lay["offsets"]
    rows = []
    for e in range(len(offs) - 1):
        a, b = int(offs[e]), int(offs[e + 1])
        for r0 in range(a, b, tile):
            rows += [r0, min(r0 + tile, b) - 1]
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, n_tokens), replace=False)]))
    return np.unique(np.asarray(rows, np.int64)), tokens


# --------------------------------------------------------------------------------------
# small problems: every output compared
# --------------------------------------------------------------------------------------
SMALL = [
    Workload("prefill_ragged", T=1000, H=576, E=4, k=2, I=320, capacity=0, dtype="bf16",
             logits="normal", seed=11),
    Workload("prefill_cap", T=700, H=256, E=8, k=3, I=192, capacity=200, dtype="bf16",
             logits="normal+zipf1.2", seed=12),
    Workload("decode_bias", T=40, H=512, E=64, k=4, I=256, capacity=0, dtype="bf16",
             logits="normal+bias0.5", seed=13),
    Workload("decode_all_to_one", T=40, H=256, E=64, k=4, I=128, capacity=0, dtype="bf16",
             logits="all_to_one", seed=14),
    Workload("single_token", T=1, H=128, E=8, k=2, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=15),
    Workload("one_expert", T=130, H=128, E=1, k=1, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=16),
    Workload("f32_cap_ties", T=100, H=64, E=4, k=2, I=32, capacity=30, dtype="f32",
             logits="ties012", seed=17),
    synth.WORKLOADS["tiny_f32"],
    # 500 rows per expert on average: four or five 128-row M tiles per expert with ragged
    # tails, a partial N group (H = 320: 10 panels)
    Workload("prefill_many_tiles", T=2000, H=320, E=4, k=2, I=192, capacity=0, dtype="bf16",
             logits="normal+bias0.5", seed=19),
    # many experts on the prefill kernels (T*k > 24 E): expert lookup and XCD ranges over
    # 600 experts, most with a handful of rows, some empty
    Workload("prefill_E600", T=2048, H=128, E=600, k=8, I=64, capacity=0, dtype="bf16",
             logits="normal+bias0.5", seed=18),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_layer_parity(wl):
    say(f"case {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity} {wl.dtype}")
    p = problem_of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_staged(p, inp)
    ids, w, keep, lay = check_routing(p, host(inp["logits"]), g)
    check_ffn_and_combine(p, wl, inp, g, lay, w)


# --------------------------------------------------------------------------------------
# routing and layout only: bit-exact on edge cases (ties, equal logits, maximum E and k,
# no renormalisation, every token on one expert)
# --------------------------------------------------------------------------------------
ROUTING = [
    Workload("max_E_k", T=257, H=64, E=1024, k=32, I=64, capacity=0, dtype="bf16", logits="normal", seed=21),
    Workload("no_renorm", T=300, H=64, E=64, k=6, I=64, capacity=0, dtype="bf16", logits="normal",
             seed=22, renormalize=0),
    Workload("no_renorm_E1000", T=65, H=64, E=1000, k=8, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=23, renormalize=0),
    Workload("equal_logits_cap", T=100, H=64, E=16, k=4, I=64, capacity=10, dtype="bf16",
             logits="equal", seed=24),
    Workload("ties_cap", T=1000, H=64, E=64, k=4, I=64, capacity=50, dtype="bf16", logits="ties012", seed=25),
    Workload("all_to_one_cap", T=500, H=64, E=32, k=2, I=64, capacity=100, dtype="bf16",
             logits="all_to_one", seed=26),
    Workload("cap_above_T", T=129, H=64, E=8, k=2, I=64, capacity=1000, dtype="bf16", logits="normal", seed=27),
    # two experts with 20,000 candidates each: more keys than the selection holds in LDS
    Workload("all_to_one_cap_big", T=20000, H=64, E=8, k=2, I=64, capacity=5000, dtype="bf16",
             logits="all_to_one", seed=29),
    Workload("E1_k1", T=3, H=64, E=1, k=1, I=64, capacity=0, dtype="bf16", logits="normal", seed=28),
    # layouts of more than 65536 slots over 300 chunks, with and without a capacity (the
    # column scan then splits each expert's chunks over all 16 wavefronts of its block)
    Workload("many_chunks", T=20000, H=64, E=64, k=4, I=64, capacity=0, dtype="bf16",
             logits="normal+bias0.5", seed=30),
    Workload("many_chunks_cap", T=18000, H=64, E=64, k=4, I=64, capacity=400, dtype="bf16",
             logits="normal", seed=32),
    # 256 chunks with the last one ragged, and 250 chunks with a capacity (its candidate
    # list too): chunk counts that split unevenly over the column scan's 16 wavefronts
    Workload("fused_scan_limit", T=16383, H=64, E=64, k=4, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=33),
    Workload("fused_scan_cap", T=16000, H=64, E=64, k=4, I=64, capacity=300, dtype="bf16",
             logits="normal+bias0.5", seed=34),
]


@pytest.mark.parametrize("wl", ROUTING, ids=[w.name for w in ROUTING])
def test_routing_and_dispatch_edge_cases(wl):
    say(f"case {wl.name}: T={wl.T} E={wl.E} k={wl.k} C={wl.capacity} renorm={wl.renormalize}")
    m = moe()
    p = problem_of(wl)
    logits = synth.make_logits(wl, DEV)
    x = synth.make_x(wl, DEV)
    ids, w, keep = m.route(p, logits)
    d = m.dispatch(p, x, ids, keep)
    torch.cuda.synchronize()
    g = dict(topk_ids=ids, topk_w=w, keep=keep, **d)
    _, _, _, lay = check_routing(p, host(logits), g)
    N = lay["N"]
    xp = oracle.gather(host(x), lay["row_token"], N)
    assert np.array_equal(host(d["xp"])[:N], xp)
    # the layer builds its layout from the selection's own histogram: the same layout
    inp = synth.make_inputs(wl, DEV)
    assert torch.equal(inp["logits"], logits)
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    r = m.routing_buffers(p)
    m.layer(p, inp["x"], inp["logits"], pgu, pd, routing=r)
    torch.cuda.synchronize()
    for n in ("topk_ids", "topk_w", "keep", "counts", "offsets", "slot_to_row"):
        assert torch.equal(r[n], g[n]), n
    assert torch.equal(r["row_token"][:N], g["row_token"][:N])


def test_dispatch_without_keep_and_with_caller_routing():
    """moe_dispatch on caller-supplied ids (keep = NULL means every slot is kept)."""
    m = moe()
    wl = Workload("caller_ids", T=333, H=128, E=16, k=3, I=64, capacity=0, dtype="bf16",
                  logits="normal", seed=31)
    p = problem_of(wl)
    rng = np.random.default_rng(31)
    ids = np.stack([rng.permutation(wl.E)[:wl.k] for _ in range(wl.T)]).astype(np.int32)
    x = synth.make_x(wl, DEV)
    d = m.dispatch(p, x, torch.as_tensor(ids, device=DEV), None)
    torch.cuda.synchronize()
    lay = oracle.layout(ids, None, wl.E)
    assert np.array_equal(host(d["counts"]), lay["counts"])
    assert np.array_equal(host(d["offsets"]), lay["offsets"])
    assert np.array_equal(host(d["row_token"])[:lay["N"]], lay["row_token"][:lay["N"]])
    assert np.array_equal(host(d["slot_to_row"]), lay["slot_to_row"])
    assert np.array_equal(host(d["xp"]), oracle.gather(host(x), lay["row_token"], lay["N"]))


def test_layer_matches_staged_calls_and_is_deterministic():
    m = moe()
    wl = SMALL[1]  # with a cap
    say(f"case layer vs staged: {wl.name}")
    p = problem_of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_staged(p, inp)
    outs = []
    for _ in range(2):
        r = m.routing_buffers(p)
        y = m.layer(p, inp["x"], inp["logits"], g["pgu"], g["pd"], routing=r)
        torch.cuda.synchronize()
        outs.append((y, r))
    for y, r in outs:
        assert torch.equal(y, g["y"])
        for n in ("topk_ids", "topk_w", "keep", "counts", "offsets", "slot_to_row"):
            assert torch.equal(r[n], g[n]), n
        N = int(g["offsets"][-1])
        assert torch.equal(r["row_token"][:N], g["row_token"][:N])
    # the staged path is deterministic too
    g2 = gpu_staged(p, inp)
    N = int(g["offsets"][-1])
    assert torch.equal(g2["y"], g["y"])
    for n in ("yp", "xp", "a"):  # rows past N are never written
        assert torch.equal(g2[n][:N], g[n][:N]), n


def test_layer_with_a_dirty_workspace():
    """moe_layer keeps no state in its workspace between calls: whatever the workspace holds
    beforehand (its prefill GEMMs' work-item counters included, which the layer zeroes
    itself), the output equals the staged calls' bit for bit.  A prefill-shaped problem
    (4,000 rows per expert: 256 M tiles and 512 items per GEMM, two per block) so that the
    blocks take items from the counters."""
    m = moe()
    wl = Workload("claims", T=16000, H=1024, E=8, k=2, I=512, capacity=0, dtype="bf16",
                  logits="normal", seed=41)
    say(f"case layer with a dirty workspace: {wl.name}")
    p = problem_of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_staged(p, inp)
    ws = m.workspace(p, m.OP_LAYER, DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    for fill in ("ones", "random", "random", "zeros"):
        if fill == "ones":
            ws.fill_(0xFF)
        elif fill == "zeros":
            ws.zero_()
        else:
            ws.copy_(torch.randint(0, 256, ws.shape, generator=gen, device=DEV,
                                   dtype=torch.int32).to(torch.uint8))
        y = m.layer(p, inp["x"], inp["logits"], g["pgu"], g["pd"], ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, g["y"]), fill


def test_expert_ffn_equals_gate_up_then_down():
    m = moe()
    wl = SMALL[0]
    p = problem_of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_staged(p, inp)
    yp = m.expert_ffn(p, g["xp"], g["offsets"], g["pgu"], g["pd"])
    torch.cuda.synchronize()
    N = int(g["offsets"][-1])
    assert torch.equal(yp[:N], g["yp"][:N])


@pytest.mark.parametrize("wl", [SMALL[0], SMALL[2], SMALL[6]], ids=lambda w: w.name)
def test_gate_up_gather_equals_gate_up_on_gathered_rows(wl):
    """Reading the token rows through row_token (no xp) gives the xp result bit for bit,
    for the prefill, decode and fp32 kernels; the layout-only dispatch gives the same
    layout as the full one."""
    m = moe()
    p = problem_of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_staged(p, inp)
    d = m.dispatch(p, inp["x"], g["topk_ids"], g["keep"], rows=False)
    a = m.expert_gate_up_gather(p, inp["x"], d["row_token"], d["offsets"], g["pgu"])
    torch.cuda.synchronize()
    assert d["xp"] is None
    for name in ("counts", "offsets", "row_token", "slot_to_row"):
        N = int(g["offsets"][-1]) if name == "row_token" else None
        assert torch.equal(d[name][:N], g[name][:N]), name
    N = int(g["offsets"][-1])
    assert torch.equal(a[:N], g["a"][:N])


def test_workspace_too_small_is_an_error():
    m = moe()
    p = m.Problem(T=64, H=128, E=8, k=2, I=64, capacity=0)
    x = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros(64, 2, dtype=torch.int32, device=DEV)
    ids[:, 1] = 1
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(m.MoeError) as ei:
        m.dispatch(p, x, ids, None, ws=ws)
    assert ei.value.status == m.MOE_ERR_WORKSPACE


# --------------------------------------------------------------------------------------
# the five full-size workloads: routing and layout in full, FFN/combine on samples
# --------------------------------------------------------------------------------------
FULL = ["tiny_f32", "qwen3_30b_a3b", "glm_skew_cap", "dsv3_prefill", "dsv3_decode"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    wl = synth.WORKLOADS[name]
    say(f"case {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity} {wl.dtype}")
    m = moe()
    p = problem_of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_staged(p, inp)
    ids, w, keep, lay = check_routing(p, host(inp["logits"]), g)
    N = lay["N"]
    say(f"  routing/layout bit-exact, N={N} kept of {wl.T * wl.k}")
    # every gathered row is its token's row (checked on the device, any size)
    rt = g["row_token"][:N].long()
    assert torch.equal(g["xp"][:N], inp["x"].index_select(0, rt))
    # gate/up reading the token rows through row_token equals gate/up on xp
    a2 = m.expert_gate_up_gather(p, inp["x"], g["row_token"], g["offsets"], g["pgu"])
    torch.cuda.synchronize()
    assert torch.equal(a2[:N], g["a"][:N])
    del a2
    # the fused layer gives the same result as the staged calls
    r = m.routing_buffers(p)
    y = m.layer(p, inp["x"], inp["logits"], g["pgu"], g["pd"], routing=r)
    torch.cuda.synchronize()
    assert torch.equal(y, g["y"])
    rng = np.random.default_rng(wl.seed)
    if wl.T * wl.k * wl.H * wl.I <= 2 ** 31:
        rows, tokens = None, None  # small enough: everything
    else:
        rows, tokens = sampled_rows_and_tokens(lay, wl.T, rng)
    check_ffn_and_combine(p, wl, inp, g, lay, w, rows=rows, tokens=tokens)
    del g, inp
    torch.cuda.empty_cache()

