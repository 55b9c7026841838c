"""GPU parity of the FP8 path (E4M3 codes, UE8M0 scales per 32 along K) against the oracle.

Bar:
  * quantisation (moe_quantize_fp8, and the weight quantisation inside moe_pack_weights,
    checked through the layer result): codes and scale bytes bit-exact;
  * the quantised intermediate `a`: the value that gets quantised carries the fp32
    accumulation error of g and u (the oracle's is exact), which is large relative to a
    where g or u nearly cancel, so a code may land a step or more away from the oracle's.
    Checked element by element: dequant(a_gpu) is within half an E4M3 step of the exact
    value plus the propagated accumulation bound eps_acc(K) * sum|terms| for g and u
    (K = H terms, each an exact product of two E4M3 values and two power-of-two scales;
    any order of floating-point summation of K terms errs by at most
    gamma_{K-1} = (K-1) u / (1 - (K-1) u) of the sum of their magnitudes, taken here with
    u = 2^-23 so that the bound holds whether the adders round to nearest or truncate);
    scales differ from the oracle's by at most one; at most 1% of codes and of scales
    differ at all;
  * yp and y: max|gpu - ref| <= 2e-2 * max|ref|, ref the oracle's fp64 result on the
    same quantised operands (bf16 output rounding is 2^-9 relative; the rest is the
    accumulation order and the rare adjacent-code roundings above).
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
TOL = 2e-2


def say(*a):
    print(*a, flush=True)


def moe():
    import expert_ffn_moe_amd

    return expert_ffn_moe_amd


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits(t)
    return t.detach().cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def normwise(got_bits: np.ndarray, ref: np.ndarray):
    got = bf16_to_f64(got_bits)
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    return err <= TOL * scale, err, scale


def eps_acc(K: int) -> float:
    """Error bound of a K-term floating-point sum relative to the sum of the terms'
    magnitudes, gamma_{K-1} with unit roundoff 2^-23 (fp32 summation, rounding to nearest
    or toward zero; the terms are exact products)."""
    ku = (K - 1) * 2.0 ** -23
    return ku / (1.0 - ku)


def e4m3_quantum(v: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """Spacing of the E4M3 grid (times the block scale) at the magnitude of v: 2^(x - 3)
    for v in the binade [2^x, 2^(x+1)), x >= -6; 2^-9 in the subnormal range."""
    e = scale_bytes.astype(np.int64) - 127
    s = np.abs(v) * np.exp2(-e.astype(np.float64))
    x = np.floor(np.log2(np.maximum(s, 2.0 ** -6)))
    return np.exp2(x - 3 + e)


def check_intermediate(codes_g, scales_g, codes_o, scales_o, a_exact, g, u, sg, su, K):
    """The quantised intermediate against the oracle (rows x I):
    every GPU element lies within half an E4M3 step (at its own scale) of a value that the
    fp32 accumulation could have produced: |dequant(a_gpu) - a| <= q/2 + da, with a the
    exact fp64 SwiGLU value, da = |d silu(g)/dg * u| * eps * sum|g terms|
    + |silu(g)| * eps * sum|u terms| + 1e-5 |a|, eps = eps_acc(K); scales differ by at
    most one."""
    EPS_ACC = eps_acc(K)
    ds = scales_g.astype(np.int64) - scales_o.astype(np.int64)
    assert np.abs(ds).max(initial=0) <= 1, "a: scale off by more than one"
    sc = np.repeat(scales_g, oracle.QBLOCK, axis=1)
    deq = oracle.dequant(codes_g, scales_g, 1)
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    da = np.abs(dsilu * u) * EPS_ACC * sg + np.abs(g * sig) * EPS_ACC * su + 1e-5 * np.abs(a_exact)
    bound = 0.5 * e4m3_quantum(deq, sc) + da
    err = np.abs(deq - a_exact)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), ("a", worst, deq[worst], a_exact[worst], bound[worst])
    frac_s = np.count_nonzero(ds) / max(ds.size, 1)
    frac_c = np.count_nonzero(codes_g != codes_o) / max(codes_g.size, 1)
    say(f"  a : scales differ from the oracle's on {frac_s:.2e} of blocks, codes on {frac_c:.2e}")
    assert frac_c <= 0.01 and frac_s <= 0.01, (frac_c, frac_s)


# --------------------------------------------------------------------------------------
# the quantiser: bit-exact
# --------------------------------------------------------------------------------------
def special_rows(cols: int, rng) -> np.ndarray:
    """bf16 rows that cover the format's corners, one block of 32 per case."""
    f = np.float32
    cases = [
        np.zeros(32, f),                                     # all-zero block: scale 2^0
        -np.zeros(32, f),                                    # signed zeros
        np.full(32, 448.0, f),                               # amax exactly 448: scale 2^0
        np.full(32, 448.0 * 2.0 ** -8, f),                   # the 2^-8 scale case
        np.array([1.75 * 2.0 ** -8] + [2.0 ** -20] * 31, f), # tiny elements under a big one
        np.array([3.0e38] + [1.0] * 31, f),                  # near the bf16 maximum
        np.array([1.0e-38] * 32, f),                         # bf16 subnormal range
        np.linspace(-448, 448, 32, dtype=f),                 # both signs
        (rng.standard_normal(32) * 1e-3).astype(f),
        (np.arange(32) * 0.0625 - 1.0).astype(f),            # E4M3 half-way points
    ]
    blocks = [cases[i % len(cases)] for i in range(cols // 32)]
    return np.concatenate(blocks)[None, :]


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (1000, 2048), (129, 7168)])
def test_quantize_fp8_bit_exact(rows, cols):
    say(f"case quantize rows={rows} cols={cols}")
    m = moe()
    g = torch.Generator().manual_seed(rows * 131 + cols)
    x = (torch.randn(rows, cols, generator=g) * torch.exp(torch.randn(rows, 1, generator=g) * 4))
    x = x.to(torch.bfloat16)
    rng = np.random.default_rng(cols)
    sp = torch.as_tensor(special_rows(cols, rng)).to(torch.bfloat16)
    x[0] = sp[0]
    xd = x.to(DEV)
    codes, scales = m.quantize_fp8(xd)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quant_rows(synth.bf16_bits(x))
    assert np.array_equal(host(scales), s_ref), "scales"
    assert np.array_equal(host(codes), c_ref), "codes"


def test_quantize_fp8_empty_is_a_no_op():
    m = moe()
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    codes, scales = m.quantize_fp8(x)
    torch.cuda.synchronize()
    assert codes.shape == (0, 64) and scales.shape == (0, 2)


# --------------------------------------------------------------------------------------
# the FP8 FFN on small problems: every row compared
# --------------------------------------------------------------------------------------
SMALL = [
    # ragged tails, 5 stages of 128 along H (odd), 3 along I (odd), several M tiles
    Workload("fp8_prefill_ragged", T=1000, H=640, E=4, k=2, I=384, capacity=0, dtype="fp8",
             logits="normal", seed=41),
    Workload("fp8_prefill_cap", T=700, H=256, E=8, k=3, I=256, capacity=200, dtype="fp8",
             logits="normal+zipf1.2", seed=42),
    # few rows per expert: 64-row tiles
    Workload("fp8_decode_bias", T=40, H=512, E=64, k=4, I=256, capacity=0, dtype="fp8",
             logits="normal+bias0.5", seed=43),
    Workload("fp8_single_token", T=1, H=128, E=8, k=2, I=128, capacity=0, dtype="fp8",
             logits="normal", seed=44),
    Workload("fp8_one_expert", T=300, H=128, E=1, k=1, I=128, capacity=0, dtype="fp8",
             logits="normal", seed=45),
]


def gpu_fp8_staged(p, inp):
    m = moe()
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    ids, w, keep = m.route(p, inp["logits"])
    d = m.dispatch(p, inp["x"], ids, keep)
    a = m.expert_gate_up(p, d["xp"], d["offsets"], pgu)
    yp = m.expert_down(p, a, d["offsets"], pd)
    y = m.combine(p, yp, w, d["slot_to_row"])
    torch.cuda.synchronize()
    return dict(topk_ids=ids, topk_w=w, keep=keep, a=a, yp=yp, y=y, pgu=pgu, pd=pd, **d)


def oracle_weights(inp, experts):
    idx = torch.as_tensor(experts, device=inp["w_gate"].device)
    return [oracle.quant_weights(host(inp[n].index_select(0, idx)))
            for n in ("w_gate", "w_up", "w_down")]


def check_fp8_ffn(p, inp, g, rows=None, tokens=None, a_experts=None):
    """yp on `rows`, y on `tokens` (None: all) against the oracle; the intermediate a on
    the rows of `a_experts` among them (None: all; its exact reference needs each expert's
    weights dequantised on the host)."""
    m = moe()
    ids, w = oracle.route(host(inp["logits"]), p.k, p.renormalize)
    keep = oracle.capacity(ids, w, p.E, p.capacity)
    lay = oracle.layout(ids, keep, p.E)
    N = lay["N"]
    assert np.array_equal(host(g["offsets"]), lay["offsets"]), "offsets"
    assert np.array_equal(host(g["slot_to_row"]), lay["slot_to_row"]), "slot_to_row"
    rows = np.arange(N) if rows is None else np.asarray(rows)
    tokens = np.arange(p.T) if tokens is None else np.asarray(tokens)
    s2r = lay["slot_to_row"]
    need = s2r[tokens].ravel()
    rows = np.unique(np.concatenate([rows, need[need >= 0]])).astype(np.int64)
    rexp = (np.searchsorted(lay["offsets"], rows, side="right") - 1).astype(np.int32)
    experts = np.unique(rexp)
    local = np.searchsorted(experts, rexp).astype(np.int32)
    wq = oracle_weights(inp, experts)
    xrows = host(inp["x"])[lay["row_token"][rows]]
    xq, xs = oracle.quant_rows(xrows)
    yp_ref, a_ref, ac, asc = oracle.ffn_rows_fp8(xq, xs, local, *wq, want_a=True,
                                                 nthreads=ORACLE_THREADS)
    # exact gate/up values and the sums of |terms| that bound their accumulation error
    asel = np.ones(rows.size, bool) if a_experts is None else np.isin(experts[local], a_experts)
    xd = oracle.dequant(xq[asel], xs[asel], 1)
    la = local[asel]
    gu = np.empty((2, int(asel.sum()), p.I))
    su = np.empty((2, int(asel.sum()), p.I))
    for li in np.unique(la):
        sel = la == li
        for j, (cq, cs) in enumerate(wq[:2]):
            wdq = oracle.dequant(cq[li], cs[li], 0)
            gu[j][sel] = xd[sel] @ wdq
            su[j][sel] = np.abs(xd[sel]) @ np.abs(wdq)
    ridx = torch.as_tensor(rows[asel], device=DEV)
    codes_g, scales_g = m.split_quantized(p, g["a"])
    check_intermediate(host(codes_g.index_select(0, ridx)), host(scales_g.index_select(0, ridx)),
                       ac[asel], asc[asel], a_ref[asel], gu[0], gu[1], su[0], su[1], p.H)
    ridx = torch.as_tensor(rows, device=DEV)
    ok, err, scale = normwise(host(g["yp"].index_select(0, ridx)), yp_ref)
    say(f"  yp: {rows.size} rows, max err {err:.3e} of max|ref| {scale:.3e}")
    assert ok, ("yp", err, scale)
    pos = {int(r): i for i, r in enumerate(rows)}
    s2r_sub = np.array([[pos[int(r)] if r >= 0 else -1 for r in s2r[t]] for t in tokens], np.int32)
    y_ref = oracle.combine(np.arange(tokens.size, dtype=np.int32), w[tokens], s2r_sub, yp_ref)
    ok, err, scale = normwise(host(g["y"].index_select(0, torch.as_tensor(tokens, device=DEV))),
                              y_ref)
    say(f"  y : {tokens.size} tokens, max err {err:.3e} of max|ref| {scale:.3e}")
    assert ok, ("y", err, scale)
    return lay


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_fp8_small_layer_parity(wl):
    say(f"case {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity}")
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_fp8_staged(p, inp)
    lay = check_fp8_ffn(p, inp, g)
    N = lay["N"]
    # gate/up reading the token rows through row_token: the same bytes
    a2 = m.expert_gate_up_gather(p, inp["x"], g["row_token"], g["offsets"], g["pgu"])
    torch.cuda.synchronize()
    c1, s1 = m.split_quantized(p, g["a"])
    c2, s2 = m.split_quantized(p, a2)
    assert torch.equal(c1[:N], c2[:N]) and torch.equal(s1[:N], s2[:N])
    # the fused FFN and the fused layer give the staged result bit for bit
    yp = m.expert_ffn(p, g["xp"], g["offsets"], g["pgu"], g["pd"])
    y = m.layer(p, inp["x"], inp["logits"], g["pgu"], g["pd"])
    torch.cuda.synchronize()
    assert torch.equal(yp[:N], g["yp"][:N])
    assert torch.equal(y, g["y"])


def test_fp8_weights_quantised_at_pack_time_match_the_oracle():
    """Weights whose 32-element blocks along K span many binades (a different scale for
    every column and K block), one expert per few rows: checks the packed codes and the
    scale bytes of every column and K block."""
    m = moe()
    wl = Workload("fp8_pack", T=64, H=256, E=16, k=1, I=256, capacity=0, dtype="fp8",
                  logits="normal", seed=46)
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    gen = torch.Generator(device="cpu").manual_seed(46)
    for n in ("w_gate", "w_up", "w_down"):
        w = inp[n].float().cpu()
        E, K, N = w.shape
        f = torch.exp2(torch.randint(-12, 12, (E, K // 32, 1, N), generator=gen).float())
        inp[n] = (w * f.expand(E, K // 32, 32, N).reshape(E, K, N)).to(torch.bfloat16).to(DEV)
    g = gpu_fp8_staged(p, inp)
    check_fp8_ffn(p, inp, g)


def test_fp8_rejects_odd_widths():
    m = moe()
    p = m.Problem(T=8, H=192, E=4, k=2, I=128, dtype="fp8")
    w = torch.zeros(4, 192, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.MoeError) as ei:
        m.pack_weights(p, w, w, w.transpose(1, 2).contiguous())
    assert ei.value.status == m.MOE_ERR_UNSUPPORTED


# --------------------------------------------------------------------------------------
# full-size workloads with FP8 weights: layout and fused-vs-staged in full, the FFN on
# sampled rows and tokens
# --------------------------------------------------------------------------------------
FULL = ["qwen3_30b_a3b_fp8", "glm_skew_cap_fp8", "dsv3_prefill_fp8", "dsv3_decode_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_fp8_full_size_workload(name):
    wl = synth.WORKLOADS[name]
    say(f"case {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity}")
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    g = gpu_fp8_staged(p, inp)
    N = int(g["offsets"][-1])
    a2 = m.expert_gate_up_gather(p, inp["x"], g["row_token"], g["offsets"], g["pgu"])
    torch.cuda.synchronize()
    c1, s1 = m.split_quantized(p, g["a"])
    c2, s2 = m.split_quantized(p, a2)
    assert torch.equal(c1[:N], c2[:N]) and torch.equal(s1[:N], s2[:N])
    del a2
    y = m.layer(p, inp["x"], inp["logits"], g["pgu"], g["pd"])
    torch.cuda.synchronize()
    assert torch.equal(y, g["y"])
    del y
    rng = np.random.default_rng(wl.seed)
    offs = host(g["offsets"])
    # The oracle quantises, on the host, the weights of every expert a checked row belongs
    # to (about 1.4e8 elements a second on 16 threads) and evaluates each row with an
    # element-wise dequantisation (about 1 s of one thread per DeepSeek-V3 row): every
    # expert for the two smaller shapes (their 64 random tokens reach nearly all of them
    # anyway), the experts of 8 tokens for the DeepSeek-V3 shapes (11e9 weight elements in
    # all).  Checked: the first and the last row of every quantised expert (and, on the
    # smaller shapes, of every 128-row block inside it), the tokens' rows and their y; the
    # intermediate a on the rows of 6 of the experts.
    big = wl.E * 3 * wl.H * wl.I > 4e9
    tokens = np.unique(np.concatenate([[0, wl.T - 1],
                                       rng.choice(wl.T, 6 if big else 64, replace=False)]))
    s2r = host(g["slot_to_row"])
    need = s2r[tokens].ravel()
    need = need[need >= 0]
    experts = (np.unique(np.searchsorted(offs, need, side="right") - 1) if big
               else np.nonzero(offs[1:] > offs[:-1])[0])
    rows = []
    for e in experts:
        a_, b_ = int(offs[e]), int(offs[e + 1])
        for r0 in range(a_, b_, b_ - a_ if big else 128):
            rows += [r0, min(r0 + 128, b_) - 1] if not big else [a_, b_ - 1]
    rows = np.unique(np.asarray(rows, np.int64))
    a_experts = rng.choice(experts, min(6, experts.size), replace=False)
    say(f"  checking {rows.size} rows of {experts.size} experts and {tokens.size} tokens")
    check_fp8_ffn(p, inp, g, rows=rows, tokens=tokens, a_experts=a_experts)
    del g, inp
    torch.cuda.empty_cache()
