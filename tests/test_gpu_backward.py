"""GPU parity of the backward pass (moe_layer_backward) against the oracle's fp64 chain
rule (oracle/backward.py, itself pinned by finite differences and autograd).

Bar: every gradient normwise, max|gpu - ref| <= 2e-2 max|ref| over the checked entries
(bf16 operands and bf16 intermediate gradients -- dyp, da, [dg | du], dxp and the
recomputed g, u, a -- each rounded at 2^-9, fp32 accumulation); the routing used by the
backward is the forward's, which is bit-exact against the oracle (tested elsewhere).  The
backward with yp recomputed equals the one given the forward's yp bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import backward as ob
from synth import Workload

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-2


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


def forward(p, inp, wr=None):
    """The staged forward; returns the saved routing, yp and the logits it routed on."""
    m = moe()
    pgu, pd = m.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    if wr is not None:
        ids, w, keep, logits = m.router(p, inp["x"], wr, want_logits=True)
    else:
        logits = inp["logits"]
        ids, w, keep = m.route(p, logits)
    d = m.dispatch(p, inp["x"], ids, keep, rows=False)
    a = m.expert_gate_up_gather(p, inp["x"], d["row_token"], d["offsets"], pgu)
    yp = m.expert_down(p, a, d["offsets"], pd)
    torch.cuda.synchronize()
    routing = dict(topk_ids=ids, topk_w=w, offsets=d["offsets"], row_token=d["row_token"],
                   slot_to_row=d["slot_to_row"])
    return pgu, pd, routing, yp, logits


def make_dy(wl, device):
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 977 + 3)
    return torch.randn(wl.T, wl.H, generator=g, device=device).to(torch.bfloat16)


def check(name, got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err, scale = np.abs(got - ref).max(), np.abs(ref).max()
    say(f"  {name}: max err {err:.3e} of max|ref| {scale:.3e}")
    assert err <= TOL * scale, (name, err, scale)


def run_case(wl, router=False, tokens=None, experts=None, variants=True):
    """variants: also run the backward with yp recomputed and with the forward's saved g|u
    and compare them bit for bit (three sets of weight gradients in device memory at once;
    the largest shape runs only the saved-g|u backward)."""
    m = moe()
    p = m.Problem.of(wl)
    inp = synth.make_inputs(wl, DEV)
    wr = synth.make_router_weights(wl, DEV) if router else None
    pgu, pd, routing, yp, logits = forward(p, inp, wr)
    pbgu, pbd = m.pack_weights_backward(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    dy = make_dy(wl, DEV)
    # the forward's gate/up with the pre-activations saved: the same a
    a1 = m.expert_gate_up_gather(p, inp["x"], routing["row_token"], routing["offsets"], pgu)
    a2, gu = m.expert_gate_up_gather_gu(p, inp["x"], routing["row_token"], routing["offsets"],
                                        pgu)
    torch.cuda.synchronize()
    N = int(routing["offsets"][-1].item())
    assert torch.equal(a1[:N], a2[:N]), "a of the g|u-saving gate/up differs"
    del a1, a2
    g = m.layer_backward(p, inp["x"], logits, pgu, pd, pbgu, pbd, routing, dy, yp=yp,
                         w_router=wr, gu=gu)
    torch.cuda.synchronize()
    if variants:
        # the backward on the saved g|u gives the same bits as with its own recompute, and
        # recomputing yp changes nothing either
        for yp_in, gu_in, what in ((yp, None, "recomputed g|u"), (None, gu, "recomputed yp")):
            g2 = m.layer_backward(p, inp["x"], logits, pgu, pd, pbgu, pbd, routing, dy,
                                  yp=yp_in, w_router=wr, gu=gu_in)
            torch.cuda.synchronize()
            for n in g:
                assert torch.equal(g[n], g2[n]), f"{n}: {what} differs"
            del g2
    exps_gu = np.arange(p.E) if experts is None else np.asarray(experts)
    rg, ru = ob.gate_up_rows(host(inp["x"]), host(routing["row_token"]), host(routing["offsets"]),
                             host(inp["w_gate"]), host(inp["w_up"]), experts=exps_gu)
    offs = host(routing["offsets"])
    rows = np.concatenate([np.arange(offs[e], offs[e + 1]) for e in exps_gu]).astype(np.int64)
    gu_h = as_f64(host(gu)[rows]).reshape(len(rows), p.I // 32, 2, 32)  # rows >= N: unset
    check("g (saved)", gu_h[:, :, 0, :].reshape(len(rows), p.I), rg[rows])
    check("u (saved)", gu_h[:, :, 1, :].reshape(len(rows), p.I), ru[rows])
    ref = ob.layer_backward(host(inp["x"]), host(logits), host(inp["w_gate"]), host(inp["w_up"]),
                            host(inp["w_down"]), p.k, host(dy), p.capacity, p.renormalize,
                            w_router=None if wr is None else host(wr), experts=experts,
                            tokens=tokens)
    assert np.array_equal(host(routing["topk_ids"]), ref["topk_ids"])
    toks = np.arange(p.T) if tokens is None else np.asarray(tokens)
    exps = np.arange(p.E) if experts is None else np.asarray(experts)
    check("dx", as_f64(host(g["dx"]))[toks], ref["dx"][toks])
    check("dtopk_w", host(g["dtopk_w"])[toks], ref["dtopk_w"][toks])
    check("dlogits", host(g["dlogits"])[toks], ref["dlogits"][toks])
    sel = torch.as_tensor(exps, device=DEV)
    for n in ("dw_gate", "dw_up", "dw_down"):  # (only the checked experts leave the device)
        check(n, host(g[n].index_select(0, sel)), ref[n])
    if router and tokens is None:
        check("dw_router", host(g["dw_router"]), ref["dw_router"])


SMALL = [
    Workload("bwd_prefill", T=300, H=256, E=8, k=2, I=128, capacity=0, dtype="bf16",
             logits="normal", seed=71),
    Workload("bwd_cap_plain", T=200, H=128, E=4, k=2, I=192, capacity=60, dtype="bf16",
             logits="normal+zipf1.2", seed=72, renormalize=0),
    Workload("bwd_decode", T=20, H=256, E=64, k=4, I=128, capacity=0, dtype="bf16",
             logits="normal+bias0.5", seed=73),
    Workload("bwd_one_expert", T=70, H=128, E=1, k=1, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=74),
    # several 128-row gradient tiles (the last of 64 rows), column groups with idle
    # wavefronts, skewed experts with odd stage counts along their rows
    Workload("bwd_multi_tile", T=1000, H=384, E=8, k=2, I=320, capacity=0, dtype="bf16",
             logits="normal+zipf1.2", seed=76),
    # 600 rows per expert on average: the data-gradient GEMMs (and the g|u recompute) over
    # several 128-row M tiles per expert, ragged in rows and in columns (I = 192)
    Workload("bwd_many_tiles", T=1200, H=256, E=4, k=2, I=192, capacity=0, dtype="bf16",
             logits="normal", seed=77),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_backward_small(wl):
    say(f"case {wl.name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity} renorm={wl.renormalize}")
    run_case(wl)


def test_backward_with_router():
    wl = Workload("bwd_router", T=256, H=256, E=64, k=4, I=128, capacity=0, dtype="bf16",
                  logits="normal", seed=75)
    say(f"case {wl.name} (router)")
    run_case(wl, router=True)


def test_backward_rejects_what_it_does_not_handle():
    m = moe()
    p = m.Problem(T=8, H=192, E=4, k=2, I=64)  # H % 128
    w = torch.zeros(4, 192, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.MoeError) as ei:
        m.pack_weights_backward(p, w, w, w.transpose(1, 2).contiguous())
    assert ei.value.status == m.MOE_ERR_UNSUPPORTED
    x = torch.zeros(8, 192, dtype=torch.bfloat16, device=DEV)
    rt = torch.zeros(16, dtype=torch.int32, device=DEV)
    off = torch.zeros(5, dtype=torch.int32, device=DEV)
    pgu = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(m.MoeError) as ei:
        m.expert_gate_up_gather_gu(p, x, rt, off, pgu)
    assert ei.value.status == m.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["qwen3_30b_a3b", "dsv3_decode", "glm_skew_cap", "dsv3_prefill"])
def test_backward_full_size(name):
    wl = synth.WORKLOADS[name]
    say(f"case backward {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} I={wl.I} C={wl.capacity}")
    rng = np.random.default_rng(wl.seed)
    tokens = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 6, replace=False)]))
    experts = np.unique(rng.choice(wl.E, 2, replace=False))
    # dsv3_prefill: 45 GB of fp32 weight gradients per backward call, so one call
    run_case(wl, tokens=tokens, experts=experts, variants=name != "dsv3_prefill")
