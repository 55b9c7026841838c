"""GPU parity of the routing front-end: group-limited top-k (moe_route_grouped) and the
router GEMM with the selection fused after it (moe_router), against the oracle.

Bar:
  * selection, weights, keep flags from given logits: bit-exact (ids, weight bits, keep);
  * router logits: |gpu - exact| <= H * 2^-24 * sum_h |x[t,h] w[e,h]| (bf16 products are
    exact in fp32; the bound is the worst case of fp32 summation over H terms) against
    the oracle's fp64 logits;
  * the selection moe_router takes is exactly the oracle's rule applied to the fp32 logits
    it computed (checked bit for bit on every token); against the selection from the exact
    logits it may differ only where the exact logits tie within the bound above, so at
    least 95% of tokens must agree (a sanity check; validity rests on the two above).
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


def check_selection(p, logits_f32, n_group, topk_group, ids, w, keep):
    rid, rw = oracle.route_grouped(logits_f32, p.k, n_group, topk_group, p.renormalize)
    assert np.array_equal(host(ids), rid), "topk_ids"
    assert np.array_equal(host(w).view(np.uint32), rw.view(np.uint32)), "topk_w bits"
    rkeep = oracle.capacity(rid, rw, p.E, p.capacity)
    assert np.array_equal(host(keep), rkeep), "keep"
    return rid


GROUPED = [
    # (T, E, k, n_group, topk_group, renormalize, capacity, logits recipe)
    (1000, 256, 8, 8, 4, 1, 0, "normal"),
    (1000, 256, 8, 8, 4, 0, 0, "normal"),
    (777, 64, 6, 8, 3, 1, 100, "normal+zipf1.2"),
    (500, 160, 4, 32, 2, 1, 0, "ties012"),
    (300, 1024, 32, 64, 16, 1, 0, "normal"),
    (257, 8, 2, 4, 1, 1, 0, "equal"),
    (129, 128, 8, 1, 1, 1, 0, "normal"),          # one group: plain top-k
    (65, 96, 8, 3, 3, 0, 0, "normal"),            # every group taken
]


@pytest.mark.parametrize("case", GROUPED, ids=[f"T{c[0]}_E{c[1]}_k{c[2]}_g{c[3]}_{c[4]}_r{c[5]}_C{c[6]}_{c[7]}"
                                               for c in GROUPED])
def test_route_grouped_bit_exact(case):
    T, E, k, n_group, topk_group, renorm, cap, recipe = case
    say(f"case grouped {case}")
    m = moe()
    wl = Workload("grouped", T=T, H=64, E=E, k=k, I=64, capacity=cap, dtype="bf16",
                  logits=recipe, seed=T + E, renormalize=renorm)
    p = m.Problem.of(wl)
    logits = synth.make_logits(wl, DEV)
    ids, w, keep = m.route_grouped(p, logits, n_group, topk_group)
    torch.cuda.synchronize()
    check_selection(p, host(logits), n_group, topk_group, ids, w, keep)


def make_router_inputs(wl, device):
    """x [T, H] and W_r [E, H] ~ N(0, 1/sqrt(H)) in bf16 (logits of order 1)."""
    return synth.make_x(wl, device), synth.make_router_weights(wl, device)


def check_router(p, x, wr, n_group, topk_group, tokens=None):
    m = moe()
    ids, w, keep, logits = m.router(p, x, wr, n_group, topk_group, want_logits=True)
    ids2, w2, keep2, _ = m.router(p, x, wr, n_group, topk_group)      # without logits out
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(keep, keep2)
    lg = host(logits)
    rid = check_selection(p, lg, n_group, topk_group, ids, w, keep)
    tokens = np.arange(p.T) if tokens is None else np.asarray(tokens)
    xs, wh = host(x)[tokens], host(wr)
    exact = oracle.router_logits(xs, wh)
    xf = (xs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (wh.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = p.H * 2.0 ** -24 * (np.abs(xf) @ np.abs(wf).T) + 1e-30
    err = np.abs(lg[tokens] - exact)
    say(f"  logits: max err {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.all(err <= bound)
    eid, _ = oracle.route_grouped(exact.astype(np.float32), p.k, n_group, topk_group,
                                  p.renormalize)
    same = np.mean(np.all(eid == rid[tokens], axis=1))
    say(f"  tokens whose selection equals the exact logits' selection: {same:.5f}")
    # validity is established above (exact rule on logits within the bound); this is a
    # sanity check against gross errors (slot order counts, so near-ties among the top k
    # also show up here)
    assert same >= 0.95


ROUTER = [
    # name, T, H, E, k, n_group, topk_group, capacity
    ("small_e16", 100, 64, 16, 2, 1, 1, 0),
    ("ragged_e48", 1000, 256, 48, 4, 4, 2, 0),
    ("e128", 513, 512, 128, 8, 1, 1, 0),
    ("e256_grouped", 300, 1024, 256, 8, 8, 4, 0),
    ("e64_cap", 2000, 256, 64, 4, 1, 1, 100),
    # multiples of 32 that are not of 64: staged gate pieces not a multiple of the threads
    ("e32", 70, 64, 32, 4, 1, 1, 0),
    ("e96", 333, 192, 96, 6, 3, 2, 0),
    ("e224_grouped", 1000, 128, 224, 8, 8, 4, 0),
]


@pytest.mark.parametrize("case", ROUTER, ids=[c[0] for c in ROUTER])
def test_router_small(case):
    name, T, H, E, k, n_group, topk_group, cap = case
    say(f"case router {case}")
    m = moe()
    wl = Workload(name, T=T, H=H, E=E, k=k, I=64, capacity=cap, dtype="bf16", logits="normal",
                  seed=T + H + E)
    p = m.Problem.of(wl)
    x, wr = make_router_inputs(wl, DEV)
    check_router(p, x, wr, n_group, topk_group)


def test_router_rejects_what_it_does_not_handle():
    m = moe()
    p = m.Problem(T=8, H=64, E=320, k=2, I=64)
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.MoeError) as ei:
        m.router(p, x, torch.zeros(320, 64, dtype=torch.bfloat16, device=DEV))
    assert ei.value.status == m.MOE_ERR_UNSUPPORTED
    p = m.Problem(T=8, H=64, E=64, k=8, I=64)
    with pytest.raises(m.MoeError) as ei:  # k = 8 does not fit in 1 group of 4 experts
        m.router(p, x, torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV), 16, 1)
    assert ei.value.status == m.MOE_ERR_INVALID_ARG


# the three routed layer shapes, with the gate computed from x (DeepSeek-V3-style groups on
# the 256-expert shape)
FULL = [("qwen3_30b_a3b", 1, 1), ("glm_skew_cap", 1, 1), ("dsv3_prefill", 8, 4),
        ("dsv3_decode", 8, 4)]


@pytest.mark.parametrize("name,n_group,topk_group", FULL, ids=[f[0] for f in FULL])
def test_router_full_size(name, n_group, topk_group):
    wl = synth.WORKLOADS[name]
    say(f"case router {name}: T={wl.T} H={wl.H} E={wl.E} k={wl.k} C={wl.capacity} groups {n_group}/{topk_group}")
    m = moe()
    p = m.Problem.of(wl)
    x, wr = make_router_inputs(wl, DEV)
    rng = np.random.default_rng(wl.seed)
    tokens = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, min(wl.T, 200), replace=False)]))
    check_router(p, x, wr, n_group, topk_group, tokens=tokens)
