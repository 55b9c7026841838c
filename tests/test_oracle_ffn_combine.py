"""Pins for the expert SwiGLU FFN and the weighted combine.

Special cases that reduce the MoE layer to a textbook dense SwiGLU MLP (numpy fp64
matmul), plus exact algebraic properties (x = 0, scaling W_down by 2, a single expert
with non-zero W_down, k = 1, every slot of a token dropped).
"""
import numpy as np
import pytest

import oracle


def mlp64(x, wg, wu, wd):
    """Dense SwiGLU MLP: (silu(x Wg) * (x Wu)) Wd in fp64 (numpy matmul)."""
    x = x.astype(np.float64)
    g = x @ wg.astype(np.float64)
    u = x @ wu.astype(np.float64)
    return (g / (1.0 + np.exp(-g)) * u) @ wd.astype(np.float64)


def weights(rng, E, H, I):
    wg = (rng.standard_normal((E, H, I)) / np.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, H, I)) / np.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, I, H)) / np.sqrt(I)).astype(np.float32)
    return wg, wu, wd


def to_bf16_bits(a):
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def from_bf16_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def close(a, b, rtol=1e-12):
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() <= rtol * scale


def test_single_expert_top1_is_dense_mlp():
    rng = np.random.default_rng(1)
    T, H, I = 37, 16, 24
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu, wd = weights(rng, 1, H, I)
    out = oracle.layer(x, np.zeros((T, 1), np.float32), wg, wu, wd, k=1)
    assert close(out["y"], mlp64(x, wg[0], wu[0], wd[0]))
    # the intermediate activation is silu(g) * u
    g = x.astype(np.float64) @ wg[0].astype(np.float64)
    a = g / (1 + np.exp(-g)) * (x.astype(np.float64) @ wu[0].astype(np.float64))
    assert close(out["a"], a)


def test_bf16_inputs_are_upcast_exactly():
    rng = np.random.default_rng(2)
    T, H, I = 19, 32, 16
    xb = to_bf16_bits(rng.standard_normal((T, H)))
    wg, wu, wd = (to_bf16_bits(w) for w in weights(rng, 1, H, I))
    out = oracle.layer(xb, np.zeros((T, 1), np.float32), wg, wu, wd, k=1)
    ref = mlp64(from_bf16_bits(xb), from_bf16_bits(wg[0]), from_bf16_bits(wu[0]), from_bf16_bits(wd[0]))
    assert close(out["y"], ref)


def test_identical_experts_give_the_dense_mlp_whatever_the_routing():
    rng = np.random.default_rng(3)
    T, H, I, E, k = 50, 16, 24, 6, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg1, wu1, wd1 = weights(rng, 1, H, I)
    wg, wu, wd = (np.repeat(w, E, axis=0) for w in (wg1, wu1, wd1))
    out = oracle.layer(x, rng.standard_normal((T, E)).astype(np.float32), wg, wu, wd, k=k)
    # sum_j w_j = 1 up to 4k fp32 roundings
    assert close(out["y"], mlp64(x, wg1[0], wu1[0], wd1[0]), rtol=8 * k * 2.0 ** -24)


def test_top1_uses_the_chosen_experts_mlp():
    rng = np.random.default_rng(4)
    T, H, I, E = 40, 8, 16, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu, wd = weights(rng, E, H, I)
    l = rng.standard_normal((T, E)).astype(np.float32)
    out = oracle.layer(x, l, wg, wu, wd, k=1)
    assert np.all(out["topk_w"] == 1.0)
    for t in range(T):
        e = int(np.argmax(l[t]))
        assert close(out["y"][t], mlp64(x[t:t + 1], wg[e], wu[e], wd[e])[0])


def test_one_live_expert_gets_its_slot_weight():
    # W_down zero for every expert but one: y[t] = w[t, slot of e*] * MLP_e*(x[t])
    rng = np.random.default_rng(5)
    T, H, I, E, k, es = 60, 8, 12, 4, 2, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu, wd = weights(rng, E, H, I)
    wd[np.arange(E) != es] = 0.0
    out = oracle.layer(x, rng.standard_normal((T, E)).astype(np.float32), wg, wu, wd, k=k)
    ref_full = mlp64(x, wg[es], wu[es], wd[es])
    for t in range(T):
        slots = np.nonzero(out["topk_ids"][t] == es)[0]
        ref = ref_full[t] * float(out["topk_w"][t, slots[0]]) if slots.size else np.zeros(H)
        assert np.abs(out["y"][t] - ref).max() <= 1e-12 * max(1.0, np.abs(ref_full[t]).max())


def test_zero_input_gives_zero_and_down_scaling_is_exact():
    rng = np.random.default_rng(6)
    T, H, I, E, k = 30, 8, 8, 4, 2
    wg, wu, wd = weights(rng, E, H, I)
    l = rng.standard_normal((T, E)).astype(np.float32)
    out0 = oracle.layer(np.zeros((T, H), np.float32), l, wg, wu, wd, k=k)
    assert np.all(out0["y"] == 0.0)
    x = rng.standard_normal((T, H)).astype(np.float32)
    a = oracle.layer(x, l, wg, wu, wd, k=k)["y"]
    b = oracle.layer(x, l, wg, wu, (wd * 2).astype(np.float32), k=k)["y"]
    assert np.array_equal(b, 2 * a)


def test_fully_dropped_token_outputs_zero():
    T, H, I, E, k, C = 12, 8, 8, 3, 1, 4
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu, wd = weights(rng, E, H, I)
    l = np.zeros((T, E), np.float32)
    l[:, 1] = 1.0  # all tokens want expert 1, equal weights: tokens >= C are dropped
    out = oracle.layer(x, l, wg, wu, wd, k=k, capacity_=C)
    assert np.all(out["y"][C:] == 0.0)
    assert close(out["y"][:C], mlp64(x[:C], wg[1], wu[1], wd[1]))


def test_combine_respects_slot_to_row():
    # a direct check of the combine formula on hand-built maps
    yp = np.arange(12, dtype=np.float64).reshape(4, 3)
    w = np.array([[0.5, 0.25], [1.0, 0.0]], np.float32)
    s2r = np.array([[2, 0], [3, -1]], np.int32)
    y = oracle.combine(np.array([0, 1]), w, s2r, yp)
    assert np.array_equal(y, np.array([0.5 * yp[2] + 0.25 * yp[0], yp[3]]))
