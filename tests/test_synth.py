"""The seeded input generator: reproducible, with the distributions the workloads name."""
import numpy as np
import torch

import oracle
import synth


def test_reproducible():
    wl = synth.WORKLOADS["tiny_f32"]
    a = synth.make_inputs(wl)
    b = synth.make_inputs(wl)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_shapes_and_moments():
    wl = synth.WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(wl)
    assert inp["x"].shape == (256, 128) and inp["logits"].shape == (256, 8)
    assert inp["w_gate"].shape == (8, 128, 256) and inp["w_down"].shape == (8, 256, 128)
    assert abs(inp["x"].std().item() - 1.0) < 0.02
    assert abs(inp["w_gate"].std().item() * np.sqrt(128) - 1.0) < 0.02
    assert abs(inp["w_down"].std().item() * np.sqrt(256) - 1.0) < 0.02


def test_expert_subset_regenerates_the_same_values():
    wl = synth.WORKLOADS["tiny_f32"]
    full = synth.make_weights(wl)
    sub = synth.make_weights(wl, experts=range(3, 5))
    for f, s in zip(full, sub):
        assert torch.equal(f[3:5], s)


def test_zipf_skew_overflows_several_experts():
    wl = synth.WORKLOADS["glm_skew_cap"]
    lg = synth.make_logits(wl).numpy()
    ids, w = oracle.route(lg, wl.k)
    counts = np.bincount(ids.ravel(), minlength=wl.E)
    assert (counts > wl.capacity).sum() >= 4
    keep = oracle.capacity(ids, w, wl.E, wl.capacity)
    assert 10_000 < keep.sum() < 20_000
