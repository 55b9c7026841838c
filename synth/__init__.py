"""Seeded synthetic inputs for the MoE layer workloads.

This module only draws random numbers; it holds none of the layer's arithmetic
(no routing, no softmax, no matmul).  The same tensors feed the HIP path and the
CPU oracle: a caller generates once and copies to the other side, so both see the
same bytes.

Distributions (readings of the workload descriptions, documented with the tests):
  * x ~ N(0, 1); router logits ~ N(0, 1) in fp32, plus a per-expert bias where the
    workload asks for load imbalance (added into the logits: the logits are an input).
  * W_gate, W_up: [E, H, I]; W_down: [E, I, H]; N(0, sigma = 1/sqrt(fan_in)) with
    fan_in = H for gate/up and I for down.
  * bf16 tensors are drawn in fp32 and rounded to bf16 (round to nearest even).
  * "fp8" workloads draw the same bf16 tensors; the FP8 weights are their quantisation
    (done by the path under test and, separately, by the oracle).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    capacity: int  # <= 0: no cap
    dtype: str  # "f32" or "bf16" (activations and weights), "fp8" (bf16 activations)
    logits: str  # recipe name, see make_logits
    seed: int
    renormalize: int = 1
    note: str = ""

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == F32 else torch.bfloat16  # activations

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes measured and parity-tested.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", T=256, H=128, E=8, k=2, I=256, capacity=0, dtype=F32,
                         logits="normal", seed=1,
                         note="tiny fp32 MoE layer, no cap"),
    "qwen3_30b_a3b": Workload("qwen3_30b_a3b", T=4096, H=2048, E=128, k=8, I=768, capacity=0,
                              dtype=BF16, logits="normal+bias0.5", seed=2,
                              note="Qwen3-30B-A3B-shaped layer, mild imbalance, no cap"),
    "glm_skew_cap": Workload("glm_skew_cap", T=8192, H=4096, E=64, k=4, I=1408, capacity=1024,
                             dtype=BF16, logits="normal+zipf1.2", seed=3,
                             note="GLM-style skewed routing with per-expert capacity 1024"),
    "dsv3_prefill": Workload("dsv3_prefill", T=16384, H=7168, E=256, k=8, I=2048, capacity=0,
                             dtype=BF16, logits="normal", seed=4,
                             note="DeepSeek-V3-shaped prefill layer"),
    "dsv3_decode": Workload("dsv3_decode", T=128, H=7168, E=256, k=8, I=2048, capacity=0,
                            dtype=BF16, logits="normal", seed=5,
                            note="DeepSeek-V3-shaped decode batch, weight-streaming bound"),
}
# The bf16 layer shapes with FP8 expert weights (same seeds, so the same bf16 draws).
for _n in ("qwen3_30b_a3b", "glm_skew_cap", "dsv3_prefill", "dsv3_decode"):
    WORKLOADS[_n + "_fp8"] = WORKLOADS[_n].replace(name=_n + "_fp8", dtype=FP8)


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    # distinct, reproducible stream per (seed, tensor)
    g.manual_seed((seed * 1_000_003 + stream * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def make_logits(wl: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Router logits [T, E] fp32 following the workload's recipe."""
    T = wl.T if T is None else T
    E = wl.E
    g = _gen(device, wl.seed, 1)
    recipe = wl.logits
    if recipe == "ties012":
        # tie-heavy: integer-valued logits in {0, 1, 2}
        return torch.randint(0, 3, (T, E), generator=g, device=device).to(torch.float32)
    if recipe == "all_to_one":
        # every token ranks expert 0 first (then a random order): worst-case skew
        lg = torch.randn(T, E, generator=g, device=device, dtype=torch.float32)
        lg[:, 0] = 100.0
        return lg
    if recipe == "equal":
        return torch.zeros(T, E, device=device, dtype=torch.float32)
    lg = torch.randn(T, E, generator=g, device=device, dtype=torch.float32)
    gb = _gen(device, wl.seed, 2)
    if recipe == "normal":
        return lg
    if recipe == "normal+bias0.5":
        bias = torch.randn(E, generator=gb, device=device, dtype=torch.float32) * 0.5
        return lg + bias[None, :]
    if recipe == "normal+zipf1.2":
        # Zipf(s=1.2) over experts: expert with popularity rank r gets bias -1.2*ln(r),
        # so exp(bias) is proportional to r^-1.2; ranks are a seeded permutation of 1..E.
        ranks = torch.randperm(E, generator=gb, device=device).to(torch.float32) + 1.0
        bias = -1.2 * torch.log(ranks)
        return lg + bias[None, :]
    raise ValueError(f"unknown logits recipe {recipe!r}")


def make_x(wl: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    T = wl.T if T is None else T
    g = _gen(device, wl.seed, 3)
    return torch.randn(T, wl.H, generator=g, device=device, dtype=torch.float32).to(wl.torch_dtype)


def make_weights(wl: Workload, device="cpu", experts: Optional[range] = None):
    """(W_gate [E,H,I], W_up [E,H,I], W_down [E,I,H]) in the workload dtype.

    Drawn expert by expert (bounded temporaries); expert e always gets the same values
    whatever subset is requested, so a slice can be regenerated elsewhere.
    """
    E, H, I = wl.E, wl.H, wl.I
    experts = range(E) if experts is None else experts
    dt = wl.torch_dtype
    n = len(experts)
    wg = torch.empty(n, H, I, device=device, dtype=dt)
    wu = torch.empty(n, H, I, device=device, dtype=dt)
    wd = torch.empty(n, I, H, device=device, dtype=dt)
    sg = 1.0 / math.sqrt(H)
    sd = 1.0 / math.sqrt(I)
    for i, e in enumerate(experts):
        g = _gen(device, wl.seed, 100 + 3 * e)
        wg[i] = (torch.randn(H, I, generator=g, device=device, dtype=torch.float32) * sg).to(dt)
        g = _gen(device, wl.seed, 101 + 3 * e)
        wu[i] = (torch.randn(H, I, generator=g, device=device, dtype=torch.float32) * sg).to(dt)
        g = _gen(device, wl.seed, 102 + 3 * e)
        wd[i] = (torch.randn(I, H, generator=g, device=device, dtype=torch.float32) * sd).to(dt)
    return wg, wu, wd


def make_router_weights(wl: Workload, device="cpu") -> torch.Tensor:
    """Gate weights W_r [E, H] ~ N(0, 1/sqrt(H)) in bf16, so that x W_r^T has logits of
    order 1 like the logits recipes."""
    g = _gen(device, wl.seed, 4)
    return (torch.randn(wl.E, wl.H, generator=g, device=device, dtype=torch.float32)
            / math.sqrt(wl.H)).to(torch.bfloat16)


def make_inputs(wl: Workload, device="cpu"):
    """All inputs of one layer call: dict(x, logits, w_gate, w_up, w_down)."""
    wg, wu, wd = make_weights(wl, device)
    return dict(x=make_x(wl, device), logits=make_logits(wl, device), w_gate=wg, w_up=wu, w_down=wd)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 tensor's bits (host copy)."""
    import numpy as np

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
