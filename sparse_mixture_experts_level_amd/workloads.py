"""Seeded synthetic inputs for the sparse MoE layer forward pass.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the HIP path and the CPU oracle are fed the same
drawn tensors (the oracle receives host copies), so neither side depends on
how the values were produced.

Recipe (all layer shapes are the ones listed in ``WORKLOADS``):
  * hidden states x ~ N(0, 1);
  * router, gate and up weights ~ N(0, 1) / sqrt(d_model), down weights
    ~ N(0, 1) / sqrt(d_ff): standard deviation 1/sqrt(fan_in);
  * values are drawn in float32 by torch's generator on the requested device,
    one independently seeded stream per tensor (and per expert for the expert
    weights), then rounded to nearest-even bfloat16 for the bf16 workloads;
  * optional per-expert logit offsets create skewed expert load: +2.0 on
    experts 0..3 ("boost4"), or log of a Zipf(1.1) weight by expert rank,
    -1.1 * ln(e + 1) ("zipf1.1").

Draws depend on the device that makes them (torch's CPU and GPU generators
differ), so a workload drawn on the GPU is copied to the host for the oracle,
never redrawn there.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "MoEInputs", "make_inputs", "get_workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    d_model: int
    num_experts: int
    top_k: int
    d_ff: int
    capacity_factor: Optional[float]  # None: no capacity limit
    dtype: str  # "f32" or "bf16"
    d_ff_shared: int = 0
    offset: Optional[str] = None  # None, "boost4" or "zipf1.1"
    description: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 64, 128, 8, 2, 256, 1.25, "f32",
                 description="tiny fp32 layer: T=64, d=128, E=8, top-2, SwiGLU d_ff=256, capacity factor 1.25"),
        Workload("switch_bf16", 8192, 1024, 64, 1, 4096, 1.0, "bf16", offset="boost4",
                 description="Switch-style bf16 layer: T=8192, d=1024, E=64, top-1, d_ff=4096, capacity factor 1.0, "
                             "+2.0 logit offset on experts 0-3"),
        Workload("mixtral_bf16", 4096, 4096, 8, 2, 14336, None, "bf16",
                 description="Mixtral-shaped bf16 layer: T=4096, d=4096, E=8, top-2, d_ff=14336, no capacity limit"),
        Workload("gptoss_decode_bf16", 16, 2880, 32, 4, 2880, None, "bf16",
                 description="gpt-oss-20b-shaped bf16 decode step: T=16, d=2880, E=32, top-4, d_ff=2880, no capacity limit"),
        Workload("deepseek_v3_bf16", 16384, 7168, 256, 8, 2048, 1.25, "bf16", d_ff_shared=2048, offset="zipf1.1",
                 description="DeepSeek-V3-shaped bf16 layer: T=16384, d=7168, E=256 routed + 1 shared expert, top-8, "
                             "d_ff=2048, capacity factor 1.25, Zipf(1.1) logit offsets"),
    ]
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if overrides:
        w = Workload(**{**w.__dict__, **overrides})
    return w


@dataclass
class MoEInputs:
    workload: Workload
    x: torch.Tensor  # [T, d]
    w_router: torch.Tensor  # [E, d]
    w_gate_up: torch.Tensor  # [E, 2f, d]
    w_down: torch.Tensor  # [E, d, f]
    logit_offset: Optional[torch.Tensor]  # [E] float32 or None
    w_shared_gate_up: Optional[torch.Tensor] = None  # [2 f_s, d]
    w_shared_down: Optional[torch.Tensor] = None  # [d, f_s]
    extra: dict = field(default_factory=dict)


# Stream tags keep every tensor's draw independent of the order of generation.
_TAG_X, _TAG_ROUTER, _TAG_GATE_UP, _TAG_DOWN, _TAG_SH_GATE_UP, _TAG_SH_DOWN = 1, 2, 3, 4, 5, 6


def _gen(device, seed: int, tag: int, idx: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 10_007 + idx) & ((1 << 63) - 1))
    return g


def _normal(shape, std: float, dtype, device, seed, tag, idx=0) -> torch.Tensor:
    g = _gen(device, seed, tag, idx)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def logit_offsets(kind: Optional[str], num_experts: int) -> Optional[torch.Tensor]:
    if kind is None:
        return None
    if kind == "boost4":
        off = torch.zeros(num_experts, dtype=torch.float32)
        off[: min(4, num_experts)] = 2.0
        return off
    if kind == "zipf1.1":
        return torch.tensor([-1.1 * math.log(e + 1.0) for e in range(num_experts)], dtype=torch.float32)
    raise ValueError(kind)


def make_inputs(w: Workload, seed: int = 0, device="cpu") -> MoEInputs:
    """Draw every input tensor of workload ``w`` on ``device``."""
    dt = w.torch_dtype
    T, d, E, f = w.num_tokens, w.d_model, w.num_experts, w.d_ff
    x = _normal((T, d), 1.0, dt, device, seed, _TAG_X)
    w_router = _normal((E, d), 1.0 / math.sqrt(d), dt, device, seed, _TAG_ROUTER)
    w_gate_up = torch.empty((E, 2 * f, d), dtype=dt, device=device)
    w_down = torch.empty((E, d, f), dtype=dt, device=device)
    for e in range(E):  # one stream per expert: any expert can be redrawn alone
        w_gate_up[e] = _normal((2 * f, d), 1.0 / math.sqrt(d), dt, device, seed, _TAG_GATE_UP, e)
        w_down[e] = _normal((d, f), 1.0 / math.sqrt(f), dt, device, seed, _TAG_DOWN, e)
    off = logit_offsets(w.offset, E)
    if off is not None:
        off = off.to(device)
    sgu = sd = None
    if w.d_ff_shared:
        fs = w.d_ff_shared
        sgu = _normal((2 * fs, d), 1.0 / math.sqrt(d), dt, device, seed, _TAG_SH_GATE_UP)
        sd = _normal((d, fs), 1.0 / math.sqrt(fs), dt, device, seed, _TAG_SH_DOWN)
    return MoEInputs(w, x, w_router, w_gate_up, w_down, off, sgu, sd)
