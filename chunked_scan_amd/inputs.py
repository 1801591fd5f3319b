"""Seeded synthetic inputs for the chunked linear-attention path.

This module only draws random numbers and lays them out; it contains none of the method's
arithmetic, so both the GPU path and the CPU oracle may consume what it produces.  Shapes,
value distributions and seeds are those of the five workloads below (the per-device shape of
the ZeCO operator runs -- 16k tokens per device, 16 heads, head dim 128 -- is the one the review
page "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear Attention" gives in
skeptic_critique.concrete_test; no public dataset is involved).

Draw order is fixed: q, k, v, then the decay parameter, then s_in.  q, k, v are drawn in
float32 and rounded once (round-to-nearest-even) to the storage dtype before anyone sees them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    dk: int
    dv: int
    chunk: int
    nseg: int
    dtype: str          # "f32" or "bf16" (q, k, v and o)
    decay: str          # "none" | "head_uniform" | "head_pow2" | "gate"
    qkv_std: float      # q, k, v ~ N(0, 1) * qkv_std
    s_in_std: float     # s_in ~ N(0, s_in_std); 0 means no initial state
    seed: int
    gate_norm: float = 16.0

    @property
    def mode(self) -> str:
        return {"none": "none", "head_uniform": "head", "head_pow2": "head", "gate": "gate"}[self.decay]

    @property
    def tokens(self) -> int:
        return self.B * self.L

    def scaled(self, **kw) -> "Workload":
        """The same recipe at other sizes (tests use this for oracle-sized cases)."""
        return replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 check: per-head scalar decay a = exp(-u), u ~ U(0.01, 0.1), one u per head.
    0: Workload("tiny_fp32_head_decay", 1, 2, 256, 16, 16, 64, 1, "f32", "head_uniform",
                1.0 / math.sqrt(16), 0.1, 0),
    # Plain (ungated) causal linear attention at the per-device shape.
    1: Workload("plain_B1_H16_L16k_d128", 1, 16, 16384, 128, 128, 64, 1, "bf16", "none",
                1.0 / math.sqrt(128), 0.0, 1),
    # Scalar per-head decay lambda_h = -2^-(5 + 8h/H) with a random incoming state.
    2: Workload("head_decay_B2_H16_L16k_d128", 2, 16, 16384, 128, 128, 64, 1, "bf16", "head_pow2",
                1.0 / math.sqrt(128), 0.05, 2),
    # GLA-style gate: a = sigmoid(g)^(1/16) per token and key dim, g ~ N(0, 1) stored fp32.
    3: Workload("gla_gate_B4_H16_L16k_d128", 4, 16, 16384, 128, 128, 64, 1, "bf16", "gate",
                1.0 / math.sqrt(128), 0.0, 3),
    # One GPU standing in for 64 devices: 2^20 tokens cut into 64 segments of 16384.
    4: Workload("segmented_1M_P64_H16_d128", 1, 16, 1 << 20, 128, 128, 64, 64, "bf16", "head_pow2",
                1.0 / math.sqrt(128), 0.0, 4),
}


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_inputs(w: Workload, device: str = "cpu", seed: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``w`` on ``device`` with a generator of that device.

    Returns dict(q, k, v, decay, s_in) of torch tensors: q, k [B,H,L,dk]; v [B,H,L,dv] in the
    storage dtype; decay None (no decay), [H] float32 log-decay (per-head modes) or
    [B,H,L,dk] float32 raw gate (gate mode); s_in [B,H,dk,dv] float32 or None.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w)

    def normal(shape, std):
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        return x

    q = normal((w.B, w.H, w.L, w.dk), w.qkv_std).to(dt)
    k = normal((w.B, w.H, w.L, w.dk), w.qkv_std).to(dt)
    v = normal((w.B, w.H, w.L, w.dv), w.qkv_std).to(dt)
    if w.decay == "none":
        decay = None
    elif w.decay == "head_uniform":
        u = torch.rand((w.H,), generator=g, device=dev, dtype=torch.float32) * 0.09 + 0.01
        decay = -u
    elif w.decay == "head_pow2":
        h = torch.arange(w.H, device=dev, dtype=torch.float64)
        decay = (-torch.pow(2.0, -(5.0 + 8.0 * h / w.H))).to(torch.float32)
    elif w.decay == "gate":
        decay = normal((w.B, w.H, w.L, w.dk), 1.0)
    else:
        raise ValueError(w.decay)
    s_in = normal((w.B, w.H, w.dk, w.dv), w.s_in_std) if w.s_in_std > 0 else None
    return dict(q=q, k=k, v=v, decay=decay, s_in=s_in)


def make_grads(w: Workload, nseg: int = 1, device: str = "cpu", seed: Optional[int] = None,
               ds_out_std: float = 1.0) -> dict:
    """Draw the incoming derivatives of a backward pass for workload ``w``: d_o [B,H,L,dv] ~ N(0, 1)
    in the storage dtype and ds_out [B,H,nseg,dk,dv] ~ N(0, ds_out_std) float32 (None when
    ds_out_std is 0), from their own generator (default seed: the workload's seed + 1000)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed((w.seed + 1000) if seed is None else seed)
    d_o = torch.randn((w.B, w.H, w.L, w.dv), generator=g, device=dev, dtype=torch.float32).to(torch_dtype(w))
    ds_out = None
    if ds_out_std > 0:
        ds_out = torch.randn((w.B, w.H, nseg, w.dk, w.dv), generator=g, device=dev, dtype=torch.float32)
        ds_out.mul_(ds_out_std)
    return dict(d_o=d_o, ds_out=ds_out)
