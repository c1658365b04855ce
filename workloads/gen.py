"""Seeded input draws.  Random numbers only; none of the method's arithmetic.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws, in
this fixed order and in fp32, q, k, v, r and P from normal distributions with
the workload's standard deviations; bf16 workloads then round every tensor to
bf16 (round-to-nearest-even).  The oracle upcasts exactly these values.
"""
from __future__ import annotations

import torch

from .configs import Workload


def randn(shape, gen: torch.Generator, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Return CPU tensors q, k, v, r, P in the workload's dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = randn((w.B, w.Sq, w.Hq, w.d), g, w.qk_std)
    k = randn((w.B, w.Skv, w.Hkv, w.d), g, w.qk_std)
    v = randn((w.B, w.Skv, w.Hkv, w.d), g, w.v_std)
    r = randn((w.B, w.Sq, w.r_dim), g, w.r_std)
    P = randn((w.Hq, w.r_dim, w.E), g, w.p_std)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    return {n: t.to(dt) for n, t in (("q", q), ("k", k), ("v", v), ("r", r), ("P", P))}
