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


def make_paged_inputs(w: Workload, page_size: int, seq_lens=None, seed: int | None = None,
                      spare_pages: int = 3) -> dict:
    """CPU tensors for a paged KV cache with ``w``'s shapes.

    q, r, P as in ``make_inputs``.  Sequence b holds seq_lens[b] keys (drawn
    uniformly from [Sq, Skv] unless given); its pages are distinct pages of a
    shared pool, assigned in a random order:
      k_pool, v_pool : [num_pages, page_size, Hkv, d]
      block_table    : int32 [B, ceil(Skv / page_size)]; entries past a
                       sequence's last page are -1
      seq_lens       : int32 [B]
    The pool holds ``spare_pages`` pages that no sequence uses.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = randn((w.B, w.Sq, w.Hq, w.d), g, w.qk_std)
    if seq_lens is None:
        lens = torch.randint(w.Sq, w.Skv + 1, (w.B,), generator=g, dtype=torch.int64)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    need = [(int(n) + page_size - 1) // page_size for n in lens]
    n_pages = sum(need) + spare_pages
    perm = torch.randperm(n_pages, generator=g)
    n_max = (w.Skv + page_size - 1) // page_size
    table = torch.full((w.B, n_max), -1, dtype=torch.int32)
    at = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[at:at + n].to(torch.int32)
        at += n
    k_pool = randn((n_pages, page_size, w.Hkv, w.d), g, w.qk_std)
    v_pool = randn((n_pages, page_size, w.Hkv, w.d), g, w.v_std)
    r = randn((w.B, w.Sq, w.r_dim), g, w.r_std)
    P = randn((w.Hq, w.r_dim, w.E), g, w.p_std)
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    out = {n: t.to(dt) for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("r", r), ("P", P))}
    out["block_table"] = table
    out["seq_lens"] = lens.to(torch.int32)
    return out


def make_prologue_inputs(new_tokens, seq_lens, Hq=64, Hkv=8, d=128, W=4, seed=2001) -> dict:
    """CPU tensors for one attention-prologue call: B sequences receiving
    new_tokens[b] tokens, ending at lengths seq_lens[b].

      q, k, v      : bf16 [T, Hq|Hkv, d] ~ N(0, 1) (projections)
      conv_wk/wv   : fp32 [Hkv*d, W] ~ N(0, 1/W) (taps)
      norm_q/k     : fp32 [d] ~ 1 + N(0, 0.1) (RMSNorm weights)
      state_k/v    : bf16 [B, W-1, Hkv, d] ~ N(0, 1), zero for positions
                     before a sequence's start
      cu_new       : int32 [B+1], seq_lens int32 [B]
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    T = int(sum(new_tokens))
    B = len(new_tokens)
    q = randn((T, Hq, d), g).to(torch.bfloat16)
    k = randn((T, Hkv, d), g).to(torch.bfloat16)
    v = randn((T, Hkv, d), g).to(torch.bfloat16)
    wk = randn((Hkv * d, W), g, (1.0 / W) ** 0.5)
    wv = randn((Hkv * d, W), g, (1.0 / W) ** 0.5)
    nq = 1.0 + randn((d,), g, 0.1)
    nk = 1.0 + randn((d,), g, 0.1)
    sk = randn((B, max(W - 1, 0), Hkv, d), g).to(torch.bfloat16)
    sv = randn((B, max(W - 1, 0), Hkv, d), g).to(torch.bfloat16)
    for b in range(B):
        start = int(seq_lens[b]) - int(new_tokens[b])
        for j in range(W - 1):
            if start - (W - 1) + j < 0:
                sk[b, j] = 0
                sv[b, j] = 0
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.as_tensor(new_tokens, dtype=torch.int64), 0).to(torch.int32)
    return {"q": q, "k": k, "v": v, "conv_wk": wk, "conv_wv": wv, "norm_q": nq, "norm_k": nk,
            "state_k": sk, "state_v": sv, "cu_new": cu, "seq_lens": torch.as_tensor(seq_lens, dtype=torch.int32)}
