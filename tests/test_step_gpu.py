"""One decode step end to end on the GPU, against the fp64 oracle composed the
same way: the attention prologue writes each sequence's 9 new K/V rows into a
paged cache (ShortConv, RMSNorm) and normalises q, rba_relproj projects the new
tokens' features, and the paged split-KV attention reads the cache the
prologue wrote.  The oracle runs attention_prologue, places its rows into the
cache's earlier contents, and computes the attention from those.

Tolerances as in the other bf16 parity tests: max|d| <= 2e-2, mean|d| <= 2e-3,
relative L2 <= 1e-2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_prologue_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("window,log_base,splits,max_new", [(0, 0.0, 0, 0), (256, 0.0, 3, 9), (0, 4096.0, 1, 9)])
def test_decode_step_prologue_then_paged_attention(window, log_base, splits, max_new):
    """max_new = 9 runs the prologue as one launch (the bound the step knows)."""
    import relative_position_bias_rba_amd as rba
    Hq, Hkv, d, E, r_dim, ps = 16, 2, 128, 64, 32, 64
    new = [9, 9, 9]
    lens = [300, 9, 517]                     # a sequence made of its new tokens alone, and longer ones
    Skv = 576
    B = len(new)
    inp = make_prologue_inputs(new, lens, Hq=Hq, Hkv=Hkv, W=4, seed=7)
    g = torch.Generator().manual_seed(11)
    n_pages = sum((L + ps - 1) // ps for L in lens) + 2
    perm = torch.randperm(n_pages, generator=g)
    table = torch.full((B, Skv // ps), -1, dtype=torch.int32)
    at = 0
    for b, L in enumerate(lens):
        n = (L + ps - 1) // ps
        table[b, :n] = perm[at:at + n].to(torch.int32)
        at += n
    # the cache's earlier contents (positions before each sequence's new tokens)
    k_pool = torch.randn(n_pages, ps, Hkv, d, generator=g).to(torch.bfloat16)
    v_pool = torch.randn(n_pages, ps, Hkv, d, generator=g).to(torch.bfloat16)
    r = torch.randn(B, 9, r_dim, generator=g).to(torch.bfloat16)
    P = (torch.randn(Hq, r_dim, E, generator=g) * 0.02).to(torch.bfloat16)

    dev = {k: v.to(DEV) for k, v in inp.items()}
    kp, vp, tb = k_pool.to(DEV), v_pool.to(DEV), table.to(DEV)
    q_out = rba.attn_prologue(dev["q"], dev["k"], dev["v"], dev["cu_new"], dev["seq_lens"], dev["conv_wk"],
                              dev["conv_wv"], dev["norm_q"], dev["norm_k"], dev["state_k"], dev["state_v"], kp, vp,
                              block_table=tb, max_seq_len=Skv, max_new=max_new)
    R = rba.relproj(r.to(DEV), P.to(DEV))
    o = rba.attn_paged(q_out.reshape(B, 9, Hq, d), kp, vp, tb, dev["seq_lens"], R, max_seq_len=Skv,
                       window=window, log_scale_base=log_base, num_splits=splits)
    torch.cuda.synchronize()

    q_o, k_o, v_o, pos, _, _ = oracle.attention_prologue(inp["q"], inp["k"], inp["v"], inp["cu_new"].tolist(),
                                                          lens, inp["conv_wk"], inp["conv_wv"], inp["norm_q"],
                                                          inp["norm_k"], 1e-6, inp["state_k"], inp["state_v"])
    Rw = oracle.relproj(r, P)
    worst = 0.0
    for b in range(B):
        L = lens[b]
        K = oracle.gather_pages(k_pool, table[b], L).copy()
        V = oracle.gather_pages(v_pool, table[b], L).copy()
        rows = slice(9 * b, 9 * b + 9)
        K[pos[rows]] = k_o[rows]
        V[pos[rows]] = v_o[rows]
        wo, _ = oracle.attention(q_o[rows][None], K[None], V[None], Rw[b:b + 1], window=window,
                                 log_scale_base=log_base)
        got = o[b:b + 1].double().cpu().numpy()
        diff = np.abs(got - wo)
        rel = float(np.linalg.norm(got - wo) / np.linalg.norm(wo))
        say(f"step b={b} L={L}: max|d|={diff.max():.3e} mean|d|={diff.mean():.3e} rel_l2={rel:.3e}")
        assert np.all(np.isfinite(o[b].float().cpu().numpy()))
        assert diff.max() <= 2e-2 and diff.mean() <= 2e-3, b
        assert rel <= 1e-2, b
        worst = max(worst, float(diff.max()))
    say(f"worst {worst:.3e}")
