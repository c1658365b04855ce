"""GPU parity of the attention prologue (rba_attn_prologue: K/V ShortConv,
Q/K RMSNorm, KV-cache write, conv-state update) against the fp64 oracle.

bf16 outputs: |got - want| <= 2^-8 |want| + 1e-5 (one bf16 rounding of an fp32
result).  The conv state holds copies of bf16 inputs: bit-exact.  Cache rows
the call must not touch keep their sentinel value bit for bit.  The MXFP8
cache equals the library's encoder applied to the bf16 cache the same call
writes (bit-exact), and decodes to within the E4M3 step of the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_prologue_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 0.3125        # exact in bf16


def rba():
    import relative_position_bias_rba_amd as m  # fails loudly if librba.so is missing
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def close(name, got, want):
    g = got.detach().double().cpu().numpy()
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    d = np.abs(g - w)
    say(f"[{name}] max|d|={d.max():.3e} max rel={np.max(d / (np.abs(w) + 1e-6)):.3e}")
    bad = d > 2.0 ** -8 * np.abs(w) + 1e-5
    assert not bad.any(), f"{name}: {bad.sum()} entries off, first {np.argwhere(bad)[:3].tolist()}"


def run(inp, Skv, *, f8=False, paged=None, W=None, head_major=False, max_new=0):
    """head_major: the dense cache is stored [B, Hkv, Skv, ...] and passed as a
    [B, Skv, Hkv, ...] view with those strides.  max_new: the bound on new tokens
    per sequence passed to the library (0: none; 1..32 selects the one-launch
    path, which must stay exact when a sequence exceeds the bound)."""
    m = rba()
    d = {k: v.to(DEV) for k, v in inp.items()}
    B = d["seq_lens"].shape[0]
    Hkv = d["k"].shape[1]

    def cache(shape, fill, dtype):
        if not head_major:
            return torch.full(shape, fill, dtype=dtype, device=DEV)
        return torch.full((shape[0], shape[2], shape[1], shape[3]), fill, dtype=dtype, device=DEV).transpose(1, 2)

    if paged is None:
        kc = cache((B, Skv, Hkv, 128), SENTINEL, torch.bfloat16)
        vc = cache((B, Skv, Hkv, 128), -SENTINEL, torch.bfloat16)
        table = None
    else:
        ps, n_pages, table = paged
        kc = torch.full((n_pages, ps, Hkv, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
        vc = torch.full_like(kc, -SENTINEL)
        table = table.to(DEV)
    ks = vs = None
    if f8:
        kc = cache(tuple(kc.shape), 0x55, torch.uint8)
        vc = cache(tuple(vc.shape), 0x66, torch.uint8)
        ks = cache((*kc.shape[:3], 4), 0x11, torch.uint8)
        vs = cache((*kc.shape[:3], 4), 0x22, torch.uint8)
    sk, sv = d["state_k"].clone(), d["state_v"].clone()
    qo = m.attn_prologue(d["q"], d["k"], d["v"], d["cu_new"], d["seq_lens"], d["conv_wk"], d["conv_wv"],
                         d["norm_q"], d["norm_k"], sk if sk.numel() else None, sv if sv.numel() else None, kc, vc,
                         eps=1e-6, k_scale=ks, v_scale=vs, block_table=table, max_seq_len=Skv if paged else None,
                         max_new=max_new)
    torch.cuda.synchronize()
    return qo, kc, vc, ks, vs, sk, sv


def oracle_of(inp):
    return oracle.attention_prologue(inp["q"], inp["k"], inp["v"], inp["cu_new"].tolist(), inp["seq_lens"].tolist(),
                                     inp["conv_wk"], inp["conv_wv"], inp["norm_q"], inp["norm_k"], 1e-6,
                                     inp["state_k"], inp["state_v"])


def seq_of(inp):
    cu = inp["cu_new"].tolist()
    return np.concatenate([[b] * (cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]).astype(int)


# decode (1 new token), MTP verify (9), a prefill chunk from position 0 (37),
# a chunk in the middle (20), a sequence shorter than the taps (2 tokens from 0)
MIX = dict(new=[1, 9, 37, 20, 2], lens=[500, 9, 37, 100, 2])


@pytest.mark.parametrize("max_new", [0, 32, 1], ids=["chunked", "one_launch", "bound_exceeded"])
@pytest.mark.parametrize("W", [4, 2, 1])
def test_prologue_dense_bf16(W, max_new):
    say(f"prologue dense W={W} max_new={max_new}")
    inp = make_prologue_inputs(MIX["new"], MIX["lens"], Hq=16, Hkv=2, W=W)
    qo, kc, vc, _, _, sk, sv = run(inp, 512, max_new=max_new)
    q_o, k_o, v_o, pos, nsk, nsv = oracle_of(inp)
    close("q_out", qo, q_o)
    bs = seq_of(inp)
    close("k rows", kc[bs, pos], k_o)
    close("v rows", vc[bs, pos], v_o)
    # every other cache row keeps its sentinel
    mask = torch.ones(kc.shape[:2], dtype=torch.bool)
    mask[bs, pos] = False
    assert torch.all(kc[mask.to(DEV)] == SENTINEL) and torch.all(vc[mask.to(DEV)] == -SENTINEL)
    if W > 1:
        assert np.array_equal(sk.double().cpu().numpy(), nsk) and np.array_equal(sv.double().cpu().numpy(), nsv)


@pytest.mark.parametrize("f8", [False, True], ids=["bf16", "mxfp8"])
def test_prologue_head_major_cache(f8):
    # the dense cache stored head-major: the same rows land at the strided
    # addresses, every other entry keeps its fill
    say(f"prologue head-major cache f8={f8}")
    inp = make_prologue_inputs(MIX["new"], MIX["lens"], Hq=16, Hkv=2, W=4, seed=23)
    got = run(inp, 512, f8=f8, head_major=True)
    ref = run(inp, 512, f8=f8)
    assert not got[1].is_contiguous() and ref[1].is_contiguous()
    for g, r in zip(got, ref):
        if r is not None:
            assert torch.equal(g, r)


def test_prologue_two_calls_carry_the_state():
    """The same tokens in two calls (the state carried by the library) equal one call."""
    m = rba()
    new, lens = [6, 4], [40, 4]
    inp = make_prologue_inputs(new, lens, Hq=8, Hkv=1, W=4, seed=7)
    q_o, k_o, v_o, pos, nsk, nsv = oracle_of(inp)
    first = {"idx": [0, 1, 2, 6], "cu": [0, 3, 4], "lens": [37, 1]}
    second = {"idx": [3, 4, 5, 7, 8, 9], "cu": [0, 3, 6], "lens": [40, 4]}
    d = {k: v.to(DEV) for k, v in inp.items()}
    kc = torch.full((2, 64, 1, 128), SENTINEL, dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, -SENTINEL)
    sk, sv = d["state_k"].clone(), d["state_v"].clone()
    qs = []
    for part in (first, second):
        ix = torch.tensor(part["idx"], device=DEV)
        qs.append(m.attn_prologue(d["q"][ix], d["k"][ix], d["v"][ix], torch.tensor(part["cu"], dtype=torch.int32, device=DEV),
                                  torch.tensor(part["lens"], dtype=torch.int32, device=DEV), d["conv_wk"], d["conv_wv"],
                                  d["norm_q"], d["norm_k"], sk, sv, kc, vc, eps=1e-6))
    torch.cuda.synchronize()
    order = first["idx"] + second["idx"]
    qo = torch.empty_like(d["q"])
    qo[torch.tensor(order, device=DEV)] = torch.cat(qs)
    close("q_out", qo, q_o)
    bs = seq_of(inp)
    close("k rows", kc[bs, pos], k_o)
    close("v rows", vc[bs, pos], v_o)
    assert np.array_equal(sk.double().cpu().numpy(), nsk) and np.array_equal(sv.double().cpu().numpy(), nsv)


def test_prologue_paged_bf16():
    new, lens = [1, 9, 30], [300, 200, 30]
    inp = make_prologue_inputs(new, lens, Hq=16, Hkv=2, W=4, seed=11)
    g = torch.Generator().manual_seed(5)
    n_pages = 16
    table = torch.randperm(n_pages, generator=g)[:15].reshape(3, 5).to(torch.int32)   # 5 pages of 64 per sequence
    qo, kc, vc, _, _, sk, sv = run(inp, 320, paged=(64, n_pages, table))
    q_o, k_o, v_o, pos, nsk, nsv = oracle_of(inp)
    close("q_out", qo, q_o)
    bs = seq_of(inp)
    pg = table[bs, pos // 64].long()
    close("k rows", kc[pg, pos % 64], k_o)
    close("v rows", vc[pg, pos % 64], v_o)
    written = torch.zeros(kc.shape[:2], dtype=torch.bool)
    written[pg, pos % 64] = True
    assert torch.all(kc[~written.to(DEV)] == SENTINEL)
    assert np.array_equal(sk.double().cpu().numpy(), nsk)


def test_prologue_mxfp8_cache():
    m = rba()
    inp = make_prologue_inputs(MIX["new"], MIX["lens"], Hq=16, Hkv=2, W=4, seed=13)
    _, kc16, vc16, _, _, _, _ = run(inp, 512)
    _, kc8, vc8, ks8, vs8, _, _ = run(inp, 512, f8=True)
    bs = seq_of(inp)
    q_o, k_o, v_o, pos, _, _ = oracle_of(inp)
    for name, c16, c8, s8 in (("k", kc16, kc8, ks8), ("v", vc16, vc8, vs8)):
        rows16 = c16[bs, pos]
        ec, es = m.mxfp8_quantize(rows16)
        assert torch.equal(c8[bs, pos], ec) and torch.equal(s8[bs, pos], es), name
        # untouched rows keep their bytes
        mask = torch.ones(c8.shape[:2], dtype=torch.bool)
        mask[bs, pos] = False
        assert torch.all(c8[mask.to(DEV)] == (0x55 if name == "k" else 0x66))
        # decoded rows against the oracle: within one E4M3 step of the block (or the clip of a saturated entry)
        dec = oracle.mxfp8_dequantize(c8[bs, pos].cpu().numpy(), s8[bs, pos].cpu().numpy())
        want = k_o if name == "k" else v_o
        sc = np.ldexp(1.0, s8[bs, pos].cpu().numpy().astype(int) - 127).repeat(32, axis=-1)
        step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(want) / sc, 2.0 ** -6))).astype(int) - 3) * sc
        ok = (np.abs(dec - want) <= step * 0.51 + 2.0 ** -8 * np.abs(want)) | (np.abs(want) / sc > 448)
        say(f"[mxfp8 {name}] rows {len(bs)}, entries within a half step: {ok.mean():.6f}")
        assert ok.all(), f"{name}: {np.sum(~ok)} entries off"


@pytest.mark.parametrize("max_new", [0, 32], ids=["chunked", "one_launch"])
def test_prologue_ignores_garbage_state_before_sequence_start(max_new):
    """Conv-state rows of positions before a sequence's start hold large
    garbage here (the generator zeroes them; a serving engine need not): the
    rows the call writes must not depend on them.  The oracle of the same
    inputs treats those rows as zero, and the outputs must also equal those of
    the zeroed state; the carried state is a plain copy either way."""
    inp = make_prologue_inputs(MIX["new"], MIX["lens"], Hq=16, Hkv=2, W=4, seed=17)
    clean_q, clean_k, clean_v, pos, _, _ = oracle_of(inp)
    g = torch.Generator().manual_seed(99)
    garbage = dict(inp)
    garbage["state_k"] = inp["state_k"].clone()
    garbage["state_v"] = inp["state_v"].clone()
    n_garbage = 0
    for b, (n, L) in enumerate(zip(MIX["new"], MIX["lens"])):
        start = L - n
        for j in range(3):
            if start - 3 + j < 0:
                garbage["state_k"][b, j] = (torch.randn(2, 128, generator=g) * 300).to(torch.bfloat16)
                garbage["state_v"][b, j] = (torch.randn(2, 128, generator=g) * 300).to(torch.bfloat16)
                n_garbage += 1
    assert n_garbage >= 6          # the two sequences that start inside the call, and the 2-token one
    qo, kc, vc, _, _, sk, sv = run(garbage, 512, max_new=max_new)
    q_o, k_o, v_o, pos_g, nsk, nsv = oracle_of(garbage)
    assert np.array_equal(pos, pos_g)
    assert np.allclose(k_o, clean_k, rtol=0, atol=0) and np.allclose(v_o, clean_v, rtol=0, atol=0)
    close("q_out", qo, clean_q)
    bs = seq_of(inp)
    close("k rows (garbage state)", kc[bs, pos], clean_k)
    close("v rows (garbage state)", vc[bs, pos], clean_v)
    assert np.array_equal(sk.double().cpu().numpy(), nsk) and np.array_equal(sv.double().cpu().numpy(), nsv)


@pytest.mark.parametrize("case", ["bf16", "mxfp8", "paged", "W8", "W1"])
def test_prologue_one_launch_equals_chunked(case):
    """With a bound on the new tokens per sequence the prologue runs as one
    launch (K/V rows of a sequence taken in order by one half wave, which also
    advances its conv state); without it, in chunks of 8 tokens plus a launch
    for the states.  The arithmetic is the same, so every output (q_out, cache
    rows and scales, untouched sentinels, conv states) must agree bit for bit,
    here on a decode/verify batch (64 sequences of 9 tokens, the bound met) and
    on the mixed batch with the bound exceeded."""
    W = 8 if case == "W8" else (1 if case == "W1" else 4)
    f8 = case == "mxfp8"
    for new, lens, bound in (([9] * 64, [700 + 3 * b for b in range(64)], 9), (MIX["new"], MIX["lens"], 8)):
        say(f"prologue one launch vs chunked: {case}, B={len(new)}, bound {bound}")
        inp = make_prologue_inputs(new, lens, Hq=16, Hkv=2, W=W, seed=31)
        paged = None
        Skv = 1024
        if case == "paged":
            g = torch.Generator().manual_seed(3)
            n_pages = 16 * len(new) + 1
            table = torch.randperm(n_pages, generator=g)[:16 * len(new)].reshape(len(new), 16).to(torch.int32)
            paged = (64, n_pages, table)
        a = run(inp, Skv, f8=f8, paged=paged, max_new=0)
        b = run(inp, Skv, f8=f8, paged=paged, max_new=bound)
        for x, y in zip(a, b):
            if x is not None:
                assert torch.equal(x, y)
        if not f8:
            q_o, k_o, v_o, pos, nsk, nsv = oracle_of(inp)
            close("q_out", b[0], q_o)
            if W > 1:
                assert np.array_equal(b[5].double().cpu().numpy(), nsk)
                assert np.array_equal(b[6].double().cpu().numpy(), nsv)
