"""GPU parity of the MXFP8 KV path: the encoder (rba_mxfp8_quantize) bit for
bit against the oracle's encoder, and attention over an MXFP8 cache against
the fp64 oracle on the decoded values.

The cache codes and scales given to the attention kernels come from the
oracle's encoder on the CPU, never from the GPU encoder.  Decoding an E4M3
code times a power of two into bf16 is exact, so attention over the MXFP8
cache must also agree bit for bit with the bf16 path run on the decoded
cache (same kernel arithmetic); tolerances against the oracle are those of
the bf16 path (max|d| <= 2e-2, mean|d| <= 2e-3).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs, make_paged_inputs
from workloads.configs import scaled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def rba():
    import relative_position_bias_rba_amd as m  # fails loudly if librba.so is missing
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, want, fp32=False, tol=None):
    g = got.detach().double().cpu().numpy()
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    d = np.abs(g - w)
    mx, mean = float(d.max()), float(d.mean())
    rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
    say(f"[{name}] max|d|={mx:.3e} mean|d|={mean:.3e} rel_l2={rel:.3e}")
    if fp32:
        assert mx <= (1e-5 if tol is None else tol), name
        assert rel <= (1e-5 if tol is None else 2e-3), f"{name}: rel_l2 {rel:.3e}"
    else:
        assert mx <= 2e-2 and mean <= 2e-3, name
        assert rel <= 1e-2, f"{name}: rel_l2 {rel:.3e}"


def quantize_cpu(x):
    """Oracle encoding of a CPU tensor [..., 128] -> (codes, scales) as uint8 tensors."""
    c, s = oracle.mxfp8_quantize(x)
    return torch.from_numpy(c), torch.from_numpy(s)


def decoded_bf16(codes, scales):
    """The decoded cache as a bf16 tensor (exact: every decoded value fits bf16)."""
    d = oracle.mxfp8_dequantize(codes.numpy(), scales.numpy())
    t = torch.from_numpy(d).to(torch.bfloat16)
    assert np.array_equal(t.double().numpy(), d)
    return t


# --------------------------------------------------------------------------- encoder

def _encoder_inputs(rows, n, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, n, generator=g)
    # a different magnitude per block, an all-zero block, a block of exact ties
    mags = torch.pow(2.0, torch.randint(-20, 20, (rows, n // 32), generator=g).float())
    x = x * mags.repeat_interleave(32, dim=1)
    x[0, :32] = 0.0
    if n >= 64:
        # values halfway between E4M3 neighbours once the block scale 2^-8 is applied
        x[0, 32:64] = torch.tensor([(1.0 + (2 * i + 1) / 16.0) * 2.0 ** -8 for i in range(8)] * 4)
        x[0, 32] = 1.0
    if rows > 1:
        x[1, :32] = 1.9 * torch.sign(torch.randn(32, generator=g))      # saturating block
    return x.to(dtype)


@pytest.mark.parametrize("rows,n,dtype,pad", [
    (300, 128, torch.bfloat16, 0),
    (97, 128, torch.bfloat16, 64),      # row stride past n
    (64, 256, torch.float32, 0),
    (33, 32, torch.float32, 4),
])
def test_encoder_bitexact(rows, n, dtype, pad):
    m = rba()
    say(f"mxfp8 encode rows={rows} n={n} {dtype} pad={pad}")
    x = _encoder_inputs(rows, n, dtype, seed=rows + n)
    if pad:     # a view with row stride n + pad
        x = torch.cat([x, torch.ones(rows, pad, dtype=dtype)], dim=1)[:, :n]
    codes, scales = m.mxfp8_quantize(x.to(DEV))
    torch.cuda.synchronize()
    wc, ws = oracle.mxfp8_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), ws)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != wc)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: {got[tuple(bad[0])]} vs {wc[tuple(bad[0])]}"


def test_encoder_kv_cache_shape():
    """The encoder on a [B, S, Hkv, 128] cache (one vector per key and head)."""
    m = rba()
    g = torch.Generator().manual_seed(3)
    k = torch.randn(2, 70, 3, 128, generator=g).to(torch.bfloat16)
    c, s = m.mxfp8_quantize(k.to(DEV))
    wc, ws = oracle.mxfp8_quantize(k)
    assert c.shape == (2, 70, 3, 128) and s.shape == (2, 70, 3, 4)
    assert np.array_equal(c.cpu().numpy(), wc) and np.array_equal(s.cpu().numpy(), ws)


# --------------------------------------------------------------------------- attention over an MXFP8 cache

def _f8_inputs(w, seed=None):
    inp = make_inputs(w, seed)
    kc, ks = quantize_cpu(inp["k"])
    vc, vs = quantize_cpu(inp["v"])
    inp.update(kc=kc, ks=ks, vc=vc, vs=vs, kd=decoded_bf16(kc, ks), vd=decoded_bf16(vc, vs))
    return inp


F8_CASES = [
    # name, overrides of the decode workload, splits
    ("decode_full", dict(B=3, Sq=9, Skv=700, Hq=16, Hkv=2, E=64, window=0), [1, 3, 0]),
    ("decode_swa_log", dict(B=2, Sq=5, Skv=777, Hq=16, Hkv=2, E=96, window=300, log_scale_base=64.0), [1, 4]),
    ("long_sq1", dict(B=1, Sq=1, Skv=3000, Hq=8, Hkv=1, E=64, window=0, log_scale_base=4096.0), [1, 8]),
    ("wide_prefill", dict(B=1, Sq=300, Skv=300, Hq=16, Hkv=2, E=64, window=96), [1]),
    # every key tile carries bias: consecutive banded tiles share the one bias buffer of the
    # staging-wave kernels, which then reload it between two barriers
    ("all_banded", dict(B=2, Sq=9, Skv=400, Hq=16, Hkv=2, E=512, window=0), [1, 3]),
    # bias rows not 16-byte aligned: the bias windows go through registers
    ("unaligned_E", dict(B=2, Sq=9, Skv=500, Hq=16, Hkv=2, E=100, window=0), [1]),
    # 112 query columns: no wave without columns, every thread decodes its share
    ("wide_g112", dict(B=2, Sq=1, Skv=600, Hq=112, Hkv=1, E=64, window=0), [1, 2]),
    # exactly 96 query columns: three full waves and the staging wave
    ("cols96", dict(B=2, Sq=6, Skv=500, Hq=32, Hkv=2, E=64, window=0), [1, 2]),
]


@pytest.mark.parametrize("name,over,splits", F8_CASES, ids=[c[0] for c in F8_CASES])
def test_attention_mxfp8_parity(name, over, splits):
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], **over)
    say(f"mxfp8 attention {name}: {w}")
    inp = _f8_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    Rw = oracle.relproj(inp["r"], inp["P"])
    wo, wl = oracle.attention(inp["q"], inp["kd"], inp["vd"], Rw, window=w.window, log_scale_base=w.log_scale_base)
    kw = dict(window=w.window, log_scale_base=w.log_scale_base, return_lse=True)
    for s in splits:
        o, lse = m.attn_decode(d["q"], d["kc"], d["vc"], R, num_splits=s, k_scale=d["ks"], v_scale=d["vs"], **kw)
        torch.cuda.synchronize()
        check(f"{name}/{s} o", o, wo)
        check(f"{name}/{s} lse", lse, wl, fp32=True, tol=2e-2)
        # the same kernel arithmetic on the decoded cache in bf16
        if w.G * min(w.Sq, 32) <= 128:
            ob, lb = m.attn_decode(d["q"], d["kd"], d["vd"], R, num_splits=s, **kw)
            torch.cuda.synchronize()
            assert torch.equal(o, ob) and torch.equal(lse, lb), f"{name}/{s}: MXFP8 and decoded-bf16 paths differ"
    if name == "wide_prefill":
        o, lse = m.attn_prefill(d["q"], d["kc"], d["vc"], R, k_scale=d["ks"], v_scale=d["vs"], **kw)
        torch.cuda.synchronize()
        check(f"{name} prefill o", o, wo)
        check(f"{name} prefill lse", lse, wl, fp32=True, tol=2e-2)


def test_attention_mxfp8_paged():
    """MXFP8 pools of 64-key pages with per-sequence lengths; unowned rows hold
    NaN codes (0x7f) and NaN scales (255)."""
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], B=4, Sq=9, Skv=640, Hq=16, Hkv=2, E=64, window=0)
    inp = make_paged_inputs(w, 64, seq_lens=[9, 640, 200, 65])
    kc, ks = quantize_cpu(inp["k_pool"])
    vc, vs = quantize_cpu(inp["v_pool"])
    owned = torch.zeros(kc.shape[:2], dtype=torch.bool)
    for b, L in enumerate(inp["seq_lens"].tolist()):
        for j0 in range(0, L, 64):
            owned[int(inp["block_table"][b, j0 // 64]), :min(64, L - j0)] = True
    kd, vd = decoded_bf16(kc, ks), decoded_bf16(vc, vs)
    for t in (kc, vc):
        t[~owned] = 0x7F
    for t in (ks, vs):
        t[~owned] = 255
    Rw = oracle.relproj(inp["r"], inp["P"])
    wo, wl = oracle.attention_paged(inp["q"], kd, vd, inp["block_table"], inp["seq_lens"], Rw)
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    for s in (1, 4):
        o, lse = m.attn_paged(d["q"], kc.to(DEV), vc.to(DEV), d["block_table"], d["seq_lens"], R, max_seq_len=w.Skv,
                              num_splits=s, return_lse=True, k_scale=ks.to(DEV), v_scale=vs.to(DEV))
        torch.cuda.synchronize()
        check(f"paged mxfp8/{s} o", o, wo)
        check(f"paged mxfp8/{s} lse", lse, wl, fp32=True, tol=2e-2)


def test_attention_mxfp8_full_size_sampled():
    """The full-attention decode workload (64 sequences x 9 rows, 9216 keys, 64/8
    heads) over an MXFP8 cache encoded by the oracle, heuristic splits; sampled
    rows against the oracle on the decoded cache."""
    m = rba()
    w = CONFIGS["c4_decode_full"]
    inp = make_inputs(scaled(w, Skv=4096, B=1))
    # the cache: rows of an oracle-encoded 4096-key template, picked at random
    # per (sequence, position) by a seeded index (encoding 600M entries in fp64
    # would take minutes)
    tk, tks = quantize_cpu(inp["k"][0])
    tv, tvs = quantize_cpu(inp["v"][0])
    g = torch.Generator().manual_seed(404)
    idx = torch.randint(0, 4096, (w.B, w.Skv), generator=g)
    kc, ks, vc, vs = tk[idx], tks[idx], tv[idx], tvs[idx]
    inp = make_inputs(w)            # q, r, P at full size (k, v unused)
    d = {k: v.to(DEV) for k, v in inp.items() if k in ("q", "r", "P")}
    R = m.relproj(d["r"], d["P"])
    o, lse = m.attn_decode(d["q"], kc.to(DEV), vc.to(DEV), R, k_scale=ks.to(DEV), v_scale=vs.to(DEV),
                           window=w.window, return_lse=True)
    torch.cuda.synchronize()
    rows = [(0, 0), (0, 8), (17, 4), (40, 8), (63, 0)]
    # decoded cache of the sampled sequences only (the others stay zero)
    kd = torch.zeros(kc.shape, dtype=torch.float64)
    vd = torch.zeros(vc.shape, dtype=torch.float64)
    for b in sorted({b for b, _ in rows}):
        kd[b] = torch.from_numpy(oracle.mxfp8_dequantize(kc[b].numpy(), ks[b].numpy()))
        vd[b] = torch.from_numpy(oracle.mxfp8_dequantize(vc[b].numpy(), vs[b].numpy()))
    Rw = lambda b, t: oracle.relproj(inp["r"][b, t], inp["P"])
    wo, wl = oracle.attention_rows(inp["q"], kd, vd, Rw, rows, window=w.window)
    got_o = torch.stack([o[b, t] for b, t in rows])
    got_l = torch.stack([lse[b, :, t] for b, t in rows])
    check("full-size mxfp8 o", got_o, wo)
    check("full-size mxfp8 lse", got_l, wl, fp32=True, tol=2e-2)


# --------------------------------------------------------------------------- MXFP8 logits (q encoded, scaled FP8 MFMA)

@pytest.mark.parametrize("name,over,splits", F8_CASES, ids=[c[0] for c in F8_CASES])
def test_attention_mxfp8_logits_parity(name, over, splits):
    """rba_kv_format RBA_KV_MXFP8_QK against oracle.attention_mxfp8_logits on
    every element (q encoded with the cache's rule, logits of the decoded q
    and K, V decoded)."""
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], **over)
    say(f"mxfp8 logits {name}: {w}")
    inp = _f8_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    Rw = oracle.relproj(inp["r"], inp["P"])
    wo, wl = oracle.attention_mxfp8_logits(inp["q"], inp["kc"].numpy(), inp["ks"].numpy(), inp["vc"].numpy(),
                                           inp["vs"].numpy(), Rw, window=w.window, log_scale_base=w.log_scale_base)
    kw = dict(window=w.window, log_scale_base=w.log_scale_base, return_lse=True, k_scale=d["ks"], v_scale=d["vs"],
              qk_fp8=True)
    outs = []
    for s in splits:
        o, lse = m.attn_decode(d["q"], d["kc"], d["vc"], R, num_splits=s, **kw)
        torch.cuda.synchronize()
        check(f"{name}/{s} o", o, wo)
        check(f"{name}/{s} lse", lse, wl, fp32=True, tol=2e-2)
        outs.append(lse)
    # the encoded q moves the logits: the result is measurably not the plain
    # MXFP8-cache attention (bf16 q), which the oracle computes separately
    wp, _ = oracle.attention(inp["q"], inp["kd"], inp["vd"], Rw, window=w.window, log_scale_base=w.log_scale_base)
    g = o.double().cpu().numpy()
    assert np.linalg.norm(g - wo) < 0.5 * np.linalg.norm(g - wp), name
    if name == "wide_prefill":
        o, lse = m.attn_prefill(d["q"], d["kc"], d["vc"], R, **kw)
        torch.cuda.synchronize()
        check(f"{name} prefill o", o, wo)
        check(f"{name} prefill lse", lse, wl, fp32=True, tol=2e-2)


def test_attention_mxfp8_logits_paged():
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], B=4, Sq=9, Skv=640, Hq=16, Hkv=2, E=64, window=0)
    inp = make_paged_inputs(w, 64, seq_lens=[9, 640, 200, 65])
    kc, ks = quantize_cpu(inp["k_pool"])
    vc, vs = quantize_cpu(inp["v_pool"])
    Rw = oracle.relproj(inp["r"], inp["P"])
    kd = oracle.mxfp8_dequantize(kc.numpy(), ks.numpy())
    vd = oracle.mxfp8_dequantize(vc.numpy(), vs.numpy())
    qd = oracle.mxfp8_dequantize(*oracle.mxfp8_quantize(inp["q"]))
    wo, wl = oracle.attention_paged(qd, kd, vd, inp["block_table"], inp["seq_lens"], Rw)
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    for s in (1, 4):
        o, lse = m.attn_paged(d["q"], kc.to(DEV), vc.to(DEV), d["block_table"], d["seq_lens"], R, max_seq_len=w.Skv,
                              num_splits=s, return_lse=True, k_scale=ks.to(DEV), v_scale=vs.to(DEV), qk_fp8=True)
        torch.cuda.synchronize()
        check(f"paged mxfp8 logits/{s} o", o, wo)
        check(f"paged mxfp8 logits/{s} lse", lse, wl, fp32=True, tol=2e-2)


@pytest.mark.parametrize("name,rows", [
    ("c4_decode_full", [(0, 0), (0, 8), (17, 4), (63, 8)]),
    ("c5_long_decode", [(0, 0)]),
])
def test_attention_mxfp8_logits_full_size_sampled(name, rows):
    """The full decode workloads over an MXFP8 cache (oracle-encoded template
    rows, as in the test above) with MXFP8 logits, heuristic splits; sampled
    rows against the oracle."""
    m = rba()
    w = CONFIGS[name]
    tmpl = make_inputs(scaled(w, Skv=4096, B=1, Sq=1))
    tk, tks = quantize_cpu(tmpl["k"][0])
    tv, tvs = quantize_cpu(tmpl["v"][0])
    g = torch.Generator().manual_seed(505)
    idx = torch.randint(0, 4096, (w.B, w.Skv), generator=g)
    kc, ks, vc, vs = tk[idx], tks[idx], tv[idx], tvs[idx]
    inp = make_inputs(scaled(w, Skv=w.Sq))   # q, r, P at full size (k, v unused)
    d = {k: v.to(DEV) for k, v in inp.items() if k in ("q", "r", "P")}
    R = m.relproj(d["r"], d["P"])
    o, lse = m.attn_decode(d["q"], kc.to(DEV), vc.to(DEV), R, k_scale=ks.to(DEV), v_scale=vs.to(DEV),
                           window=w.window, log_scale_base=w.log_scale_base, return_lse=True, qk_fp8=True)
    torch.cuda.synchronize()
    # the oracle over the sampled sequences only (batch index i of bs[i])
    bs = sorted({b for b, _ in rows})
    kd = torch.stack([torch.from_numpy(oracle.mxfp8_dequantize(kc[b].numpy(), ks[b].numpy())) for b in bs])
    vd = torch.stack([torch.from_numpy(oracle.mxfp8_dequantize(vc[b].numpy(), vs[b].numpy())) for b in bs])
    qd = torch.from_numpy(oracle.mxfp8_dequantize(*oracle.mxfp8_quantize(inp["q"][bs])))
    Rw = lambda i, t: oracle.relproj(inp["r"][bs[i], t], inp["P"])
    sel = [(bs.index(b), t) for b, t in rows]
    wo, wl = oracle.attention_rows(qd, kd, vd, Rw, sel, window=w.window, log_scale_base=w.log_scale_base)
    check(f"{name} mxfp8 logits o", torch.stack([o[b, t] for b, t in rows]), wo)
    check(f"{name} mxfp8 logits lse", torch.stack([lse[b, :, t] for b, t in rows]), wl, fp32=True, tol=2e-2)
