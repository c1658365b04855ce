"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: fp32 paths max|d| <= 1e-5; bf16 paths max|d| <= 2e-2 and
mean|d| <= 2e-3, relative L2 <= 1e-2 (lse 2e-3); masking and bucket indexing
exact (one-hot tests); biased outputs must sit far closer to the oracle than
the oracle without bias does.
Small cases compare every output element; the full-size workloads run in the
launch configuration the benchmark times and compare sampled rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs
from workloads.configs import scaled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def rba():
    import relative_position_bias_rba_amd as m  # fails loudly if librba.so is missing
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, want, fp32, extra_tol=None):
    """Element-wise comparison.  Absolute bounds as stated at the top, plus a
    relative L2 bound: 1e-5 on fp32 paths, 1e-2 on bf16 outputs (one bf16
    rounding of o and of the probabilities is ~4e-3) and 2e-3 on the fp32 lse
    of bf16 paths (lse is O(ln n))."""
    g = got.detach().double().cpu().numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    d = np.abs(g - w)
    mx, mean = float(d.max()), float(d.mean())
    rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
    say(f"[{name}] max|d|={mx:.3e} mean|d|={mean:.3e} rel_l2={rel:.3e}")
    if fp32:
        assert mx <= (1e-5 if extra_tol is None else extra_tol), name
        assert rel <= (1e-5 if extra_tol is None else 2e-3), f"{name}: rel_l2 {rel:.3e}"
    else:
        assert mx <= 2e-2 and mean <= 2e-3, name
        assert rel <= 1e-2, f"{name}: rel_l2 {rel:.3e}"
    return mx, mean


def check_bias_seen(name, got, want, want_nobias, ratio=0.1):
    """The output must follow the bias: its distance to the biased oracle is
    at most `ratio` times the distance between the biased and the unbiased
    oracle (a kernel that dropped or misplaced the bias would sit about as far
    from the biased oracle as the unbiased one does).  Skipped where the bias
    cannot move the output (e.g. one visible key per row)."""
    g = got.detach().double().cpu().numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    w, w0 = np.asarray(want, np.float64), np.asarray(want_nobias, np.float64)
    effect = float(np.linalg.norm(w - w0))
    if effect <= 1e-3 * max(float(np.linalg.norm(w)), 1e-30):
        say(f"[{name}] bias effect {effect:.3e}: too small to test")
        return
    r = float(np.linalg.norm(g - w)) / effect
    say(f"[{name}] |got - oracle| / |oracle - oracle(R=0)| = {r:.3e}")
    assert r <= ratio, f"{name}: the output does not follow the bias ({r:.3e})"


def to_dev(inp):
    return {k: v.to(DEV) for k, v in inp.items()}


def small(w, **over):
    return scaled(w, **over)


# --------------------------------------------------------------------------- relproj

@pytest.mark.parametrize("T,Hq,r_dim,E,dt,odt", [
    (256, 4, 32, 64, torch.float32, torch.float32),
    (1000, 8, 64, 512, torch.bfloat16, torch.bfloat16),
    (77, 3, 40, 100, torch.bfloat16, torch.bfloat16),
    (300, 5, 17, 37, torch.float32, torch.float32),
    (129, 2, 128, 200, torch.bfloat16, torch.float32),
    (1, 64, 64, 512, torch.bfloat16, torch.bfloat16),
    (64, 3, 128, 1000, torch.bfloat16, torch.bfloat16),   # several distance chunks, ragged last one
    (40, 2, 128, 130, torch.float32, torch.float32),      # the smallest chunk size
])
def test_relproj_parity(T, Hq, r_dim, E, dt, odt):
    say(f"relproj T={T} Hq={Hq} r_dim={r_dim} E={E} {dt}->{odt}")
    g = torch.Generator().manual_seed(T * 7 + E)
    r = torch.randn(T, r_dim, generator=g).to(dt)
    P = (torch.randn(Hq, r_dim, E, generator=g) * 0.02).to(dt)
    R = rba().relproj(r.to(DEV), P.to(DEV), out_dtype=odt)
    torch.cuda.synchronize()
    want = oracle.relproj(r, P)
    fp32 = odt == torch.float32 and dt == torch.float32
    if odt == torch.bfloat16:
        # one bf16 rounding of the fp32 sum: |d| <= 2^-8 |R| (+ fp32 sum error)
        g_ = R.double().cpu().numpy()
        assert np.all(np.abs(g_ - want) <= np.abs(want) * 2.0 ** -8 + 1e-5)
    check(f"relproj {T}x{Hq}x{r_dim}x{E}", R, want, fp32)


@pytest.mark.parametrize("T,Hq,r_dim,E,dt,sliced", [
    (200, 4, 64, 96, torch.bfloat16, False),
    (77, 3, 40, 100, torch.bfloat16, True),     # rows not 16-byte aligned: element loads
    (130, 2, 32, 64, torch.float32, False),
])
def test_relproj_per_head_parity(T, Hq, r_dim, E, dt, sliced):
    say(f"relproj per-head T={T} Hq={Hq} r_dim={r_dim} E={E} {dt} sliced={sliced}")
    g = torch.Generator().manual_seed(T + 13 * E)
    full = torch.randn(T, Hq, r_dim + (3 if sliced else 0), generator=g).to(dt)
    r = full[..., :r_dim]                       # head stride r_dim (+3 when sliced)
    P = (torch.randn(Hq, r_dim, E, generator=g) * 0.02).to(dt)
    R = rba().relproj(full.to(DEV)[..., :r_dim], P.to(DEV), per_head=True)
    torch.cuda.synchronize()
    want = oracle.relproj(r, P, per_head=True)
    if dt == torch.float32:
        check("relproj per-head", R, want, True)
    else:
        g_ = R.double().cpu().numpy()
        assert np.all(np.abs(g_ - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)


@pytest.mark.parametrize("case", ["wide_g256", "decode_g256", "narrow_g128", "fp32_g128", "mxfp8_g128"])
def test_largest_groups(case):
    """The largest query-head groups each variant takes (one query row per block)."""
    m = rba()
    cfg = {
        "wide_g256": ("c2_swa_prefill", dict(B=1, Sq=40, Skv=100, Hq=256, Hkv=1, E=32, window=0), None),
        "decode_g256": ("c4_decode_full", dict(B=2, Sq=1, Skv=300, Hq=256, Hkv=1, E=32, window=0), 3),
        "narrow_g128": ("c4_decode_full", dict(B=2, Sq=1, Skv=300, Hq=128, Hkv=1, E=32, window=64), 2),
        "fp32_g128": ("c1_tiny_fp32", dict(B=1, Sq=5, Skv=70, Hq=128, Hkv=1, E=16), None),
        "mxfp8_g128": ("c4_decode_full", dict(B=2, Sq=1, Skv=300, Hq=128, Hkv=1, E=32, window=0), 3),
    }[case]
    w = small(CONFIGS[cfg[0]], **cfg[1])
    say(f"largest group {case}: {w}")
    inp = make_inputs(w)
    d = to_dev(inp)
    R = m.relproj(d["r"], d["P"])
    kw = dict(window=w.window, log_scale_base=w.log_scale_base, return_lse=True)
    k, v = inp["k"], inp["v"]
    if case == "mxfp8_g128":
        kc, ks = oracle.mxfp8_quantize(inp["k"])
        vc, vs = oracle.mxfp8_quantize(inp["v"])
        k, v = oracle.mxfp8_dequantize(kc, ks), oracle.mxfp8_dequantize(vc, vs)
        o, lse = m.attn_decode(d["q"], torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV), R,
                               num_splits=cfg[2], k_scale=torch.from_numpy(ks).to(DEV),
                               v_scale=torch.from_numpy(vs).to(DEV), **kw)
    elif cfg[2] is None:
        o, lse = m.attn_prefill(d["q"], d["k"], d["v"], R, **kw)
    else:
        o, lse = m.attn_decode(d["q"], d["k"], d["v"], R, num_splits=cfg[2], **kw)
    torch.cuda.synchronize()
    wo, wl = oracle.attention(inp["q"], k, v, oracle.relproj(inp["r"], inp["P"]), window=w.window,
                              log_scale_base=w.log_scale_base)
    fp32 = w.dtype == "fp32"
    check(f"{case} o", o, wo, fp32)
    check(f"{case} lse", lse, wl, True, extra_tol=None if fp32 else 2e-2)


def test_calibration_kernels_run():
    """The measurement aids launch, report their flop count and leave the sink alone."""
    import ctypes
    m = rba()
    buf = torch.ones(1 << 24, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(4, dtype=torch.float32, device=DEV)
    st = m._stream(torch.device(DEV))
    assert m._lib.rba_calib_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), ctypes.c_void_p(sink.data_ptr()),
                                 st) == 0
    flops = ctypes.c_double(0.0)
    assert m._lib.rba_calib_mfma(3, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops), st) == 0
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops.value == 8 * cus * 4 * 3 * 4 * 2 * 32 * 32 * 16
    assert torch.count_nonzero(sink).item() == 0


# --------------------------------------------------------------------------- prefill, small shapes, every element

def head_major(x):
    """The same [B, S, H, d] values stored head-major ([B, H, S, d]), as a view."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def run_path(inp, w, *, decode=False, splits=0, return_lse=True, kv_head_major=False):
    m = rba()
    d = to_dev(inp)
    if kv_head_major:
        d["k"], d["v"] = head_major(d["k"]), head_major(d["v"])
    R = m.relproj(d["r"], d["P"])
    fn = m.attn_decode if decode else m.attn_prefill
    kw = dict(window=w.window, log_scale_base=w.log_scale_base, return_lse=return_lse)
    if decode:
        kw["num_splits"] = splits
    out = fn(d["q"], d["k"], d["v"], R, **kw)
    torch.cuda.synchronize()
    return out


def oracle_full(inp, w):
    R = oracle.relproj(inp["r"], inp["P"])
    return oracle.attention(inp["q"], inp["k"], inp["v"], R, window=w.window, log_scale_base=w.log_scale_base)


def test_c1_tiny_fp32_full():
    w = CONFIGS["c1_tiny_fp32"]
    say(f"prefill {w}")
    inp = make_inputs(w)
    o, lse = run_path(inp, w)
    wo, wl = oracle_full(inp, w)
    check("c1 o", o, wo, True)
    check("c1 lse", lse, wl, True)


PREFILL_CASES = [
    # name, overrides of the windowed bf16 workload
    ("swa_ragged", dict(B=1, Sq=300, Skv=300, Hq=16, Hkv=2, window=96, E=64)),
    ("full_logscale", dict(B=2, Sq=517, Skv=517, Hq=16, Hkv=2, window=0, E=64, log_scale_base=4096.0)),
    ("swa_wide_extent", dict(B=1, Sq=400, Skv=400, Hq=8, Hkv=1, window=70, E=200)),
    ("ext_not_mult8", dict(B=1, Sq=333, Skv=333, Hq=8, Hkv=2, window=0, E=100)),
    ("gqa4", dict(B=1, Sq=260, Skv=260, Hq=8, Hkv=2, window=0, E=64)),
    ("mha", dict(B=1, Sq=200, Skv=200, Hq=2, Hkv=2, window=50, E=32)),
    ("gqa16", dict(B=1, Sq=150, Skv=150, Hq=32, Hkv=2, window=0, E=64)),
    ("sq_lt_skv", dict(B=2, Sq=77, Skv=333, Hq=16, Hkv=2, window=128, E=64, log_scale_base=64.0)),
    ("window1", dict(B=1, Sq=130, Skv=130, Hq=8, Hkv=1, window=1, E=16)),
    ("tiny", dict(B=1, Sq=1, Skv=1, Hq=8, Hkv=1, window=0, E=8)),
    ("wide_partial", dict(B=2, Sq=20, Skv=150, Hq=8, Hkv=1, window=0, E=64)),   # 160 of 256 columns
    ("gqa12", dict(B=1, Sq=100, Skv=100, Hq=24, Hkv=2, window=40, E=64)),      # 12 heads x 21 rows
]


@pytest.mark.parametrize("name,over", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_bf16_small(name, over):
    w = small(CONFIGS["c2_swa_prefill"], **over)
    say(f"prefill {name}: {w}")
    inp = make_inputs(w)
    o, lse = run_path(inp, w)
    wo, wl = oracle_full(inp, w)
    check(f"{name} o", o, wo, False)
    check(f"{name} lse", lse, wl, True, extra_tol=2e-2)
    wo0, _ = oracle.attention(inp["q"], inp["k"], inp["v"], None, window=w.window, log_scale_base=w.log_scale_base)
    check_bias_seen(f"{name} bias", o, wo, wo0)


def _strided_R(R, layout):
    """R [B, Sq, Hq, E] in a layout whose rows are not 16-byte aligned:
    'wide' = a view into rows of E + 3 entries, 'offset' = a view starting
    3 entries into each row (the base pointer itself unaligned)."""
    B, Sq, Hq, E = R.shape
    big = torch.full((B, Sq, Hq, E + 3), float("nan"), dtype=R.dtype, device=R.device)
    view = big[..., :E] if layout == "wide" else big[..., 3:]
    view.copy_(R)
    return view


UNALIGNED_CASES = [
    # name, overrides of the windowed bf16 workload (G = 8: the two-group prefill kernel), R layout
    ("ext100_full", dict(B=1, Sq=333, Skv=333, Hq=16, Hkv=2, window=0, E=100), "contiguous"),
    ("ext100_swa", dict(B=2, Sq=300, Skv=300, Hq=16, Hkv=2, window=96, E=100), "contiguous"),
    ("ext64_wide_rows", dict(B=1, Sq=260, Skv=260, Hq=16, Hkv=2, window=0, E=64), "wide"),
    ("ext72_offset", dict(B=1, Sq=200, Skv=270, Hq=16, Hkv=2, window=150, E=72,
                          log_scale_base=64.0), "offset"),
]


@pytest.mark.parametrize("name,over,layout", UNALIGNED_CASES, ids=[c[0] for c in UNALIGNED_CASES])
def test_prefill_unaligned_bias_rows(name, over, layout):
    """Bias rows that are not 16-byte aligned (extent not a multiple of 8, or
    a strided / offset view of R): the prefill kernel stages them with element
    loads instead of direct-to-LDS copies."""
    m = rba()
    w = small(CONFIGS["c2_swa_prefill"], **over)
    say(f"prefill unaligned bias {name} ({layout}): {w}")
    inp = make_inputs(w)
    d = to_dev(inp)
    R = m.relproj(d["r"], d["P"])
    if layout != "contiguous":
        R = _strided_R(R, layout)
    o, lse = m.attn_prefill(d["q"], d["k"], d["v"], R, window=w.window, log_scale_base=w.log_scale_base,
                            return_lse=True)
    torch.cuda.synchronize()
    wo, wl = oracle_full(inp, w)
    check(f"{name} o", o, wo, False)
    check(f"{name} lse", lse, wl, True, extra_tol=2e-2)
    wo0, _ = oracle.attention(inp["q"], inp["k"], inp["v"], None, window=w.window, log_scale_base=w.log_scale_base)
    check_bias_seen(f"{name} bias", o, wo, wo0)


def test_prefill_kv_spans_beyond_31_bits():
    """K and V rows 8 MiB apart (each tensor spans more than 2^31 bytes): the
    prefill takes its 64-bit-offset path; results as for dense K and V."""
    m = rba()
    w = small(CONFIGS["c2_swa_prefill"], B=1, Sq=300, Skv=300, Hq=16, Hkv=2, window=96, E=64)
    say(f"prefill with 8 MiB K/V row stride: {w}")
    inp = make_inputs(w)
    d = to_dev(inp)
    rs = 1 << 22                      # elements between consecutive key rows
    kv = []
    for name in ("k", "v"):
        buf = torch.empty(w.Skv * rs, dtype=torch.bfloat16, device=DEV)
        view = buf.as_strided((w.B, w.Skv, w.Hkv, w.d), (w.Skv * rs, rs, w.d, 1))
        view.copy_(d[name])
        kv.append(view)
    R = m.relproj(d["r"], d["P"])
    o, lse = m.attn_prefill(d["q"], kv[0], kv[1], R, window=w.window, return_lse=True)
    torch.cuda.synchronize()
    wo, wl = oracle_full(inp, w)
    check("large-stride o", o, wo, False)
    check("large-stride lse", lse, wl, True, extra_tol=2e-2)
    # the same kernel with bias rows that are not 16-byte aligned (element loads)
    Ru = _strided_R(R, "wide")
    o2, lse2 = m.attn_prefill(d["q"], kv[0], kv[1], Ru, window=w.window, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse)
    del kv, buf
    torch.cuda.empty_cache()


def test_prefill_kv_spans_beyond_31_bits_unaligned_extent():
    """The 64-bit-offset prefill with an extent of 100 (bias rows not 16-byte
    aligned) against the oracle."""
    m = rba()
    w = small(CONFIGS["c2_swa_prefill"], B=1, Sq=200, Skv=200, Hq=16, Hkv=2, window=0, E=100)
    say(f"prefill with 8 MiB K/V row stride, E=100: {w}")
    inp = make_inputs(w)
    d = to_dev(inp)
    rs = 1 << 22
    kv = []
    for name in ("k", "v"):
        buf = torch.empty(w.Skv * rs, dtype=torch.bfloat16, device=DEV)
        view = buf.as_strided((w.B, w.Skv, w.Hkv, w.d), (w.Skv * rs, rs, w.d, 1))
        view.copy_(d[name])
        kv.append(view)
    R = m.relproj(d["r"], d["P"])
    o, lse = m.attn_prefill(d["q"], kv[0], kv[1], R, window=w.window, return_lse=True)
    torch.cuda.synchronize()
    wo, wl = oracle_full(inp, w)
    check("large-stride E100 o", o, wo, False)
    check("large-stride E100 lse", lse, wl, True, extra_tol=2e-2)
    wo0, _ = oracle.attention(inp["q"], inp["k"], inp["v"], None, window=w.window)
    check_bias_seen("large-stride E100 bias", o, wo, wo0)
    del kv, buf
    torch.cuda.empty_cache()


def test_prefill_fp32_variants():
    base = CONFIGS["c1_tiny_fp32"]
    for over in (dict(Sq=200, Skv=200, window=33, E=50), dict(B=2, Sq=70, Skv=150, Hq=8, Hkv=2, log_scale_base=16.0),
                 dict(Sq=100, Skv=100, Hq=6, Hkv=3, E=7, window=0)):
        w = small(base, **over)
        say(f"prefill fp32 {w}")
        inp = make_inputs(w)
        o, lse = run_path(inp, w)
        wo, wl = oracle_full(inp, w)
        check("fp32 o", o, wo, True)
        check("fp32 lse", lse, wl, True)


def test_prefill_without_bias_and_noncontiguous_q():
    m = rba()
    w = small(CONFIGS["c2_swa_prefill"], B=1, Sq=200, Skv=200, Hq=16, Hkv=2, window=0, E=64)
    inp = make_inputs(w)
    d = to_dev(inp)
    # q as a strided view into a wider buffer
    qbig = torch.zeros(1, 200, 16, 256, dtype=torch.bfloat16, device=DEV)
    qbig[..., 64:192] = d["q"]
    qv = qbig[..., 64:192]
    o = m.attn_prefill(qv, d["k"], d["v"], None, window=0)
    torch.cuda.synchronize()
    wo, _ = oracle.attention(inp["q"], inp["k"], inp["v"], None)
    check("nobias strided", o, wo, False)


# --------------------------------------------------------------------------- decode, small shapes

DECODE_CASES = [
    ("full", dict(B=3, Sq=9, Skv=700, window=0, log_scale_base=0.0)),
    ("swa", dict(B=3, Sq=9, Skv=1000, window=256, log_scale_base=0.0)),
    ("full_log", dict(B=2, Sq=1, Skv=1500, window=0, log_scale_base=4096.0)),
    ("swa_log", dict(B=2, Sq=5, Skv=777, window=300, log_scale_base=64.0)),
]


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 0])
@pytest.mark.parametrize("name,over", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_small(name, over, splits):
    w = small(CONFIGS["c4_decode_full"], Hq=16, Hkv=2, E=64, **over)
    say(f"decode {name} splits={splits}: {w}")
    inp = make_inputs(w)
    o, lse = run_path(inp, w, decode=True, splits=splits)
    wo, wl = oracle_full(inp, w)
    check(f"decode {name}/{splits} o", o, wo, False)
    check(f"decode {name}/{splits} lse", lse, wl, True, extra_tol=2e-2)


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("name,over", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_small_head_major_cache(name, over, splits):
    # the cache stored [B, Hkv, Skv, d] and passed with its strides: every key
    # tile of a kv head is one contiguous block
    w = small(CONFIGS["c4_decode_full"], Hq=16, Hkv=2, E=64, **over)
    say(f"decode head-major {name} splits={splits}: {w}")
    inp = make_inputs(w)
    o, lse = run_path(inp, w, decode=True, splits=splits, kv_head_major=True)
    o_tm, lse_tm = run_path(inp, w, decode=True, splits=splits)
    wo, wl = oracle_full(inp, w)
    check(f"decode head-major {name}/{splits} o", o, wo, False)
    check(f"decode head-major {name}/{splits} lse", lse, wl, True, extra_tol=2e-2)
    # the layout changes addresses only
    assert torch.equal(o, o_tm) and torch.equal(lse, lse_tm)


@pytest.mark.parametrize("Sq", [6, 7])
def test_decode_column_boundary(Sq):
    """16 query heads a kv head: 96 columns (the 4-wave kernel with V by DMA and
    a 96-row bias slab) and 112 (the general 4-wave kernel), dense and paged."""
    w = small(CONFIGS["c4_decode_full"], B=2, Sq=Sq, Skv=600, Hq=32, Hkv=2, E=64, window=0)
    say(f"decode columns {16 * Sq}: {w}")
    inp = make_inputs(w)
    wo, wl = oracle_full(inp, w)
    for splits in (1, 3):
        o, lse = run_path(inp, w, decode=True, splits=splits)
        check(f"columns {16 * Sq}/{splits} o", o, wo, False)
        check(f"columns {16 * Sq}/{splits} lse", lse, wl, True, extra_tol=2e-2)


def test_decode_split_invariance_and_prefill_agreement():
    m = rba()
    w = small(CONFIGS["c4_decode_full"], B=2, Sq=9, Skv=1200, Hq=16, Hkv=2, E=64, window=0)
    inp = make_inputs(w)
    outs = [run_path(inp, w, decode=True, splits=s) for s in (1, 2, 3, 7, 19)]
    o1, l1 = outs[0]
    # row sums are taken over the bf16-rounded probabilities the PV product
    # uses, so the lse of different key splits agrees to ~1e-4, not fp32 eps
    for o, l in outs[1:]:
        assert torch.max(torch.abs(l - l1)).item() <= 1e-3
        assert torch.max(torch.abs(o.float() - o1.float())).item() <= 2.0 ** -7 * max(1.0, o1.float().abs().max().item())
    # decode with Sq rows equals prefill of the same rows (o and lse)
    op, lp = run_path(inp, w, decode=False)
    assert torch.max(torch.abs(lp - l1)).item() <= 1e-3
    assert torch.max(torch.abs(op.float() - o1.float())).item() <= 2.0 ** -7 * max(1.0, o1.float().abs().max().item())


# --------------------------------------------------------------------------- combine kernel on its own

@pytest.mark.parametrize("S,B,Sq,Hq", [
    (6, 2, 3, 8),        # many rows, few splits: one lane group per row
    (64, 1, 1, 64),      # few rows, many splits: the splits spread over lane groups of a row
    (13, 1, 2, 5),       # few rows, split count not a multiple of the group count
])
def test_combine_kernel_parity(S, B, Sq, Hq):
    say(f"combine S={S} B={B} Sq={Sq} Hq={Hq}")
    m = rba()
    g = torch.Generator().manual_seed(5 + S)
    op = torch.randn(S, B, Sq, Hq, 128, generator=g)
    lp = torch.randn(S, B, Sq, Hq, generator=g) * 3
    lp[1, 0] = -math.inf            # an empty split for some rows
    lp[:, B - 1, Sq - 1, Hq - 1] = -math.inf   # a row with no visible key at all
    lp[0:8, 0, 0, 0] = -math.inf    # a whole lane group's share of one row empty
    q_like = torch.empty(B, Sq, Hq, 128, dtype=torch.float32, device=DEV)
    k_like = torch.empty(B, Sq, 1, 128, dtype=torch.float32, device=DEV)
    o, lse = m.splitkv_combine(op.to(DEV), lp.to(DEV), q_like, k_like, return_lse=True)
    torch.cuda.synchronize()
    wo, wl = oracle.lse_combine(op.numpy(), lp.numpy())
    check("combine o", o, wo, True)
    got_l = lse.cpu().numpy().transpose(0, 2, 1)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(wl))
    fin = np.isfinite(wl)
    assert np.max(np.abs(got_l[fin] - wl[fin])) <= 1e-5


# --------------------------------------------------------------------------- exact structure tests

@pytest.mark.parametrize("dstar,window", [(0, 0), (1, 0), (63, 0), (17, 40), (5, 3)])
@pytest.mark.parametrize("decode", [False, True])
def test_one_hot_bias_exact(dstar, window, decode):
    """q = k = 0, R one-hot 30 at distance d*, v coded by position in two
    bf16-exact channels: o must decode exactly to key p - d* (or equal the
    plain mean when that key is not visible)."""
    one_hot_case(2, 600, 9 if decode else 600, 64, 16, 2, dstar, window, decode)


@pytest.mark.parametrize("dstar,window", [(0, 0), (1, 0), (99, 0), (37, 60), (70, 50)])
def test_one_hot_bias_exact_unaligned_rows(dstar, window):
    """As above through the two-group prefill kernel (G = 8) with an extent
    of 100: bias rows not 16-byte aligned, staged by element loads."""
    one_hot_case(1, 333, 333, 100, 16, 2, dstar, window, False)


@pytest.mark.parametrize("dstar,window", [(0, 0), (1, 0), (99, 0), (37, 60)])
def test_one_hot_bias_exact_decode_unaligned_rows(dstar, window):
    """Decode (72 query columns, the kernel that loads V by DMA) with an
    extent of 100: bias rows not 16-byte aligned, staged by element loads."""
    one_hot_case(1, 333, 9, 100, 16, 2, dstar, window, True)


@pytest.mark.parametrize("dstar,window", [(0, 0), (1, 0), (300, 0), (390, 0), (5, 200)])
def test_one_hot_bias_exact_decode_all_banded(dstar, window):
    """Decode with every key tile inside the extent (E = 512 over 400 keys):
    consecutive banded tiles share the single bias buffer, which is then
    reloaded between two barriers."""
    one_hot_case(2, 400, 9, 512, 16, 2, dstar, window, True)


@pytest.mark.parametrize("dstar,window", [(0, 0), (1, 0), (511, 0), (300, 700), (64, 0)])
def test_one_hot_bias_exact_persistent_rounds(dstar, window):
    """The prefill workloads' heads and extent (Hq = 64, Hkv = 8, E = 512) at
    1100 rows: 8 x 35 = 280 work items, more than the CUs and a multiple of 8,
    so the persistent grid takes them in rounds with its XCD-aware order."""
    one_hot_case(1, 1100, 1100, 512, 64, 8, dstar, window, False)


def one_hot_case(B, S, Sq, E, Hq, Hkv, dstar, window, decode):
    m = rba()
    say(f"one-hot B={B} S={S} Sq={Sq} E={E} Hq={Hq} Hkv={Hkv} d*={dstar} W={window} decode={decode}")
    q = torch.zeros(B, Sq, Hq, 128, dtype=torch.bfloat16)
    k = torch.zeros(B, S, Hkv, 128, dtype=torch.bfloat16)
    v = torch.zeros(B, S, Hkv, 128, dtype=torch.bfloat16)
    j = torch.arange(S)
    v[:, :, :, 0] = (j % 256).to(torch.bfloat16)[None, :, None]
    v[:, :, :, 1] = (j // 256).to(torch.bfloat16)[None, :, None]
    v[:, :, Hkv - 1, 2] = 1.0
    R = torch.zeros(B, Sq, Hq, E, dtype=torch.bfloat16)
    R[..., dstar] = 30.0
    d = {n: t.to(DEV) for n, t in dict(q=q, k=k, v=v, R=R).items()}
    if decode:
        o = m.attn_decode(d["q"], d["k"], d["v"], d["R"], window=window, num_splits=3)
    else:
        o = m.attn_prefill(d["q"], d["k"], d["v"], d["R"], window=window)
    torch.cuda.synchronize()
    o = o.float().cpu()
    wo, _ = oracle.attention(q, k, v, R, window=window)
    leak = S * 255 * math.exp(-30.0) * 4    # total weight of all other keys, times max |v|
    exact_rows = 0
    for t in range(Sq):
        p = S - Sq + t
        lo = 0 if window == 0 else max(0, p - window + 1)
        if p - dstar >= lo:
            target = p - dstar
            c0, c1 = o[:, t, :, 0], o[:, t, :, 1]
            # the selected key is decoded exactly; everything else leaks < e^-30
            assert torch.all(torch.round(c0) == float(target % 256)), (t, c0)
            assert torch.all(torch.round(c1) == float(target // 256)), (t, c1)
            assert torch.all(torch.abs(c0 - float(target % 256)) <= leak), (t, c0)
            assert torch.all(torch.abs(c1 - float(target // 256)) <= leak), (t, c1)
            exact_rows += 1
    if window == 0 or dstar < window:
        assert exact_rows > 0
    else:
        assert exact_rows == 0      # the key at distance d* is outside the window
    # every output is within one bf16 rounding of the oracle (values reach 255,
    # so the bound is relative)
    diff = np.abs(o.double().numpy() - wo)
    assert np.all(diff <= np.abs(wo) * 2.0 ** -8 + 1e-6), float(diff.max())


def test_window_one_returns_v_exactly():
    m = rba()
    w = small(CONFIGS["c2_swa_prefill"], B=1, Sq=333, Skv=333, Hq=16, Hkv=2, window=1, E=64)
    inp = make_inputs(w)
    o = run_path(inp, w, return_lse=False)
    G = 8
    vv = inp["v"].repeat_interleave(G, dim=2)
    assert torch.equal(o.cpu(), vv)


def test_future_keys_never_leak():
    """Make every future key dominant (k_j = 4 q for j > p): any leak through
    the causal mask would change o far beyond tolerance."""
    w = small(CONFIGS["c2_swa_prefill"], B=1, Sq=256, Skv=256, Hq=8, Hkv=8, window=0, E=32)
    inp = make_inputs(w)
    # one query vector per head shared by all rows; keys equal 4 q
    q = inp["q"].clone()
    q[:] = q[:, :1]
    inp["q"] = q
    inp["k"] = (4 * q.float()).to(torch.bfloat16)
    o, _ = run_path(inp, w)
    wo, _ = oracle_full(inp, w)
    check("no-leak", o, wo, False)


def test_uniform_weights_visible_mean():
    """q = k = 0, R = 0: o is the mean of the visible v (exact counting)."""
    m = rba()
    S, Hq, Hkv = 500, 8, 1
    for window in (0, 37, 64, 65):
        q = torch.zeros(1, S, Hq, 128, dtype=torch.bfloat16, device=DEV)
        k = torch.zeros(1, S, Hkv, 128, dtype=torch.bfloat16, device=DEV)
        v = torch.randn(1, S, Hkv, 128, generator=torch.Generator().manual_seed(window)).to(torch.bfloat16)
        o, lse = m.attn_prefill(q, k, v.to(DEV), None, window=window, return_lse=True)
        torch.cuda.synchronize()
        vd = v.double()[0, :, 0]
        cs = torch.cat([torch.zeros(1, 128, dtype=torch.float64), torch.cumsum(vd, 0)])
        pos = torch.arange(S)
        lo = torch.zeros(S, dtype=torch.long) if window == 0 else torch.clamp(pos - window + 1, min=0)
        n = (pos - lo + 1).double()
        mean = (cs[pos + 1] - cs[lo]) / n[:, None]
        check(f"mean W={window}", o[0, :, 0], mean.numpy(), False)
        assert torch.max(torch.abs(lse[0, 0].cpu().double() - torch.log(n))).item() <= 1e-5


def test_repeat_runs_are_bitwise_identical():
    w = small(CONFIGS["c2_swa_prefill"], B=1, Sq=700, Skv=700, Hq=16, Hkv=2, window=200, E=64)
    inp = make_inputs(w)
    a, la = run_path(inp, w)
    b, lb = run_path(inp, w)
    assert torch.equal(a, b) and torch.equal(la, lb)
    wd = small(CONFIGS["c4_decode_full"], B=2, Sq=9, Skv=3000, Hq=16, Hkv=2, E=64)
    inpd = make_inputs(wd)
    a, la = run_path(inpd, wd, decode=True, splits=5)
    b, lb = run_path(inpd, wd, decode=True, splits=5)
    assert torch.equal(a, b) and torch.equal(la, lb)
