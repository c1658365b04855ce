"""GPU parity of the fused prefill (rba_attn_prefill_fused): relative logits
computed inside the attention kernel from r and the packed projection.

Its rows of R are computed with relproj_kernel's operands in relproj_kernel's
order, so the whole output must equal rba_relproj + rba_attn_prefill bit for
bit; small cases are also compared element by element with the fp64 oracle
(bf16 tolerances: max|d| <= 2e-2, mean|d| <= 2e-3).  The packing kernel is an
exact rearrangement of P, checked against the layout written out by indexing.
"""
import ctypes
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


def check(name, got, want, tol_max=2e-2, tol_mean=2e-3):
    g = got.detach().double().cpu().numpy()
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    d = np.abs(g - w)
    rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
    say(f"[{name}] max|d|={d.max():.3e} mean|d|={d.mean():.3e} rel_l2={rel:.3e}")
    assert d.max() <= tol_max and d.mean() <= tol_mean, name
    # relative L2: 1e-2 on bf16 outputs, 2e-3 on lse (looser mean bound given)
    assert rel <= (1e-2 if tol_mean <= 2e-3 else 2e-3), f"{name}: rel_l2 {rel:.3e}"


def per_head_r(inp, w, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(w.B, w.Sq, w.Hq, w.r_dim, generator=g) * w.r_std).to(torch.bfloat16)


def both_paths(d, w, r, per_head, on_chip=False):
    """(fused o, lse), (relproj + prefill o, lse) on the same device inputs."""
    m = rba()
    PT = m.relproj_pack(d["P"])
    kw = dict(window=w.window, log_scale_base=w.log_scale_base, return_lse=True)
    of, lf = m.attn_prefill_fused(d["q"], d["k"], d["v"], r, PT, per_head=per_head, on_chip=on_chip, **kw)
    R = m.relproj(r, d["P"], per_head=per_head)
    ou, lu = m.attn_prefill(d["q"], d["k"], d["v"], R, **kw)
    torch.cuda.synchronize()
    return (of, lf), (ou, lu)


def packed_reference(P):
    """The packed layout written out by indexing alone: for head h, tile eb of
    32 distances, k-step k and lane l, P[h, 16k + 8(l // 32) + x, 32 eb +
    m(l % 32)] for x = 0..7, zero past E, with m(i) = 16((i // 4) % 2) +
    4(i // 8) + i % 4."""
    Hq, r_dim, E = P.shape
    nEB, nks = (E + 31) // 32, r_dim // 16
    Pp = torch.zeros(Hq, r_dim, nEB * 32, dtype=P.dtype)
    Pp[:, :, :E] = P
    lane = torch.arange(64)
    i = lane % 32
    m = 16 * ((i // 4) % 2) + 4 * (i // 8) + i % 4
    eb = torch.arange(nEB)
    k = torch.arange(nks)
    x = torch.arange(8)
    e_idx = (32 * eb[:, None, None, None] + m[None, None, :, None]).expand(nEB, nks, 64, 8)
    c_idx = (16 * k[None, :, None, None] + 8 * (lane // 32)[None, None, :, None] + x).expand(nEB, nks, 64, 8)
    return Pp[:, c_idx, e_idx].reshape(-1)


@pytest.mark.parametrize("Hq,r_dim,E", [(4, 64, 512), (3, 16, 37), (2, 128, 200), (5, 48, 8), (1, 32, 1)])
def test_pack_layout(Hq, r_dim, E):
    g = torch.Generator().manual_seed(Hq * 1000 + E)
    P = torch.randn(Hq, r_dim, E, generator=g).to(torch.bfloat16)
    PT = rba().relproj_pack(P.to(DEV))
    torch.cuda.synchronize()
    assert (PT.Hq, PT.r_dim, PT.E) == (Hq, r_dim, E)
    assert torch.equal(PT.data.cpu(), packed_reference(P))


FUSED_CASES = [
    # name, overrides of the windowed bf16 workload, per-head r
    ("swa_ragged", dict(B=1, Sq=300, Skv=300, Hq=16, Hkv=2, window=96, E=64), False),
    ("full_logscale_r32", dict(B=2, Sq=517, Skv=517, Hq=16, Hkv=2, window=0, E=64, r_dim=32,
                               log_scale_base=4096.0), False),
    ("extent_200", dict(B=1, Sq=400, Skv=400, Hq=8, Hkv=1, window=70, E=200), False),
    ("extent_not_mult8", dict(B=1, Sq=333, Skv=333, Hq=16, Hkv=2, window=0, E=100), False),
    ("gqa16_r128", dict(B=1, Sq=150, Skv=150, Hq=32, Hkv=2, window=0, E=64, r_dim=128), False),
    ("sq_lt_skv", dict(B=2, Sq=77, Skv=333, Hq=16, Hkv=2, window=128, E=64, log_scale_base=64.0), False),
    ("gqa12", dict(B=1, Sq=100, Skv=100, Hq=24, Hkv=2, window=40, E=64), False),
    ("per_head_r", dict(B=1, Sq=200, Skv=200, Hq=16, Hkv=2, window=0, E=64, r_dim=32), True),
    ("rows_17_r16", dict(B=1, Sq=17, Skv=17, Hq=8, Hkv=1, window=0, E=8, r_dim=16), False),
    ("extent_past_seq", dict(B=1, Sq=40, Skv=40, Hq=16, Hkv=2, window=0, E=512), False),
    ("extent_1000_swa", dict(B=1, Sq=700, Skv=700, Hq=16, Hkv=2, window=300, E=1000), False),
    ("extent_2050_r128", dict(B=1, Sq=300, Skv=2300, Hq=16, Hkv=2, window=0, E=2050, r_dim=128), False),
]


@pytest.mark.parametrize("on_chip", [False, True], ids=["workspace", "on_chip"])
@pytest.mark.parametrize("name,over,ph", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_prefill_parity(name, over, ph, on_chip):
    w = scaled(CONFIGS["c2_swa_prefill"], **over)
    if on_chip and w.r_dim > 64:
        pytest.skip("the on-chip path takes features of at most 64 channels")
    say(f"fused {name}: {w} per_head={ph} on_chip={on_chip}")
    inp = make_inputs(w)
    if ph:
        inp["r"] = per_head_r(inp, w, 17)
    d = {k: v.to(DEV) for k, v in inp.items()}
    (of, lf), (ou, lu) = both_paths(d, w, d["r"], ph, on_chip)
    assert torch.equal(of, ou), f"{name}: fused and two-kernel outputs differ"
    assert torch.equal(lf, lu), f"{name}: fused and two-kernel lse differ"
    R = oracle.relproj(inp["r"], inp["P"], per_head=ph)
    wo, wl = oracle.attention(inp["q"], inp["k"], inp["v"], R, window=w.window, log_scale_base=w.log_scale_base)
    check(f"fused {name} o", of, wo)
    check(f"fused {name} lse", lf, wl, tol_max=2e-2, tol_mean=2e-2)


@pytest.mark.parametrize("B,Sq,Hq,Hkv,window", [
    (1, 8192, 16, 2, 4096),   # 512 items: two rounds per workgroup, XCD-aware snake order
    (3, 3000, 8, 1, 0),       # 282 items (not a multiple of 8): plain round robin
])
def test_fused_persistent_rounds_bitwise(B, Sq, Hq, Hkv, window):
    w = scaled(CONFIGS["c2_swa_prefill"], B=B, Sq=Sq, Skv=Sq, Hq=Hq, Hkv=Hkv, window=window)
    say(f"fused rounds: {w}")
    d = {k: v.to(DEV) for k, v in make_inputs(w).items()}
    for on_chip in (False, True):
        (of, lf), (ou, lu) = both_paths(d, w, d["r"], False, on_chip)
        assert torch.equal(of, ou) and torch.equal(lf, lu), f"on_chip={on_chip}"


def test_fused_full_size_workload_bitwise_and_sampled():
    """The sliding-window prefill workload (B=1, S=8192, 64 query / 8 kv heads,
    E=512, W=4096): bit for bit the two-kernel path, and sampled rows against
    the oracle."""
    w = CONFIGS["c2_swa_prefill"]
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    (of, lf), (ou, lu) = both_paths(d, w, d["r"], False)
    assert torch.equal(of, ou) and torch.equal(lf, lu)
    (oc, lc), _ = both_paths(d, w, d["r"], False, on_chip=True)
    assert torch.equal(oc, ou) and torch.equal(lc, lu), "on-chip path"
    rows = [0, 31, 4095, 4096, 8191]
    R = oracle.relproj(inp["r"][:, rows], inp["P"])
    for i, t in enumerate(rows):
        wo, wl = oracle.attention(inp["q"][:, t:t + 1], inp["k"][:, :t + 1], inp["v"][:, :t + 1],
                                  R[:, i:i + 1], window=w.window, log_scale_base=w.log_scale_base)
        check(f"full-size row {t} o", of[:, t:t + 1], wo)


def test_fused_full_causal_workload_bitwise():
    """The full-causal workload (B=2, S=32768, log-scale 4096): 16,384 blocks,
    64 rounds per workgroup; bit for bit the two-kernel path."""
    w = CONFIGS["c3_full_prefill"]
    d = {k: v.to(DEV) for k, v in make_inputs(w).items()}
    (of, lf), (ou, lu) = both_paths(d, w, d["r"], False)
    assert torch.equal(of, ou) and torch.equal(lf, lu)
    (oc, lc), _ = both_paths(d, w, d["r"], False, on_chip=True)
    assert torch.equal(oc, ou) and torch.equal(lc, lu), "on-chip path"


def test_fused_workspace_checks_and_reuse():
    """Too small or missing workspace is refused before any launch; a workspace
    reused across calls (stale rows of an earlier call in it) changes nothing."""
    m = rba()
    w = scaled(CONFIGS["c2_swa_prefill"], B=1, Sq=256, Skv=256, Hq=16, Hkv=2, window=0, E=64)
    d = {k: v.to(DEV) for k, v in make_inputs(w).items()}
    PT = m.relproj_pack(d["P"])
    need = m.prefill_fused_workspace_bytes(d["q"], d["k"], d["v"], w.E)
    assert need > 0
    o = torch.empty_like(d["q"])
    a = m.make_args(d["q"], d["k"], d["v"], None, o, None)
    a.E = w.E
    rb = m.make_relbias(d["r"], PT)
    small_ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    st = m._stream(d["q"].device)
    assert m._lib.rba_attn_prefill_fused(ctypes.byref(a), ctypes.byref(rb), ctypes.c_void_p(small_ws.data_ptr()),
                                         need - 16, st) == m.RBA_E_WORKSPACE
    # no workspace at all: accepted (on-chip path) for r_dim <= 64, refused above
    w128 = scaled(w, r_dim=128)
    r128 = make_inputs(w128)["r"].to(DEV)
    rb128 = m.make_relbias(r128, m.relproj_pack(make_inputs(w128)["P"].to(DEV)))
    assert m._lib.rba_attn_prefill_fused(ctypes.byref(a), ctypes.byref(rb128), None, 0, st) == m.RBA_E_WORKSPACE
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)   # NaN-like bf16 garbage
    o1 = m.attn_prefill_fused(d["q"], d["k"], d["v"], d["r"], PT, workspace=ws)
    # a different problem through the same workspace, then the first again
    d2 = {k: v.to(DEV) for k, v in make_inputs(w, seed=5).items()}
    m.attn_prefill_fused(d2["q"], d2["k"], d2["v"], d2["r"], m.relproj_pack(d2["P"]), workspace=ws)
    o2 = m.attn_prefill_fused(d["q"], d["k"], d["v"], d["r"], PT, workspace=ws)
    R = m.relproj(d["r"], d["P"])
    ou = m.attn_prefill(d["q"], d["k"], d["v"], R)
    torch.cuda.synchronize()
    assert torch.equal(o1, ou) and torch.equal(o2, ou)


def test_fused_on_chip_needs_no_workspace():
    """r_dim <= 64 with no workspace: the relative logits go straight to LDS;
    two calls in a row (different inputs, then the first again) each equal
    the two-kernel path bit for bit."""
    m = rba()
    w = scaled(CONFIGS["c2_swa_prefill"], B=1, Sq=256, Skv=256, Hq=16, Hkv=2, window=0, E=64)
    outs = []
    for seed in (None, 5, None):
        inp = make_inputs(w) if seed is None else make_inputs(w, seed=seed)
        d = {k: v.to(DEV) for k, v in inp.items()}
        PT = m.relproj_pack(d["P"])
        o = torch.empty_like(d["q"])
        a = m.make_args(d["q"], d["k"], d["v"], None, o, None)
        a.E = w.E
        rb = m.make_relbias(d["r"], PT)
        assert m._lib.rba_attn_prefill_fused(ctypes.byref(a), ctypes.byref(rb), None, 0, m._stream(d["q"].device)) \
            == m.RBA_OK
        ou = m.attn_prefill(d["q"], d["k"], d["v"], m.relproj(d["r"], d["P"]))
        torch.cuda.synchronize()
        assert torch.equal(o, ou)
        outs.append(o)
    assert torch.equal(outs[0], outs[2])
