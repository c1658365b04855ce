"""GPU parity of the paged, variable-length KV path (rba_attn_paged) against
the fp64 oracle.

Every sequence has its own length and its keys sit in randomly assigned pages
of a shared pool.  Rows past a sequence's length in its last page and the
pool's spare pages are filled with NaN, so a read of any key the sequence does
not own shows up as a non-finite output.  Tolerances as in the dense parity
tests: bf16 max|d| <= 2e-2 and mean|d| <= 2e-3; fp32 max|d| <= 1e-5.
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


def check(name, got, want, fp32, extra_tol=None):
    g = got.detach().double().cpu().numpy()
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


def poison(inp, page_size):
    """NaN in every pool row no sequence owns."""
    owned = torch.zeros(inp["k_pool"].shape[:2], dtype=torch.bool)
    for b, L in enumerate(inp["seq_lens"].tolist()):
        for j0 in range(0, L, page_size):
            pg = int(inp["block_table"][b, j0 // page_size])
            owned[pg, :min(page_size, L - j0)] = True
    for name in ("k_pool", "v_pool"):
        inp[name][~owned] = float("nan")
    return inp


def run_paged(inp, w, page_size, splits, R=None, head_major=False):
    """head_major: every page stored [Hkv, page_size, d], passed as a strided
    [page_size, Hkv, d] view."""
    m = rba()
    d = {k: v.to(DEV) for k, v in inp.items()}
    if head_major:
        for n in ("k_pool", "v_pool"):
            d[n] = d[n].transpose(1, 2).contiguous().transpose(1, 2)
    if R is None:
        R = m.relproj(d["r"], d["P"])
    o, lse = m.attn_paged(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], R,
                          max_seq_len=w.Skv, window=w.window, log_scale_base=w.log_scale_base,
                          num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def oracle_paged(inp, w, table=None, lens=None):
    R = oracle.relproj(inp["r"], inp["P"])
    return oracle.attention_paged(inp["q"], inp["k_pool"], inp["v_pool"],
                                  inp["block_table"] if table is None else table,
                                  inp["seq_lens"] if lens is None else lens, R,
                                  window=w.window, log_scale_base=w.log_scale_base)


PAGED_CASES = [
    # name, workload, overrides, page size
    ("decode_full", "c4_decode_full", dict(B=5, Sq=9, Skv=700, Hq=16, Hkv=2, E=64, window=0), 64),
    ("decode_swa_p128", "c4_decode_swa", dict(B=4, Sq=9, Skv=1000, Hq=16, Hkv=2, E=64, window=256), 128),
    ("decode_log_sq1", "c5_long_decode", dict(B=3, Sq=1, Skv=1500, Hq=16, Hkv=2, E=96), 64),
    ("verify_wide_p192", "c4_decode_full", dict(B=2, Sq=40, Skv=600, Hq=16, Hkv=1, E=64, window=0), 192),
    ("swa_log_ragged", "c4_decode_swa", dict(B=3, Sq=5, Skv=777, Hq=8, Hkv=1, E=100, window=300,
                                             log_scale_base=64.0), 64),
    ("fp32", "c1_tiny_fp32", dict(B=3, Sq=4, Skv=300, Hq=4, Hkv=1, E=64), 64),
]


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("name,wname,over,ps", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_paged_parity(name, wname, over, ps, splits):
    w = scaled(CONFIGS[wname], **over)
    say(f"paged {name} page={ps} splits={splits}: {w}")
    inp = poison(make_paged_inputs(w, ps), ps)
    say(f"  seq_lens={inp['seq_lens'].tolist()} pages={inp['k_pool'].shape[0]}")
    o, lse = run_paged(inp, w, ps, splits)
    wo, wl = oracle_paged(inp, w)
    fp32 = w.dtype == "fp32"
    check(f"paged {name}/{splits} o", o, wo, fp32)
    check(f"paged {name}/{splits} lse", lse, wl, True, extra_tol=None if fp32 else 2e-2)


@pytest.mark.parametrize("name,wname,over,ps", PAGED_CASES[:3], ids=[c[0] for c in PAGED_CASES[:3]])
def test_paged_head_major_pages(name, wname, over, ps):
    w = scaled(CONFIGS[wname], **over)
    say(f"paged head-major {name} page={ps}: {w}")
    inp = poison(make_paged_inputs(w, ps), ps)
    for splits in (1, 0):
        o, lse = run_paged(inp, w, ps, splits, head_major=True)
        o_tm, lse_tm = run_paged(inp, w, ps, splits)
        wo, wl = oracle_paged(inp, w)
        check(f"paged head-major {name}/{splits} o", o, wo, False)
        check(f"paged head-major {name}/{splits} lse", lse, wl, True, extra_tol=2e-2)
        assert torch.equal(o, o_tm) and torch.equal(lse, lse_tm)


def test_paged_lengths_at_both_ends():
    """Lengths Sq (the queries alone) and Skv (a full table), and a single page."""
    w = scaled(CONFIGS["c4_decode_full"], B=4, Sq=9, Skv=640, Hq=16, Hkv=2, E=64, window=0)
    inp = poison(make_paged_inputs(w, 64, seq_lens=[9, 640, 64, 65]), 64)
    for splits in (1, 4):
        o, lse = run_paged(inp, w, 64, splits)
        wo, wl = oracle_paged(inp, w)
        check(f"ends/{splits} o", o, wo, False)
        check(f"ends/{splits} lse", lse, wl, True, extra_tol=2e-2)


def test_paged_clamps_lengths_and_table_entries():
    """Device-side values outside their ranges are clamped, never used as
    addresses: a length above Skv reads Skv keys, one below Sq reads Sq keys,
    and a table entry outside [0, num_pages) reads the nearest page."""
    w = scaled(CONFIGS["c4_decode_full"], B=3, Sq=9, Skv=320, Hq=16, Hkv=2, E=64, window=0)
    inp = make_paged_inputs(w, 64, seq_lens=[320, 9, 200], spare_pages=0)
    n_pages = inp["k_pool"].shape[0]
    table = inp["block_table"].clone()
    lens = inp["seq_lens"].clone()
    dev = dict(inp)
    dev["seq_lens"] = torch.tensor([320 + 1000, 3, 200], dtype=torch.int32)
    dev_table = table.clone()
    dev_table[2, 1] = n_pages + 7
    dev_table[2, 2] = -5
    dev["block_table"] = dev_table
    o, lse = run_paged(dev, w, 64, 2)
    want_table = table.clone()
    want_table[2, 1] = n_pages - 1
    want_table[2, 2] = 0
    wo, wl = oracle_paged(inp, w, table=want_table, lens=lens)
    check("clamp o", o, wo, False)
    check("clamp lse", lse, wl, True, extra_tol=2e-2)


def test_paged_equals_dense_bitwise():
    """All lengths equal to Skv: the paged kernel does the dense kernel's
    arithmetic in the same order, so the outputs agree bit for bit."""
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], B=3, Sq=9, Skv=704, Hq=16, Hkv=2, E=64, window=0)
    inp = make_paged_inputs(w, 64, seq_lens=[704] * 3, spare_pages=2)
    # the dense cache holding the same keys
    k = torch.stack([oracle_free_gather(inp["k_pool"], inp["block_table"][b], 704) for b in range(3)])
    v = torch.stack([oracle_free_gather(inp["v_pool"], inp["block_table"][b], 704) for b in range(3)])
    d = {n: t.to(DEV) for n, t in inp.items()}
    R = m.relproj(d["r"], d["P"])
    for splits in (1, 5):
        op, lp = run_paged(inp, w, 64, splits, R=R)
        od, ld = m.attn_decode(d["q"], k.to(DEV), v.to(DEV), R, num_splits=splits, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(op, od), splits
        assert torch.equal(lp, ld), splits


def oracle_free_gather(pool, row, L):
    """Keys 0..L-1 of one sequence as a dense [L, Hkv, d] tensor (indexing only)."""
    ps = pool.shape[1]
    idx = torch.arange(L)
    return pool[row.long()[idx // ps], idx % ps]


def test_paged_full_size_decode_sampled():
    """The decode workload (64 sequences, 9 new tokens, 64 query / 8 kv heads,
    up to 9216 keys) in 64-key pages with lengths drawn from [8192, 9216],
    the splits the heuristic picks; four sequences checked against the oracle."""
    w = CONFIGS["c4_decode_full"]
    g = torch.Generator().manual_seed(77)
    lens = torch.randint(8192, 9217, (w.B,), generator=g).tolist()
    inp = make_paged_inputs(w, 64, seq_lens=lens, spare_pages=0)
    o, lse = run_paged(inp, w, 64, 0)
    R = oracle.relproj(inp["r"], inp["P"])
    for b in (0, 17, 40, 63):
        L = lens[b]
        K = oracle.gather_pages(inp["k_pool"], inp["block_table"][b], L)[None]
        V = oracle.gather_pages(inp["v_pool"], inp["block_table"][b], L)[None]
        wo, wl = oracle.attention(inp["q"][b:b + 1], K, V, R[b:b + 1], window=w.window,
                                  log_scale_base=w.log_scale_base)
        check(f"full-size paged b={b} L={L} o", o[b:b + 1], wo, False)
        check(f"full-size paged b={b} lse", lse[b:b + 1], wl, True, extra_tol=2e-2)
