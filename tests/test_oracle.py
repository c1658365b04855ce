"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The pages define the method in prose only ("SGLang と Miles が Inkling を初日から
サポート", section "相対位置バイアス付き Attention"): they print no worked
example and no numbers for it.  So every pin here is a closed form, a special
case that reduces to a library routine, or brute force on tiny inputs, chosen
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention, attention_paged, attention_partial, attention_rows, brute_attention,
                    e4m3_value, gather_pages, log_scale_factor, lse_combine, mxfp8_dequantize, mxfp8_quantize,
                    relproj)
from oracle import attention_prologue, rms_norm, short_conv
from oracle.rba_oracle import _e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand(shape, seed, std=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * std


def _case(B=1, Sq=7, Skv=7, Hq=4, Hkv=2, d=8, E=5, seed=0):
    q = _rand((B, Sq, Hq, d), seed)
    k = _rand((B, Skv, Hkv, d), seed + 1)
    v = _rand((B, Skv, Hkv, d), seed + 2)
    R = _rand((B, Sq, Hq, E), seed + 3)
    return q, k, v, R


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("window,base,Sq,Skv,E,G", [
    (0, 0.0, 9, 9, 4, 2),
    (3, 0.0, 9, 9, 6, 2),
    (0, 4096.0, 8, 8, 3, 1),
    (4, 16.0, 5, 12, 7, 4),      # decode-like: queries at the bottom-right
    (0, 0.0, 11, 11, 20, 1),     # E larger than every distance
    (1, 0.0, 6, 6, 2, 2),
])
def test_oracle_matches_brute_force(window, base, Sq, Skv, E, G):
    Hkv = 2
    q, k, v, R = _case(B=2, Sq=Sq, Skv=Skv, Hq=Hkv * G, Hkv=Hkv, d=6, E=E, seed=window * 7 + Sq)
    o1, l1 = attention(q, k, v, R, window=window, log_scale_base=base, chunk=4)
    o2, l2 = brute_attention(q, k, v, R, window=window, log_scale_base=base)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_rows_and_partial_agree_with_full():
    q, k, v, R = _case(B=2, Sq=10, Skv=13, Hq=4, Hkv=2, d=8, E=6, seed=5)
    for window, base in ((0, 0.0), (4, 0.0), (0, 64.0)):
        o, l = attention(q, k, v, R, window=window, log_scale_base=base)
        rows = [(0, 0), (1, 9), (0, 5), (1, 3)]
        orow, lrow = attention_rows(q, k, v, R, rows, window=window, log_scale_base=base)
        for i, (b, t) in enumerate(rows):
            assert np.max(np.abs(orow[i] - o[b, t])) <= 1e-13
            assert np.max(np.abs(lrow[i] - l[b, :, t])) <= 1e-13
        op, lp = attention_partial(q, k, v, R, key_lo=0, key_hi=13, window=window, log_scale_base=base)
        assert np.max(np.abs(op - o)) <= 1e-13


# --------------------------------------------------------------------------- library routine

@pytest.mark.parametrize("window,base", [(0, 0.0), (5, 0.0), (0, 4096.0), (3, 100.0)])
def test_zero_bias_equals_sdpa(window, base):
    """With no bias the method is plain causal (windowed) GQA attention:
    torch's scaled_dot_product_attention in fp64 with an explicit mask and the
    kv heads repeated per group.  The log-scale factor is folded into q."""
    B, Sq, Skv, Hq, Hkv, d = 2, 11, 14, 6, 2, 16
    q, k, v, _ = _case(B, Sq, Skv, Hq, Hkv, d, 1, seed=11)
    o, _ = attention(q, k, v, None, window=window, log_scale_base=base)
    o0, _ = attention(q, k, v, np.zeros((B, Sq, Hq, 9)), window=window, log_scale_base=base)
    assert np.max(np.abs(o - o0)) <= 1e-14
    G = Hq // Hkv
    pos = Skv - Sq + np.arange(Sq)
    f = np.ones(Sq) if not base else np.log(pos + 1.0) / math.log(base)
    qt = torch.tensor(q * f[None, :, None, None]).permute(0, 2, 1, 3)
    kt = torch.tensor(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.tensor(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    j = np.arange(Skv)
    dist = pos[:, None] - j[None, :]
    mask = dist >= 0
    if window:
        mask &= dist < window
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.tensor(mask))
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


# --------------------------------------------------------------------------- closed forms

def test_golden_closed_forms():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 5
    for c in cases:
        S = c["S"]
        q = np.zeros((1, S, 1, 1))
        k = np.zeros((1, S, 1, 1))
        v = np.array(c["v"], dtype=np.float64).reshape(1, S, 1, 1)
        E = c["E"]
        R = None
        if E:
            R = np.zeros((1, S, 1, E))
            for dist, val in c["bias"].items():
                R[0, :, 0, int(dist)] = val
        o, lse = attention(q, k, v, R, window=c["window"], log_scale_base=c["log_scale_base"])
        np.testing.assert_allclose(o[0, :, 0, 0], c["o"], rtol=0, atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0, :], c["lse"], rtol=0, atol=1e-13, err_msg=c["name"])


@pytest.mark.parametrize("window,Sq,Skv", [(0, 12, 12), (5, 12, 12), (1, 12, 12), (4, 3, 20), (0, 1, 30)])
def test_uniform_weights_give_visible_mean(window, Sq, Skv):
    """q = k = 0 and R = 0: every visible key has logit 0, so o_t is the mean of
    the visible v (prefix sums) and lse = ln(#visible).  Pins the causal and
    window counting and the bottom-right query alignment."""
    Hq, Hkv, d = 4, 2, 3
    q = np.zeros((1, Sq, Hq, d))
    k = np.zeros((1, Skv, Hkv, d))
    v = _rand((1, Skv, Hkv, d), 3)
    o, lse = attention(q, k, v, np.zeros((1, Sq, Hq, 7)), window=window)
    csum = np.concatenate([np.zeros((1, Hkv, d)), np.cumsum(v[0], axis=0)])
    for t in range(Sq):
        p = Skv - Sq + t
        lo = 0 if window == 0 else max(0, p - window + 1)
        n = p - lo + 1
        for h in range(Hq):
            g = h // (Hq // Hkv)
            mean = (csum[p + 1, g] - csum[lo, g]) / n
            assert np.max(np.abs(o[0, t, h] - mean)) <= 1e-13
            assert abs(lse[0, h, t] - math.log(n)) <= 1e-13


def test_window_one_returns_v_and_first_row_returns_v0():
    q, k, v, R = _case(B=1, Sq=9, Skv=9, Hq=2, Hkv=1, d=5, E=4, seed=21)
    o, lse = attention(q, k, v, R, window=1)
    assert np.max(np.abs(o[0, :, 0] - v[0, :, 0])) == 0.0
    o, lse = attention(q, k, v, R, window=0, log_scale_base=4096.0)
    assert np.max(np.abs(o[0, 0] - v[0, 0, 0][None])) == 0.0


def test_constant_v_gives_constant_output():
    q, k, v, R = _case(B=2, Sq=10, Skv=10, Hq=4, Hkv=2, d=4, E=6, seed=8)
    v = np.ones_like(v) * 3.5
    o, _ = attention(q, k, v, R * 10, window=3, log_scale_base=64.0)
    assert np.max(np.abs(o - 3.5)) <= 1e-13


def test_gqa_grouping_is_contiguous():
    """Query head h reads kv head h // (Hq/Hkv): a constant v per kv head shows it."""
    B, S, Hq, Hkv, d = 1, 6, 8, 4, 2
    q, k, _, R = _case(B, S, S, Hq, Hkv, d, 3, seed=2)
    v = np.zeros((B, S, Hkv, d))
    for g in range(Hkv):
        v[:, :, g, :] = g
    o, _ = attention(q, k, v, R)
    for h in range(Hq):
        assert np.max(np.abs(o[0, :, h] - h // (Hq // Hkv))) <= 1e-13


@pytest.mark.parametrize("dstar,window", [(0, 0), (1, 0), (63, 0), (2, 3), (5, 3)])
def test_one_hot_bias_selects_distance(dstar, window):
    """q = k = 0, R one-hot 30 at distance d*, v coded by position in two
    channels: each row must pick the key at p - d* with weight >= 1 - Skv e^-30
    (or the plain visible mean when no visible key sits at that distance)."""
    S, E, Hq = 300, 64, 2
    q = np.zeros((1, S, Hq, 4))
    k = np.zeros((1, S, 1, 4))
    v = np.zeros((1, S, 1, 4))
    j = np.arange(S)
    v[0, :, 0, 0] = j % 256
    v[0, :, 0, 1] = j // 256
    R = np.zeros((1, S, Hq, E))
    R[..., dstar] = 30.0
    o, _ = attention(q, k, v, R, window=window)
    tol = 256 * S * math.exp(-30.0) * 2
    for t in range(S):
        lo = 0 if window == 0 else max(0, t - window + 1)
        target = t - dstar
        if target >= lo:
            want = v[0, target, 0]
        else:
            want = v[0, lo:t + 1, 0].mean(axis=0)
        for h in range(Hq):
            assert np.max(np.abs(o[0, t, h] - want)) <= tol, (t, h)


@pytest.mark.parametrize("base", [0.0, 4096.0])
def test_shift_invariance_when_window_within_extent(base):
    """Adding c to every R entry adds f(p)*c to every visible logit when W <= E,
    which softmax ignores; when W > E the far keys get no shift, so o moves."""
    q, k, v, R = _case(B=1, Sq=16, Skv=16, Hq=2, Hkv=1, d=8, E=6, seed=4)
    o1, l1 = attention(q, k, v, R, window=6, log_scale_base=base)
    o2, l2 = attention(q, k, v, R + 2.5, window=6, log_scale_base=base)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    f = log_scale_factor(np.arange(16), base)
    assert np.max(np.abs((l2 - l1)[0] - 2.5 * f[None, :])) <= 1e-12
    o3, _ = attention(q, k, v, R, window=0, log_scale_base=base)
    o4, _ = attention(q, k, v, R + 2.5, window=0, log_scale_base=base)
    assert np.max(np.abs(o3 - o4)) > 1e-3


def test_log_scale_factor_closed_form():
    p = np.array([0, 1, 3, 4095, 32767])
    f = log_scale_factor(p, 4096.0)
    assert f[0] == 0.0
    assert abs(f[3] - 1.0) <= 1e-15
    assert abs(f[4] - 15.0 / 12.0) <= 1e-15
    assert abs(f[2] - 2.0 / 12.0) <= 1e-15
    assert np.all(log_scale_factor(p, 0.0) == 1.0)


def test_log_scale_scales_logit_including_bias():
    """Self bias c with q = k = 0 under f(p): the self weight is e^{f(p) c}
    against p unit weights; position-coded v gives a closed form per row."""
    S, c, L = 40, 3.0, 8.0
    q = np.zeros((1, S, 1, 1))
    k = np.zeros((1, S, 1, 1))
    v = np.arange(S, dtype=np.float64).reshape(1, S, 1, 1)
    R = np.zeros((1, S, 1, 2))
    R[..., 0] = c
    o, lse = attention(q, k, v, R, log_scale_base=L)
    for p in range(S):
        w = math.exp(math.log(p + 1.0) / math.log(L) * c)
        want = (w * p + p * (p - 1) / 2.0) / (w + p)
        assert abs(o[0, p, 0, 0] - want) <= 1e-12
        assert abs(lse[0, 0, p] - math.log(w + p)) <= 1e-12


# --------------------------------------------------------------------------- relproj

def test_relproj_one_hot_r_selects_P_row():
    Hq, r_dim, E = 3, 5, 7
    P = _rand((Hq, r_dim, E), 1)
    r = np.zeros((2, 4, r_dim))
    for t in range(4):
        r[0, t, t] = 1.0
        r[1, t, (t + 2) % r_dim] = -2.0
    R = relproj(r, P)
    assert R.shape == (2, 4, Hq, E)
    for t in range(4):
        assert np.array_equal(R[0, t], P[:, t, :])
        assert np.array_equal(R[1, t], -2.0 * P[:, (t + 2) % r_dim, :])


def test_relproj_one_hot_P_selects_r_channel():
    Hq, r_dim, E = 4, 6, 9
    r = _rand((3, 5, r_dim), 2)
    P = np.zeros((Hq, r_dim, E))
    for h in range(Hq):
        P[h, (h + 1) % r_dim, (2 * h) % E] = h + 1.0
    R = relproj(r, P)
    for h in range(Hq):
        want = np.zeros((3, 5, E))
        want[..., (2 * h) % E] = (h + 1.0) * r[..., (h + 1) % r_dim]
        assert np.array_equal(R[:, :, h], want)


def test_relproj_small_brute_force():
    Hq, r_dim, E = 2, 3, 4
    r = _rand((1, 3, r_dim), 3)
    P = _rand((Hq, r_dim, E), 4)
    R = relproj(r, P)
    for t in range(3):
        for h in range(Hq):
            for e in range(E):
                s = 0.0
                for c in range(r_dim):
                    s += r[0, t, c] * P[h, c, e]
                assert abs(R[0, t, h, e] - s) <= 1e-14


def test_relproj_per_head_brute_force_and_shared_case():
    Hq, r_dim, E = 3, 4, 5
    rh = _rand((2, 3, Hq, r_dim), 5)
    P = _rand((Hq, r_dim, E), 6)
    R = relproj(rh, P, per_head=True)
    assert R.shape == (2, 3, Hq, E)
    for b in range(2):
        for t in range(3):
            for h in range(Hq):
                for e in range(E):
                    s = 0.0
                    for c in range(r_dim):
                        s += rh[b, t, h, c] * P[h, c, e]
                    assert abs(R[b, t, h, e] - s) <= 1e-14
    # every head holding the same feature reduces to the shared form
    r = _rand((2, 3, r_dim), 7)
    same = np.repeat(r[:, :, None, :], Hq, axis=2)
    assert np.array_equal(relproj(same, P, per_head=True), relproj(r, P))


# --------------------------------------------------------------------------- combine

@pytest.mark.parametrize("bounds", [[0, 13], [0, 5, 13], [0, 1, 2, 7, 13], [0, 13, 13, 13], [0, 4, 4, 9, 13]])
def test_lse_combine_reassembles_split_softmax(bounds):
    """Softmax over a union of disjoint key ranges equals the lse-weighted merge
    of per-range results; empty ranges (lse = -inf) get weight 0."""
    q, k, v, R = _case(B=2, Sq=4, Skv=13, Hq=4, Hkv=2, d=6, E=5, seed=9)
    for window in (0, 3):
        o, l = attention(q, k, v, R, window=window, log_scale_base=32.0)
        parts = [attention_partial(q, k, v, R, key_lo=a, key_hi=b, window=window, log_scale_base=32.0)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        op = np.stack([p[0] for p in parts])                      # [S, B, Sq, Hq, d]
        lp = np.stack([p[1].transpose(0, 2, 1) for p in parts])   # [S, B, Sq, Hq]
        oc, lc = lse_combine(op, lp)
        assert np.max(np.abs(oc - o)) <= 1e-12
        assert np.max(np.abs(lc - l.transpose(0, 2, 1))) <= 1e-12


def test_lse_combine_all_empty_rows():
    op = np.zeros((3, 2, 4))
    lp = np.full((3, 2), -np.inf)
    o, l = lse_combine(op, lp)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


# --------------------------------------------------------------------------- paged cache

def _scatter_to_pages(dense_seqs, page_size, order, n_pages):
    """Write each sequence's keys page by page into a pool, pages taken in
    ``order``; returns pool [n_pages, page_size, H, d] (unused rows NaN) and
    the table.  The inverse of reading a paged cache, written as stores."""
    H, d = dense_seqs[0].shape[1:]
    pool = np.full((n_pages, page_size, H, d), np.nan)
    n_max = max(-(-len(x) // page_size) for x in dense_seqs)
    table = -np.ones((len(dense_seqs), n_max), dtype=np.int64)
    it = iter(order)
    for b, x in enumerate(dense_seqs):
        for i in range(-(-len(x) // page_size)):
            pg = next(it)
            table[b, i] = pg
            chunk = x[i * page_size:(i + 1) * page_size]
            pool[pg, :len(chunk)] = chunk
    return pool, table


@pytest.mark.parametrize("window,base", [(0, 0.0), (4, 0.0), (0, 100.0)])
def test_paged_matches_brute_force_per_sequence(window, base):
    lens, Sq, Hq, Hkv, d, E, ps = [11, 4, 8], 3, 4, 2, 8, 6, 4
    ks = [_rand((L, Hkv, d), 10 + b) for b, L in enumerate(lens)]
    vs = [_rand((L, Hkv, d), 20 + b) for b, L in enumerate(lens)]
    q = _rand((len(lens), Sq, Hq, d), 30)
    R = _rand((len(lens), Sq, Hq, E), 31)
    order = [5, 0, 7, 2, 6, 3, 1, 4]          # 3 + 1 + 2 pages used, 2 spare
    kp, table = _scatter_to_pages(ks, ps, order, 8)
    vp, table2 = _scatter_to_pages(vs, ps, order, 8)
    assert (table == table2).all()
    o, lse = attention_paged(q, kp, vp, table, lens, R, window=window, log_scale_base=base)
    assert np.isfinite(o).all()
    for b, L in enumerate(lens):
        ob, lb = brute_attention(q[b:b + 1], ks[b][None], vs[b][None], R[b:b + 1], window=window,
                                 log_scale_base=base)
        np.testing.assert_allclose(o[b], ob[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], lb[0], rtol=1e-12, atol=1e-12)


def test_paged_invariant_under_page_relabelling():
    ps, Hkv, d, Sq, Hq = 4, 1, 8, 2, 2
    pool_k = _rand((6, ps, Hkv, d), 40)
    pool_v = _rand((6, ps, Hkv, d), 41)
    table = np.array([[3, 1, 4], [0, 5, -1]])
    lens = [10, 7]
    q = _rand((2, Sq, Hq, d), 42)
    o, lse = attention_paged(q, pool_k, pool_v, table, lens)
    perm = np.array([2, 5, 0, 4, 1, 3])        # page i moves to slot perm[i]
    pk2 = np.empty_like(pool_k)
    pv2 = np.empty_like(pool_v)
    pk2[perm] = pool_k
    pv2[perm] = pool_v
    t2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, lse2 = attention_paged(q, pk2, pv2, t2, lens)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_gather_pages_reads_rows_in_key_order():
    # page p row i holds the value 100 p + i: key j of a sequence is then
    # 100 table[j // ps] + j % ps
    ps = 4
    pool = (100 * np.arange(5)[:, None] + np.arange(ps)[None, :]).astype(float)[:, :, None, None]
    got = gather_pages(pool, [3, 0, 4], 10)[:, 0, 0]
    assert list(got) == [300, 301, 302, 303, 0, 1, 2, 3, 400, 401]


# --------------------------------------------------------------------------- MXFP8 (OCP MX v1.0)

def test_e4m3_table_closed_forms():
    v = e4m3_value(np.arange(256))
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x7E] == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    assert v[0x80] == 0.0 and np.signbit(v[0x80]) and v[0xB8] == -1.0 and v[0xFE] == -448.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # 127 increasing non-negative values
    assert np.array_equal(v[0x80:0xFF], -pos)


def _nearest_code(x):
    """Brute force: the finite E4M3 code nearest to x (x clamped to +-448),
    ties to the even code (even mantissa), zero keeping x's sign."""
    tab = e4m3_value(np.arange(256))
    xc = min(max(x, -448.0), 448.0)
    best, bd = None, None
    for c in range(256):
        v = tab[c]
        if np.isnan(v) or (v == 0 and bool(c & 0x80) != bool(np.signbit(xc))):
            continue
        d = abs(v - xc)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best


def test_e4m3_encode_matches_brute_force():
    tab = e4m3_value(np.arange(256))
    fin = tab[~np.isnan(tab)]
    pos = np.sort(fin[fin > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(5)
    xs = np.concatenate([fin, mids, -mids, np.nextafter(mids, 1e9), np.nextafter(mids, -1e9),
                         rng.standard_normal(300) * 50, rng.standard_normal(100) * 1e-2,
                         [449.0, 463.9, 464.0, 464.1, 500.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10, -(2.0 ** -10),
                          3 * 2.0 ** -11, 1e-30]])
    got = _e4m3_encode(xs)
    for x, g in zip(xs, got):
        assert int(g) == _nearest_code(float(x)), (x, g)


def test_mxfp8_scale_rule_closed_forms():
    def scale_of(block):
        _, s = mxfp8_quantize(np.asarray(block, dtype=np.float64)[None, :])
        return int(s[0, 0])
    ones = np.ones(32)
    assert scale_of(ones) == 127 - 8                      # amax 1 = 2^0 -> e = -8
    assert scale_of(ones * 1.999) == 127 - 8
    assert scale_of(ones * 2.0) == 127 - 7
    assert scale_of(ones * 0.75) == 127 - 9               # floor(log2 0.75) = -1
    assert scale_of(np.zeros(32)) == 0                    # all-zero block
    assert scale_of(ones * 2.0 ** -140) == 0              # clamped at e = -127
    assert scale_of(ones * 2.0 ** 200) == 254             # clamped at e = 127
    b = np.zeros(32)
    b[7] = -3.0                                           # the sign does not matter
    assert scale_of(b) == 127 + 1 - 8


def test_mxfp8_roundtrip_and_saturation():
    # values on the grid of a common scale survive exactly
    e = -5
    tab = e4m3_value(np.arange(256))
    fin = tab[~np.isnan(tab)]
    rng = np.random.default_rng(9)
    block = rng.choice(fin[np.abs(fin) <= 448], 32) * 2.0 ** e
    block[0] = 288.0 * 2.0 ** e                           # amax in [256, 512) * 2^e -> scale 2^e; 288 is on the grid
    c, s = mxfp8_quantize(block[None, :])
    assert int(s[0, 0]) == e + 127
    assert np.array_equal(mxfp8_dequantize(c, s)[0], block)
    # amax in (464, 512) * 2^e saturates to 448 * 2^e
    sat = np.full(32, 0.5)
    sat[3] = 1.9                                          # 1.9 / 2^-8 = 486.4 > 448
    c, s = mxfp8_quantize(sat[None, :])
    d = mxfp8_dequantize(c, s)[0]
    assert d[3] == 448.0 * 2.0 ** -8 and d[0] == 0.5


def test_mxfp8_error_bound_and_brute_force():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 128)) * np.array([1e-3, 0.1, 1, 10, 1e3, 1e5])[:, None]
    x[2, 32:64] = 0.0
    c, s = mxfp8_quantize(x)
    d = mxfp8_dequantize(c, s)
    for r in range(6):
        for k in range(4):
            blk = x[r, 32 * k:32 * k + 32]
            e = int(s[r, k]) - 127
            for i in range(32):
                # brute force per element, scale taken from the rule
                want = e4m3_value(_nearest_code(blk[i] / 2.0 ** e)) * 2.0 ** e
                assert d[r, 32 * k + i] == want
                # half a quantum of the element's binade (3 mantissa bits), or of the subnormal step
                v = abs(blk[i]) / 2.0 ** e
                if v <= 448:
                    q = 2.0 ** (max(np.floor(np.log2(v)) if v > 0 else -6, -6) - 3)
                    assert abs(d[r, 32 * k + i] - blk[i]) <= 0.5 * q * 2.0 ** e * (1 + 1e-12)


# --------------------------------------------------------------------------- attention prologue

def test_short_conv_taps_identity_shift_and_brute_force():
    rng = np.random.default_rng(21)
    n, C, W = 6, 5, 4
    x = rng.standard_normal((n, C))
    hist = rng.standard_normal((W - 1, C))
    w = np.zeros((C, W))
    w[:, 0] = 1.0
    assert np.array_equal(short_conv(x, w, hist), x)                 # tap 0 is the current row
    w = np.zeros((C, W))
    w[:, 2] = 1.0                                                     # two rows back
    y = short_conv(x, w, hist)
    assert np.array_equal(y[2:], x[:-2]) and np.array_equal(y[:2], hist[1:])
    w = rng.standard_normal((C, W))
    y = short_conv(x, w, hist)
    rows = list(hist) + list(x)
    for t in range(n):
        for c in range(C):
            want = 0.0
            for i in range(W):
                want += w[c, i] * rows[W - 1 + t - i][c]
            assert abs(y[t, c] - want) <= 1e-12


def test_rms_norm_closed_forms():
    g = np.linspace(0.5, 2.0, 8)
    x = np.full((3, 8), 2.0)
    y = rms_norm(x, g, 0.0)
    assert np.allclose(y, np.broadcast_to(g, (3, 8)), rtol=0, atol=1e-15)   # constant rows -> g
    rng = np.random.default_rng(22)
    x = rng.standard_normal((4, 128))
    y = rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(rms_norm(7.5 * x, np.ones(128), 0.0), y, rtol=0, atol=1e-12)   # scale invariant
    eps = 0.3
    y = rms_norm(np.ones((1, 4)), np.ones(4), eps)
    assert np.allclose(y, 1.0 / np.sqrt(1.0 + eps), rtol=0, atol=1e-15)


def _prologue_case(seed, lens_new, lens_total, Hq=4, Hkv=2, d=8, W=4):
    rng = np.random.default_rng(seed)
    T = sum(lens_new)
    B = len(lens_new)
    cu = np.concatenate([[0], np.cumsum(lens_new)])
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    wk = rng.standard_normal((Hkv * d, W))
    wv = rng.standard_normal((Hkv * d, W))
    gq = rng.standard_normal(d)
    gk = rng.standard_normal(d)
    sk = rng.standard_normal((B, W - 1, Hkv, d))
    sv = rng.standard_normal((B, W - 1, Hkv, d))
    return q, k, v, cu, np.array(lens_total), wk, wv, gq, gk, sk, sv


def test_prologue_split_into_two_calls_equals_one():
    q, k, v, cu, L, wk, wv, gq, gk, sk, sv = _prologue_case(23, [5, 3], [12, 3])
    full = attention_prologue(q, k, v, cu, L, wk, wv, gq, gk, 1e-6, sk, sv)
    # first call: 2 and 1 new tokens; second call: the remaining 3 and 2
    idx1 = [0, 1, 5]
    idx2 = [2, 3, 4, 6, 7]
    p1 = attention_prologue(q[idx1], k[idx1], v[idx1], [0, 2, 3], [9, 1], wk, wv, gq, gk, 1e-6, sk, sv)
    p2 = attention_prologue(q[idx2], k[idx2], v[idx2], [0, 3, 5], [12, 3], wk, wv, gq, gk, 1e-6, p1[4], p1[5])
    for out in (0, 1, 2):
        got = np.zeros_like(full[out])
        got[idx1] = p1[out]
        got[idx2] = p2[out]
        assert np.allclose(got, full[out], rtol=0, atol=1e-12)
    assert np.array_equal(np.concatenate([p1[3], p2[3]])[np.argsort(idx1 + idx2)], full[3])
    assert np.allclose(p2[4], full[4]) and np.allclose(p2[5], full[5])


def test_prologue_sequence_start_ignores_history_and_places_rows():
    # sequence 1 starts at position 0 (3 new tokens, length 3): its state must not matter
    q, k, v, cu, L, wk, wv, gq, gk, sk, sv = _prologue_case(24, [2, 3], [10, 3])
    a = attention_prologue(q, k, v, cu, L, wk, wv, gq, gk, 1e-6, sk, sv)
    sk2, sv2 = sk.copy(), sv.copy()
    sk2[1] = 1e3
    sv2[1] = -1e3
    b = attention_prologue(q, k, v, cu, L, wk, wv, gq, gk, 1e-6, sk2, sv2)
    assert np.array_equal(a[1][2:], b[1][2:]) and np.array_equal(a[2][2:], b[2][2:])
    assert list(a[3]) == [8, 9, 0, 1, 2]
    # V of the first row of sequence 1 is tap 0 times the row itself
    assert np.allclose(a[2][2], wv[:, 0].reshape(2, 8) * v[2], rtol=0, atol=1e-12)


def test_prologue_composition_closed_forms():
    """The order of the prologue's steps, from values worked out by hand.

    K is convolved first and normalised after ("SGLang と Miles が Inkling を
    初日からサポート", section "Inkling のモデルアーキテクチャ": the K
    ShortConv sits between the K projection and the Q/K normalisation); V is
    convolved only; q is normalised with its own weight.  With taps 1 on the
    current row and on the row one position back, a history row u and a new
    row c*u (c > 0):
      * convolve then normalise: g_k * (1+c)u / rms((1+c)u) = g_k * u / rms(u);
      * normalise then convolve would give 2 * g_k * u / rms(u).
    u alternates +-1, so rms(u) = 1 and the K row must equal g_k * u exactly;
    the V row (taps the same) must equal (1+c) * w for history row w and new
    row c*w.  A constant q row 3 normalises to g_q exactly (eps = 0), which
    tells g_q from g_k."""
    Hq, Hkv, d, W = 2, 1, 8, 4
    c = 3.0
    u = np.array([1.0, -1.0] * (d // 2))
    w = np.arange(1.0, d + 1.0)
    gq = np.linspace(0.5, 1.2, d)
    gk = np.linspace(2.0, -1.0, d)
    taps = np.zeros((Hkv * d, W))
    taps[:, 0] = 1.0
    taps[:, 1] = 1.0
    sk = np.zeros((1, W - 1, Hkv, d))
    sv = np.zeros((1, W - 1, Hkv, d))
    sk[0, W - 2, 0] = u          # the row one position before the new token
    sv[0, W - 2, 0] = w
    sk[0, 0, 0] = 50.0           # three back: tap 0 there, so it must not show
    q = np.full((1, Hq, d), 3.0)
    k = (c * u).reshape(1, Hkv, d)
    v = (c * w).reshape(1, Hkv, d)
    q_out, k_rows, v_rows, pos, _, _ = attention_prologue(q, k, v, [0, 1], [10], taps, taps, gq, gk, 0.0, sk, sv)
    assert np.allclose(k_rows[0, 0], gk * u, rtol=0, atol=1e-14)
    assert not np.allclose(k_rows[0, 0], 2.0 * gk * u, rtol=0, atol=1e-3)
    assert np.allclose(v_rows[0, 0], (1.0 + c) * w, rtol=0, atol=1e-13)
    assert np.allclose(q_out[0], np.broadcast_to(gq, (Hq, d)), rtol=0, atol=1e-14)
    assert list(pos) == [9]


# --------------------------------------------------------------------------- MXFP8 logits

def test_mxfp8_logits_closed_form_quantizes_q():
    """One query, two keys, hand-worked.  q's first block is (1.1, 0, ...): its
    shared exponent is floor(log2 1.1) - 8 = -8 and 1.1 * 2^8 = 281.6 rounds
    to the E4M3 value 288, so the decoded entry is 1.125.  k0 = e_0 (exact in
    E4M3), k1 = 0, v0 = e_0, v1 = e_1: o = (sigmoid(x), 1 - sigmoid(x), 0, ...)
    with x = 1.125 / sqrt(128), and lse = ln(e^x + 1).  Unquantized q (1.1)
    would give a different o, so the pin tells an encoded q from a raw one.
    A second head whose q is 1e5 in its first entry checks that blocks stay
    within a head's 128 entries: sharing a block with it would give head 0
    the exponent 16 - 8 = 8, and 1.1 / 2^8 would round to the subnormal
    2 * 2^-9, i.e. a decoded 1.0 instead of 1.125."""
    from oracle import attention_mxfp8_logits, mxfp8_quantize
    d = 128
    q = np.zeros((1, 1, 2, d))
    q[0, 0, 0, 0] = 1.1
    q[0, 0, 1, 0] = 1e5
    k = np.zeros((1, 2, 1, d))
    k[0, 0, 0, 0] = 1.0
    v = np.zeros((1, 2, 1, d))
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    kc, ks = mxfp8_quantize(k)
    vc, vs = mxfp8_quantize(v)
    o, lse = attention_mxfp8_logits(q, kc, ks, vc, vs)
    x = 1.125 / math.sqrt(d)
    w0 = 1.0 / (1.0 + math.exp(-x))
    assert abs(o[0, 0, 0, 0] - w0) <= 1e-12 and abs(o[0, 0, 0, 1] - (1.0 - w0)) <= 1e-12
    assert abs(lse[0, 0, 0] - math.log(math.exp(x) + 1.0)) <= 1e-12
    raw = 1.0 / (1.0 + math.exp(-1.1 / math.sqrt(d)))
    assert abs(o[0, 0, 0, 0] - raw) > 1e-4
    # head 1: exponent 8, 1e5 / 2^8 = 390.6 rounds to 384: decoded 98304, all weight on key 0
    assert abs(lse[0, 1, 0] - 98304.0 / math.sqrt(d)) <= 1e-9


def test_mxfp8_logits_on_grid_q_is_plain_attention_over_decoded_cache():
    """q already on the MXFP8 grid (encoded and decoded once) is left as it is,
    so the result equals attention over the decoded cache exactly."""
    from oracle import attention_mxfp8_logits, mxfp8_dequantize, mxfp8_quantize
    rng = np.random.default_rng(31)
    B, Sq, Skv, Hq, Hkv, d, E = 2, 5, 40, 4, 2, 128, 16
    x = rng.standard_normal((B, Sq, Hq, d)) * np.exp2(rng.integers(-3, 4, size=(B, Sq, Hq, 1)))
    q = mxfp8_dequantize(*mxfp8_quantize(x))
    kc, ks = mxfp8_quantize(rng.standard_normal((B, Skv, Hkv, d)))
    vc, vs = mxfp8_quantize(rng.standard_normal((B, Skv, Hkv, d)))
    R = rng.standard_normal((B, Sq, Hq, E)) * 0.3
    got = attention_mxfp8_logits(q, kc, ks, vc, vs, R, window=17, log_scale_base=64.0)
    want = attention(q, mxfp8_dequantize(kc, ks), mxfp8_dequantize(vc, vs), R, window=17, log_scale_base=64.0)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    # and an off-grid q does change the result
    got2 = attention_mxfp8_logits(x, kc, ks, vc, vs, R, window=17, log_scale_base=64.0)
    plain = attention(x, mxfp8_dequantize(kc, ks), mxfp8_dequantize(vc, vs), R, window=17, log_scale_base=64.0)
    assert np.max(np.abs(got2[0] - plain[0])) > 1e-4
