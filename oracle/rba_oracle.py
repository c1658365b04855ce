"""fp64 CPU oracle for relative-position-bias attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only thing both sides take from a common place is the seeded
input draws in ``workloads/``.

Sources, cited by page title and section (the pages give the definition in
prose only; no listing, worked example or numbers exist for this path):
  [S-RPB]  "SGLang と Miles が Inkling を初日からサポート" (winzheng.jp),
           section "相対位置バイアス付き Attention".  Every query token has a
           relative feature r besides q, k, v; a learned per-head matrix P
           maps r to relative logits indexed by causal-distance bucket; for
           query i, key j and head h the logit is the scaled dot product plus
           the bias picked by the distance i-j; distances past rel_extent add
           no bias; future keys stay causally masked.  The same section mixes
           sliding-window and full-attention layers, and full-attention layers
           may scale logits by a length-dependent log factor.
  [S-ARCH] same page, section "Inkling のモデルアーキテクチャ": the bias
           module (RelLogitsProj) adds a query-conditioned relative bias to the
           attention logits in place of a positional embedding.
  [V-ARCH] "vLLM TML Inkling サポート" (agentlenshq.com), section
           "TML Inkling モデルアーキテクチャ": GQA with head size 128 in every
           layer; the relative term is added to the logits before softmax.
  [S-SC]   "SGLang と Miles が Inkling を初日からサポート", sections "Inkling の
           モデルアーキテクチャ", "ShortConv：4カ所に現れる短距離因果畳み込み" and
           "ShortConv 最適化": ShortConv is a per-channel causal convolution
           along the tokens that reads the current token and the W-1 before
           it (W = 4); in attention it runs on the K stream after the K
           projection and before the Q/K normalisation, and on the V stream
           after the V projection; SGLang fuses the K/V convolutions, the Q/K
           RMSNorm and the KV-cache write into one attention-prologue kernel.
  [V-KV]   same page, section "vLLM テクニカル最適化": the serving engine
           keeps the caches of all layers in one unified KV cache manager and
           re-runs the multi-token-prediction heads over accepted tokens.
  [S-FA4]  "SGLang と Miles が Inkling を初日からサポート", section "Relative
           Attention と FA4 経路": the attention kernel runs in an MXFP8
           configuration together with the sheared bias.  [V-FP8] "vLLM TML
           Inkling サポート", section on future work: FP8 for global attention
           to relieve compute and KV-cache limits.  MXFP8 itself is the OCP
           Microscaling Formats (MX) v1.0 specification: blocks of 32 elements
           share a power-of-two scale (E8M0), elements are FP8 E4M3.

Readings taken where the pages leave a step open (each is one line in the
design notes):
  * r is one vector per token shared by all heads; P is one matrix per query
    head, P[h] of shape [r_dim, E].  (relproj also takes one r per head,
    the other reading, for callers whose r is per head.)
  * The bucket of distance p-j is p-j itself; R has exactly E entries and
    distances >= E get bias 0.
  * scale multiplies q.k only; the bias is added unscaled.
  * Log-scale factor f(p) = ln(p+1)/ln(base) multiplies the whole logit
    (dot + bias); base = 0 turns it off.
  * Window W > 0: key j visible iff 0 <= p-j < W.  W = 0: full causal.
  * Query row t sits at position p = Skv - Sq + t.
  * GQA: query head h reads kv head h // (Hq/Hkv).
  * MXFP8 ([S-FA4], OCP MX v1.0): a block's shared exponent is
    floor(log2(amax)) - 8 (8 = exponent of E4M3's largest normal, 448),
    clamped to [-127, 127], and -127 for an all-zero block; each element is
    x / 2^e rounded to the nearest E4M3 value, ties to even, saturated to
    +-448.  K and V are blocked along the head dimension (32 entries), and
    attention with an MXFP8 cache is the attention over the decoded values.
  * MXFP8 logits ([S-FA4]: the attention kernel itself runs in MXFP8; [V-FP8]
    names FP8 attention against compute limits): in that mode q is encoded
    the same way (blocks of 32 along the head dimension, the same rule) and
    the logits are the dot products of the decoded q and the decoded K; the
    probabilities and V stay as in the plain MXFP8-cache reading.
  * Attention prologue ([S-SC]): ShortConv tap i multiplies the row i
    positions back (tap 0 = the current token), no bias, no activation;
    positions before a sequence's start read zero.  RMSNorm is
    x / sqrt(mean(x^2) + eps) * g over the 128 entries of one head, with one
    weight vector g per stream (q or k) shared by the heads.  K is
    normalised after its convolution; V is convolved only; Q is normalised
    only.  The conv state of a sequence holds the pre-convolution rows of
    its last W-1 positions.
  * Paged cache ([V-KV]): sequence b has its own length L_b; its key j is row
    j % page_size of page block_table[b][j // page_size] of a shared pool;
    its Sq query rows are its last Sq positions, L_b - Sq + t.

Pins (tests/test_oracle.py): brute force on tiny shapes; R = 0 against
torch's scaled_dot_product_attention in fp64; closed forms for uniform
weights (mean of visible v, lse = ln n), single visible key, one-hot bias
with position-coded v, shift invariance when W <= E, and the log-scale factor
through a two-level closed form.  The LSE combine is pinned by splitting a
full oracle result over key ranges and recombining.  Paged attention is
pinned by brute force on a hand-built page layout, by a permuted pool equal
to the dense result, and by invariance under relabelling the pages.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "relproj",
    "log_scale_factor",
    "attention",
    "attention_rows",
    "attention_partial",
    "lse_combine",
    "brute_attention",
    "gather_pages",
    "attention_paged",
    "e4m3_value",
    "short_conv",
    "rms_norm",
    "attention_prologue",
    "mxfp8_quantize",
    "mxfp8_dequantize",
    "attention_mxfp8_logits",
]


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast its exact values
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def relproj(r, P, per_head=False):
    """R[..., h, e] = sum_c r[..., c] * P[h, c, e]   ([S-RPB]: P projects r to
    per-head relative logits).  r: [..., r_dim]; P: [Hq, r_dim, E].
    per_head: r is [..., Hq, r_dim], one feature per head (the alternative
    reading of r's shape), and R[..., h, e] = sum_c r[..., h, c] * P[h, c, e]."""
    r = _f64(r)
    P = _f64(P)
    Hq, r_dim, E = P.shape
    if per_head:
        lead = r.shape[:-2]
        flat = r.reshape(-1, Hq, r_dim)
        out = np.empty((flat.shape[0], Hq, E), dtype=np.float64)
        for h in range(Hq):
            out[:, h, :] = flat[:, h, :] @ P[h]
        return out.reshape(*lead, Hq, E)
    flat = r.reshape(-1, r_dim)
    out = np.empty((flat.shape[0], Hq, E), dtype=np.float64)
    for h in range(Hq):
        out[:, h, :] = flat @ P[h]
    return out.reshape(*r.shape[:-1], Hq, E)


def log_scale_factor(p, base: float):
    """f(p) = ln(p+1)/ln(base) for the full-attention log-scale ([S-RPB]); 1 if off."""
    p = np.asarray(p, dtype=np.float64)
    if not base:
        return np.ones_like(p)
    return np.log(p + 1.0) / math.log(base)


def _attend(qrows, prow, K, V, Rrows, *, window, scale, log_scale_base, key_pos=None,
            key_lo=None, key_hi=None):
    """Core definition for one head.

    qrows [n, d]; prow [n] absolute query positions; K/V [m, d] the keys at
    absolute positions key_pos (default 0..m-1); Rrows [n, E] or None.  Keys
    outside [key_lo, key_hi) count as not visible (one split of a split-KV
    decode).  Returns (o [n, d], lse [n]); a row with no visible key gets
    o = 0 and lse = -inf.
    """
    j = np.arange(K.shape[0]) if key_pos is None else np.asarray(key_pos)
    dist = prow[:, None] - j[None, :]                      # causal distance p - j
    vis = dist >= 0                                        # future keys masked
    if window > 0:
        vis &= dist < window                               # sliding window: W keys incl. self
    if key_lo is not None:
        vis &= j[None, :] >= key_lo
    if key_hi is not None:
        vis &= j[None, :] < key_hi
    s = scale * (qrows @ K.T)                              # scaled dot product
    if Rrows is not None and Rrows.shape[1] > 0:
        E = Rrows.shape[1]
        in_ext = vis & (dist < E)                          # distances >= E add nothing
        idx = np.clip(dist, 0, E - 1)
        bias = np.take_along_axis(Rrows, idx, axis=1)      # entry for distance p - j
        s = s + np.where(in_ext, bias, 0.0)
    f = log_scale_factor(prow, log_scale_base)
    s = s * f[:, None]                                     # log-scale multiplies the whole logit
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    w = np.exp(s - m_safe[:, None])                        # masked keys -> exactly 0
    l = w.sum(axis=1)
    o = np.zeros((qrows.shape[0], V.shape[1]), dtype=np.float64)
    o[has] = (w[has] @ V) / l[has, None]
    lse = np.full(qrows.shape[0], -np.inf)
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def _prep(q, k, v, R, scale):
    q, k, v, R = _f64(q), _f64(k), _f64(v), _f64(R)
    B, Sq, Hq, d = q.shape
    Bk, Skv, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    if R is not None and R.shape[:3] != (B, Sq, Hq):
        raise ValueError("R must be [B, Sq, Hq, E]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return q, k, v, R, scale


def attention(q, k, v, R=None, *, window=0, scale=None, log_scale_base=0.0, chunk=512):
    """Full oracle.  q [B,Sq,Hq,d], k/v [B,Skv,Hkv,d], R [B,Sq,Hq,E] or None.

    Returns o [B,Sq,Hq,d] and lse [B,Hq,Sq] (natural log), both fp64.
    """
    q, k, v, R, scale = _prep(q, k, v, R, scale)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    pos = Skv - Sq + np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t0 in range(0, Sq, chunk):
                t1 = min(t0 + chunk, Sq)
                Rr = None if R is None else R[b, t0:t1, h]
                oo, ll = _attend(q[b, t0:t1, h], pos[t0:t1], k[b, :, g], v[b, :, g], Rr,
                                 window=window, scale=scale, log_scale_base=log_scale_base)
                o[b, t0:t1, h] = oo
                lse[b, h, t0:t1] = ll
    return o, lse


def attention_rows(q, k, v, R=None, rows=(), *, window=0, scale=None, log_scale_base=0.0):
    """Oracle on selected query rows only.  rows: iterable of (b, t).

    Returns o [n, Hq, d] and lse [n, Hq] for the rows in the given order.
    q/k/v may be torch tensors of any float dtype (their exact values are
    upcast).  R is [B, Sq, Hq, E], or a callable (b, t) -> [Hq, E], or None.
    Only keys that can be visible to the selected rows are upcast.
    """
    rows = list(rows)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((len(rows), Hq, d))
    lse = np.zeros((len(rows), Hq))
    by_b = {}
    for i, (b, t) in enumerate(rows):
        by_b.setdefault(int(b), []).append((i, int(t)))
    for b, items in by_b.items():
        idx = [i for i, _ in items]
        ts = [t for _, t in items]
        prow = np.array([Skv - Sq + t for t in ts])
        qb = np.stack([_f64(q[b, t]) for t in ts])          # [n, Hq, d]
        if R is None:
            Rb = None
        elif callable(R):
            Rb = np.stack([_f64(R(b, t)) for t in ts])       # [n, Hq, E]
        else:
            Rb = np.stack([_f64(R[b, t]) for t in ts])
        lo = 0 if window == 0 else max(0, int(prow.min()) - window + 1)
        hi = int(prow.max()) + 1
        kpos = np.arange(lo, hi)
        for g in range(Hkv):
            Kg = _f64(k[b, lo:hi, g])
            Vg = _f64(v[b, lo:hi, g])
            for hh in range(G):
                h = g * G + hh
                oo, ll = _attend(qb[:, h], prow, Kg, Vg, None if Rb is None else Rb[:, h],
                                 window=window, scale=scale, log_scale_base=log_scale_base,
                                 key_pos=kpos)
                o[idx, h] = oo
                lse[idx, h] = ll
    return o, lse


def attention_partial(q, k, v, R=None, *, key_lo, key_hi, window=0, scale=None, log_scale_base=0.0):
    """Attention restricted to keys in [key_lo, key_hi): one split of a split-KV
    decode.  Returns (o, lse) like ``attention``; rows with no visible key in
    the range give o = 0 and lse = -inf."""
    q, k, v, R, scale = _prep(q, k, v, R, scale)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    pos = Skv - Sq + np.arange(Sq)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            Rr = None if R is None else R[b, :, h]
            oo, ll = _attend(q[b, :, h], pos, k[b, :, g], v[b, :, g], Rr, window=window, scale=scale,
                             log_scale_base=log_scale_base, key_lo=key_lo, key_hi=key_hi)
            o[b, :, h] = oo
            lse[b, h] = ll
    return o, lse


def lse_combine(o_parts, lse_parts):
    """Merge split partials: o_parts [S, ...rows, d] (each normalised within its
    split), lse_parts [S, ...rows].  Splits with lse = -inf get weight 0.
    Returns (o [...rows, d], lse [...rows])."""
    o_parts = _f64(o_parts)
    lse_parts = _f64(lse_parts)
    M = lse_parts.max(axis=0)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse_parts - M_safe[None])                 # exp(-inf) = 0
    den = w.sum(axis=0)
    num = (w[..., None] * o_parts).sum(axis=0)
    ok = den > 0
    o = np.zeros_like(num)
    o[ok] = num[ok] / den[ok][..., None]
    lse = np.full(M.shape, -np.inf)
    lse[ok] = M_safe[ok] + np.log(den[ok])
    return o, lse


def brute_attention(q, k, v, R=None, *, window=0, scale=None, log_scale_base=0.0):
    """Pure-Python loops over (b, h, t, j).  Tiny shapes only."""
    q, k, v, R, scale = _prep(q, k, v, R, scale)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    E = 0 if R is None else R.shape[3]
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for t in range(Sq):
                p = Skv - Sq + t
                f = (math.log(p + 1.0) / math.log(log_scale_base)) if log_scale_base else 1.0
                logits = []
                for j in range(Skv):
                    dist = p - j
                    if dist < 0 or (window > 0 and dist >= window):
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += q[b, t, h, c] * k[b, j, g, c]
                    bias = R[b, t, h, dist] if (R is not None and dist < E) else 0.0
                    logits.append((j, f * (scale * dot + bias)))
                m = max(x for _, x in logits)
                den = sum(math.exp(x - m) for _, x in logits)
                for c in range(d):
                    o[b, t, h, c] = sum(math.exp(x - m) * v[b, j, g, c] for j, x in logits) / den
                lse[b, h, t] = m + math.log(den)
    return o, lse


def gather_pages(pool, table_row, length):
    """Keys 0 .. length-1 of one sequence from a paged pool ([V-KV] reading):
    key j is row j % page_size of page table_row[j // page_size].
    pool [num_pages, page_size, Hkv, d] -> [length, Hkv, d] (fp64)."""
    table_row = np.asarray(table_row, dtype=np.int64)
    ps = pool.shape[1]
    j = np.arange(int(length))
    return _f64(pool[table_row[j // ps], j % ps])   # pick the rows, then upcast them


def attention_paged(q, k_pool, v_pool, block_table, seq_lens, R=None, *, window=0, scale=None,
                    log_scale_base=0.0):
    """Attention of each sequence's last Sq query rows over its own paged keys.

    q [B,Sq,Hq,d]; k_pool/v_pool [num_pages, page_size, Hkv, d];
    block_table [B, n_max] page indices; seq_lens [B] with Sq <= L_b.
    Sequence b is the dense problem over keys gather_pages(pool, table[b], L_b),
    its query row t at position L_b - Sq + t.  Returns o [B,Sq,Hq,d] and
    lse [B,Hq,Sq] like ``attention``.
    """
    q = _f64(q)
    R = _f64(R)
    B, Sq, Hq, d = q.shape
    o = np.zeros((B, Sq, Hq, d))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        L = int(seq_lens[b])
        if L < Sq:
            raise ValueError("a sequence must hold its own query rows")
        Kb = gather_pages(k_pool, block_table[b], L)[None]
        Vb = gather_pages(v_pool, block_table[b], L)[None]
        ob, lb = attention(q[b:b + 1], Kb, Vb, None if R is None else R[b:b + 1], window=window,
                           scale=scale, log_scale_base=log_scale_base)
        o[b] = ob[0]
        lse[b] = lb[0]
    return o, lse


# --------------------------------------------------------------------------- MXFP8 (OCP MX v1.0, E4M3 elements)

E4M3_MAX = 448.0          # largest finite E4M3 value, 1.75 * 2^8
E4M3_EMAX = 8             # its exponent
MX_BLOCK = 32             # elements per shared scale


def e4m3_value(code):
    """Value of an OCP E4M3 bit pattern (sign, 4-bit exponent with bias 7,
    3-bit mantissa; exponent field 0 is subnormal, S.1111.111 is NaN, no
    infinities).  Works elementwise on integer arrays."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    ef = (code >> 3) & 0xF
    m = (code & 0x7).astype(np.float64)
    val = np.where(ef == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, ef - 7))
    val = np.where((ef == 15) & ((code & 7) == 7), np.nan, val)
    return sign * val


def _e4m3_encode(v):
    """E4M3 code of each fp64 value v: nearest representable value, ties to
    the even mantissa, magnitudes saturated to 448; -0 keeps its sign."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    # quantum: 2^(floor(log2 a) - 3) for normal magnitudes, 2^-9 below 2^-6
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    q = np.round(a / quantum) * quantum                  # numpy rounds half to even
    q = np.minimum(q, E4M3_MAX)
    # bit pattern of q
    _, qx = np.frexp(np.where(q > 0, q, 1.0))
    qe = qx - 1
    normal = q >= 2.0 ** -6
    field = np.where(normal, qe + 7, 0)
    mant = np.where(normal, q / np.ldexp(1.0, qe) * 8.0 - 8.0, q / 2.0 ** -9)
    code = (field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(q == 0, 0, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(x):
    """MXFP8 encoding of x [..., n] (n a multiple of 32) along its last axis.

    Returns (codes uint8 [..., n], scales uint8 [..., n/32]) where scales
    hold the E8M0 codes e + 127 of the shared exponents."""
    x = _f64(x)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    blocks = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # floor(log2 amax) = ex - 1
    e = np.where(amax > 0, ex - 1 - E4M3_EMAX, -127)
    e = np.clip(e, -127, 127)
    scaled = blocks / np.ldexp(1.0, e)[..., None]
    codes = _e4m3_encode(scaled).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales):
    """Decoded values (fp64) of MXFP8 codes [..., n] with scales [..., n/32]."""
    codes = np.asarray(codes)
    scales = np.asarray(scales).astype(np.int64)
    n = codes.shape[-1]
    vals = e4m3_value(codes).reshape(*codes.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    s = np.where(scales == 255, np.nan, np.ldexp(1.0, scales - 127))
    return (vals * s[..., None]).reshape(codes.shape)


def attention_mxfp8_logits(q, k_codes, k_scales, v_codes, v_scales, R=None, *, window=0, scale=None,
                           log_scale_base=0.0, chunk=512):
    """Attention whose logits are computed in MXFP8 ([S-FA4]): q is encoded
    with mxfp8_quantize (blocks of 32 along the head dimension), K and V are
    an MXFP8 cache (codes [B, Skv, Hkv, d], scales [B, Skv, Hkv, d/32]); the
    logit of (query, key) is scale * <decoded q, decoded k> (+ bias, log
    scale as in attention), and the output weights the decoded V.  Returns
    o, lse as attention does."""
    qc, qs = mxfp8_quantize(q)
    return attention(mxfp8_dequantize(qc, qs), mxfp8_dequantize(k_codes, k_scales),
                     mxfp8_dequantize(v_codes, v_scales), R, window=window, scale=scale,
                     log_scale_base=log_scale_base, chunk=chunk)


# --------------------------------------------------------------------------- attention prologue ([S-SC])

def short_conv(x, w, history):
    """Causal per-channel convolution of one sequence's new rows.

    x [n, C] new pre-convolution rows; history [W-1, C] the pre-convolution
    rows of the W-1 positions before them, oldest first (rows for positions
    before the sequence start must be zero); w [C, W], tap i multiplies the
    row i positions back.  Returns y [n, C] with
    y[t, c] = sum_i w[c, i] * x_ext[t - i, c]."""
    x, w, history = _f64(x), _f64(w), _f64(history)
    W = w.shape[1]
    ext = np.concatenate([history.reshape(W - 1, x.shape[1]), x], axis=0)   # row W-1+t is x[t]
    n = x.shape[0]
    y = np.zeros_like(x)
    for i in range(W):
        y += w[:, i][None, :] * ext[W - 1 - i:W - 1 - i + n]
    return y


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g along the last axis."""
    x, g = _f64(x), _f64(g)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def attention_prologue(q, k, v, cu_new, seq_lens, wk, wv, gq, gk, eps, state_k, state_v):
    """The attention prologue for T new tokens of B sequences.

    q [T, Hq, d], k/v [T, Hkv, d]: projections of the new tokens, sequence b
    owning rows cu_new[b] .. cu_new[b+1]-1, which sit at positions
    seq_lens[b] - n_b ... seq_lens[b] - 1 (n_b = its new-token count);
    wk/wv [Hkv*d, W] conv taps; gq/gk [d] RMSNorm weights; state_k/state_v
    [B, W-1, Hkv, d] pre-convolution rows of each sequence's last W-1
    positions before this call (oldest first).

    Returns q_out [T, Hq, d] (RMSNorm of q), k_rows [T, Hkv, d] (RMSNorm of
    the convolved k), v_rows [T, Hkv, d] (convolved v), pos [T] (cache
    position of each row), new_state_k, new_state_v."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    state_k, state_v = _f64(state_k), _f64(state_v)
    cu = [int(x) for x in cu_new]
    T, Hkv, d = k.shape
    B = len(cu) - 1
    W = np.asarray(wk).shape[1]
    q_out = rms_norm(q, gq, eps)
    k_rows = np.zeros_like(k)
    v_rows = np.zeros_like(v)
    pos = np.zeros(T, dtype=np.int64)
    nsk, nsv = state_k.copy(), state_v.copy()
    for b in range(B):
        a, e = cu[b], cu[b + 1]
        n = e - a
        L = int(seq_lens[b])
        start = L - n                               # position of the first new token
        hk, hv = state_k[b].copy(), state_v[b].copy()     # [W-1, Hkv, d]
        for j in range(W - 1):                     # history rows before position 0 read zero
            if start - (W - 1) + j < 0:
                hk[j] = 0.0
                hv[j] = 0.0
        yk = short_conv(k[a:e].reshape(n, Hkv * d), wk, hk.reshape(W - 1, Hkv * d)).reshape(n, Hkv, d)
        yv = short_conv(v[a:e].reshape(n, Hkv * d), wv, hv.reshape(W - 1, Hkv * d)).reshape(n, Hkv, d)
        k_rows[a:e] = rms_norm(yk, gk, eps)
        v_rows[a:e] = yv
        pos[a:e] = start + np.arange(n)
        if W > 1:
            ext_k = np.concatenate([state_k[b], k[a:e]], axis=0)   # positions start-(W-1) ... L-1
            ext_v = np.concatenate([state_v[b], v[a:e]], axis=0)
            nsk[b] = ext_k[len(ext_k) - (W - 1):]
            nsv[b] = ext_v[len(ext_v) - (W - 1):]
    return q_out, k_rows, v_rows, pos, nsk, nsv
