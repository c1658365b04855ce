"""Benchmark of the relative-position-bias attention hot path on one MI355X.

A step is one pass of the prefill hot path over the full-causal prefill
workload (B=2, S=32768, Hq=64, Hkv=8, d=128, r_dim=64, E=512, log-scale base
4096, bf16), the largest workload that runs on one GPU: the relative-logit
projection R = r.P followed by the attention prefill, with all inputs resident
in HBM.  `value` is attention TFLOP/s (4*d*Hq flops per visible query/key
pair) over the whole step.  The same JSON line carries:
  * `roofline`: the dominant kernel (attention) of that step, timed with HIP
    events on the stream it runs on;
  * `cpu_baseline`: the fp64 CPU oracle on a bounded row sample of the same
    workload, its rate extrapolated to the whole workload;
  * `workloads`: every other workload (the fp32 parity case, the sliding-window
    prefill, the two decode halves, the long-context decode), each with its own
    `roofline` object and its own oracle timing beside it;
  * the paged, MXFP8, fused-projection and attention-prologue variants, the
    streaming-read bandwidth and MFMA rate the device attains, and the device.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--legs a,b,...]

--legs selects what runs (default: all): c1, c2, c3, c4w, c4f, c5, paged,
mxfp8, prologue, attainable.  The headline step is c3.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3      # dense fp32 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# HBM bytes per launch of each leg's dominant kernel: rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0
# (factors from a plain 1 GiB device copy under the same counters), keyed by leg and by the sha256
# prefix of the kernel source the counters were taken on; any other source reports null.  Entries of
# kernels whose machine code this source leaves unchanged (function bodies compared) carry over: the
# decode, combine and MXFP8 kernels since source ac1e0709a59684d1, the fused prefill variants since
# 781af5c0d78d6ba2, and attn_prefill_pp_kernel<0> (c3, c2) since e25a2cfed1e9566b.
PROFILED_TRAFFIC = {
    ("c3", "df79a6c97489fa01"): 6530915 * 1024 * 2 + 1048577 * 1024,
    ("c2", "df79a6c97489fa01"): 508398 * 1024 * 2 + 131455 * 1024,
    ("c3_fused_on_chip", "df79a6c97489fa01"): 2873850 * 1024 * 2 + 1048740 * 1024,
    ("c2_fused_on_chip", "df79a6c97489fa01"): 145285 * 1024 * 2 + 132533 * 1024,
    ("c3_fused_workspace", "df79a6c97489fa01"): 6296394 * 1024 * 2 + 5248363 * 1024,
    ("c2_fused_workspace", "df79a6c97489fa01"): 529767 * 1024 * 2 + 656038 * 1024,
    ("c4w/head-major", "df79a6c97489fa01"): 578556 * 1024 * 2 + 9216 * 1024,
    ("c4f/head-major", "df79a6c97489fa01"): 1225724 * 1024 * 2 + 9216 * 1024,
    ("c5/head-major", "df79a6c97489fa01"): 524484 * 1024 * 2 + 2064 * 1024,
    ("c4f_paged64/head-major", "df79a6c97489fa01"): 1163403 * 1024 * 2 + 9218 * 1024,
    ("c4f_mxfp8/head-major", "df79a6c97489fa01"): 654406 * 1024 * 2 + 9216 * 1024,
    ("c4f_mxfp8_logits/head-major", "df79a6c97489fa01"): 654449 * 1024 * 2 + 9216 * 1024,
    ("c5_mxfp8/head-major", "df79a6c97489fa01"): 270642 * 1024 * 2 + 2064 * 1024,
    ("c5_mxfp8_logits/head-major", "df79a6c97489fa01"): 270641 * 1024 * 2 + 2064 * 1024,
}


def traffic(leg):
    return PROFILED_TRAFFIC.get((leg, kernel_source_hash()))


def kernel_source_hash():
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "relative_position_bias_rba_amd", "csrc",
                        "attn_kernels.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def time_events(fn, iters, torch):
    """Average duration (ms) of fn() measured with HIP events on the current stream."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / iters


def time_launches(launch, iters, torch, warm_ms=100.0):
    """Average device time (ms) of one launch() when `iters` launches are queued back to back
    on the current stream between two HIP events.  launch() must only enqueue work (C-ABI
    call with prebuilt arguments), so the device never waits for the host between them.
    Launches run untimed for about warm_ms first so the clocks have left their idle state."""
    st = torch.cuda.current_stream()
    t0 = time.perf_counter()
    n = 0
    while n < 3 or (time.perf_counter() - t0) * 1e3 < warm_ms:
        launch()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(iters):
        launch()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def time_cold(launch, iters, torch, flush_bytes=512 << 20):
    """Median device time (ms) of one launch() with the last-level cache flushed before each:
    a read of a flush_bytes buffer (a reduction, so no dirty lines are left to write back during
    the timed launch) is enqueued, then launch() between two HIP events."""
    import statistics
    st = torch.cuda.current_stream()
    junk = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(iters, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        torch.sum(junk, dim=0, out=sink[i])
        a.record(st)
        launch()
        b.record(st)
    torch.cuda.synchronize()
    del junk, sink
    return statistics.median(a.elapsed_time(b) for a, b in evs)


def c_launcher(rba, name, *args):
    """Closure that calls the C entry point `name` with fixed arguments; checks the first call."""
    fn = getattr(rba._lib, name)
    code = fn(*args)
    if code != rba.RBA_OK:
        raise RuntimeError(f"{name} failed: {rba._lib.rba_status_string(code).decode()}")
    return lambda: fn(*args)


def cpu_threads():
    """(threads the oracle's BLAS uses, cores in this process's affinity mask)."""
    aff = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        blas = aff
    return blas, aff


def cpu_baseline(w, inp, budget_s, *, fixed=(), seed=7, batch=8, sample_note=""):
    """The fp64 oracle (test infrastructure, timed as it stands) on query rows of
    workload w (all heads): the `fixed` rows first, then seeded random rows, in
    batches, until budget_s of oracle time is spent.  Prefill reports TFLOP/s of
    visible query/key pairs, decode (Sq <= 32, every row of a sequence at once)
    KV GB/s-equivalent over the sequences it covered; both are extrapolated to
    the whole workload as `extrapolated_s`."""
    import numpy as np

    import oracle
    decode = w.Sq <= 32
    rng = np.random.default_rng(seed)
    if decode:
        seqs = [int(b) for b in rng.permutation(w.B)]
        units = [[(b, t) for t in range(w.Sq)] for b in seqs]
    else:
        rows = [(b, t) for b in range(w.B) for t in fixed if t < w.Sq]
        seen = set(rows)
        for i in rng.permutation(w.B * w.Sq)[:4096]:
            r = (int(i) // w.Sq, int(i) % w.Sq)
            if r not in seen:
                rows.append(r)
                seen.add(r)
        units = [rows[i:i + batch] for i in range(0, len(rows), batch)]

    def R_row(b, t):
        return oracle.relproj(inp["r"][b, t], inp["P"])

    done_rows, work, t_used, n_units = 0, 0.0, 0.0, 0
    for u in units:
        if t_used >= budget_s:
            break
        t0 = time.perf_counter()
        oracle.attention_rows(inp["q"], inp["k"], inp["v"], R_row, u, window=w.window,
                              log_scale_base=w.log_scale_base)
        t_used += time.perf_counter() - t0
        n_units += 1
        done_rows += len(u)
        if decode:
            p_lo, p_hi = w.Skv - w.Sq, w.Skv - 1
            lo = 0 if w.window == 0 else max(0, p_lo - w.window + 1)
            work += (p_hi - lo + 1) * w.Hkv * w.d * 2 * (4 if w.dtype == "fp32" else 2)
        else:
            for _, t in u:
                p = w.Skv - w.Sq + t
                lo = 0 if w.window == 0 else max(0, p - w.window + 1)
                work += 4.0 * w.d * w.Hq * (p - lo + 1)
    blas, aff = cpu_threads()
    if decode:
        value, unit, total = work / t_used / 1e9, "GB/s", w.kv_bytes()
        what = f"{n_units} of {w.B} sequences (all {w.Sq} rows, {w.Hq} heads)"
    else:
        value, unit, total = work / t_used / 1e12, "TFLOP/s", w.attn_flops()
        what = f"{done_rows} of {w.B * w.Sq} query rows x {w.Hq} heads"
    full = n_units == len(units)
    return {"value": round(value, 6), "unit": unit, "cores": int(blas), "affinity_cores": int(aff),
            "blas_threads": int(blas), "kind": "oracle",
            "sample": f"{what} of {w.name} (fp64 NumPy, R rows recomputed from r and P), {t_used:.1f} s"
                      + (f"; {sample_note}" if sample_note else ""),
            "oracle_s": round(t_used, 2),
            ("measured_s" if full else "extrapolated_s"): round(t_used if full else total / (work / t_used), 1)}


def decode_leg(rba, torch, name, reps, mxfp8=False, leg=None, cpu_budget=0.0, qk_fp8=False):
    """One decode workload; mxfp8: its K/V cache encoded to MXFP8 by the library's
    encoder (timed too) and attention run over the encoded cache; qk_fp8: the
    logits in MXFP8 as well (q encoded, QK^T on the scaled FP8 MFMA).  With
    cpu_budget > 0 the oracle is timed on a sample of the same inputs.

    The cache is stored head-major, [B, Hkv, Skv, d] (codes and scales alike),
    and handed over as a [B, Skv, Hkv, d] view with those strides: each key
    tile of one kv head is then one contiguous block.  The bf16 legs also time
    the token-major cache ([B, Skv, Hkv, d] contiguous) with the same values."""
    from workloads import CONFIGS, make_inputs
    w = CONFIGS[name]
    log(f"decode {name}{' mxfp8' if mxfp8 else ''}: generating inputs")
    inp = make_inputs(w)
    d = {k: v.to("cuda") for k, v in inp.items()}
    if cpu_budget <= 0:
        del inp
    R = rba.relproj(d["r"], d["P"])
    splits = rba.num_splits(d["q"], d["k"], d["v"], R, window=w.window)
    o = torch.empty_like(d["q"])
    need = rba.decode_workspace_bytes(d["q"], d["k"], d["v"], R, window=w.window, splits=splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    st = rba._stream(d["q"].device)
    extra = {}
    kv_bytes = w.kv_bytes()
    kh = d["k"].transpose(1, 2).contiguous()          # head-major storage [B, Hkv, Skv, d]
    vh = d["v"].transpose(1, 2).contiguous()
    if not mxfp8:
        a_tm = rba.make_args(d["q"], d["k"], d["v"], R, o, None, window=w.window, log_scale_base=w.log_scale_base)
        launch_tm = c_launcher(rba, "rba_attn_decode", ctypes.byref(a_tm), splits, ctypes.c_void_p(ws.data_ptr()),
                               ws.numel(), st)
        time_launches(launch_tm, 5, torch)
        ms_tm = time_cold(launch_tm, max(reps, 50), torch)
        gbs_tm = kv_bytes / (ms_tm * 1e-3) / 1e9
        extra["token_major"] = {"ms": round(ms_tm, 4), "kv_GBps": round(gbs_tm, 1),
                                "frac_hbm": round(gbs_tm / PEAK_HBM_GBS, 4),
                                "cache": "[B, Skv, Hkv, d] contiguous, same values"}
    if mxfp8:
        x = d["k"].reshape(-1, w.d)
        kc = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        ksc = torch.empty(x.shape[0], w.d // 32, dtype=torch.uint8, device="cuda")
        enc = c_launcher(rba, "rba_mxfp8_quantize", 1, x.shape[0], w.d, ctypes.c_void_p(x.data_ptr()), w.d,
                         ctypes.c_void_p(kc.data_ptr()), w.d, ctypes.c_void_p(ksc.data_ptr()), w.d // 32, st)
        ms_enc = time_launches(enc, reps, torch)
        enc_bytes = x.numel() * 2 + kc.numel() + ksc.numel()
        extra["encode_k"] = {"ms": round(ms_enc, 4), "GBps": round(enc_bytes / (ms_enc * 1e-3) / 1e9, 1),
                             "frac_hbm": round(enc_bytes / (ms_enc * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "bytes": enc_bytes}
        k8, ks = rba.mxfp8_quantize(kh)
        v8, vs = rba.mxfp8_quantize(vh)
        k8, ks, v8, vs = (t.transpose(1, 2) for t in (k8, ks, v8, vs))
        del d["k"], d["v"], x, kc, ksc, kh, vh
        torch.cuda.empty_cache()
        a = rba.make_args(d["q"], k8, v8, R, o, None, window=w.window, log_scale_base=w.log_scale_base,
                          k_scale=ks, v_scale=vs, qk_fp8=qk_fp8)
        kv_bytes = kv_bytes * (w.d + w.d // 32) // (2 * w.d)     # codes + scales per bf16 pair of bytes
        keep = (k8, ks, v8, vs)
    else:
        del d["k"], d["v"]
        torch.cuda.empty_cache()
        a = rba.make_args(d["q"], kh.transpose(1, 2), vh.transpose(1, 2), R, o, None, window=w.window,
                          log_scale_base=w.log_scale_base)
        keep = (kh, vh)
    launch = c_launcher(rba, "rba_attn_decode", ctypes.byref(a), splits, ctypes.c_void_p(ws.data_ptr()),
                        ws.numel(), st)
    ms_warm = time_launches(launch, reps, torch)
    ms = time_cold(launch, max(reps, 50), torch)
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    # the 4-wave variant the library picks for at most 96 query columns (72 and 8 here)
    kname = ("attn_fwd_kernel<bf16, 4 waves, "
             + ("MXFP8 logits, staging wave" if qk_fp8 else ("MXFP8 cache, staging wave" if mxfp8 else "V by DMA")) + ">"
             + (" + combine_kernel" if splits > 1 else ""))
    res = {"ms": round(ms, 4), "kv_GBps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
           "ms_warm": round(ms_warm, 4), "num_splits": splits, "kv_bytes": kv_bytes,
           "cache": "head-major [B, Hkv, Skv, d] storage, passed as a strided [B, Skv, Hkv, d] view",
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic(leg + "/head-major") if leg else None,
                        "kernel": kname, "avg_ms": round(ms, 4), "algorithmic_bytes": kv_bytes},
           "timing": "median of 50 launches, each after a 512 MiB read that evicts the caches; ms_warm: back-to-back mean"}
    if mxfp8:
        res["kv_format"] = "MXFP8 (E4M3 codes + E8M0 scale per 32 head-dim entries)"
        if qk_fp8:
            res["logits"] = "MXFP8: q encoded per 32 head-dim entries, QK^T on v_mfma_scale_f32_32x32x64_f8f6f4"
    res.update(extra)
    del d, R, o, ws, keep
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        log(f"decode {name}: oracle on a sample ...")
        res["cpu_baseline"] = cpu_baseline(w, inp, cpu_budget)
        res["gpu_over_cpu"] = round(gbs / res["cpu_baseline"]["value"], 1)
    return res


def paged_decode_leg(rba, torch, name, page_size, reps, len_lo, seed=77):
    """The decode workload with its cache in page_size-key pages of a shared pool
    and each sequence's length drawn uniformly from [len_lo, Skv].  Each page is
    stored head-major ([Hkv, page_size, d]); the token-major pool is timed too."""
    from workloads import CONFIGS, make_paged_inputs
    w = CONFIGS[name]
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(len_lo, w.Skv + 1, (w.B,), generator=g).tolist()
    log(f"paged decode {name}: generating inputs")
    inp = make_paged_inputs(w, page_size, seq_lens=lens, spare_pages=0)
    d = {k: v.to("cuda") for k, v in inp.items()}
    del inp
    R = rba.relproj(d["r"], d["P"])
    o = torch.empty_like(d["q"])
    kv = rba.make_paged(d["block_table"], d["seq_lens"], page_size, d["k_pool"].shape[0])

    def launcher(kp, vp):
        a = rba.make_args(d["q"], kp, vp, R, o, None, window=w.window, log_scale_base=w.log_scale_base)
        a.Skv = w.Skv
        splits = rba._lib.rba_num_splits(ctypes.byref(a), 0)
        need = rba._lib.rba_decode_workspace_bytes(ctypes.byref(a), splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        return splits, (a, ws), c_launcher(rba, "rba_attn_paged", ctypes.byref(a), ctypes.byref(kv), splits,
                                           ctypes.c_void_p(ws.data_ptr()), ws.numel(), rba._stream(d["q"].device))

    splits, keep_tm, launch_tm = launcher(d["k_pool"], d["v_pool"])
    time_launches(launch_tm, 5, torch)
    ms_tm = time_cold(launch_tm, max(reps, 50), torch)
    kh = d["k_pool"].transpose(1, 2).contiguous().transpose(1, 2)
    vh = d["v_pool"].transpose(1, 2).contiguous().transpose(1, 2)
    del d["k_pool"], d["v_pool"], keep_tm
    splits, keep, launch = launcher(kh, vh)
    ms_warm = time_launches(launch, reps, torch)
    ms = time_cold(launch, max(reps, 50), torch)
    # K and V of the keys the rows see (window 0: every key of the sequence)
    kv_bytes = 0
    for L in lens:
        lo = 0 if w.window == 0 else max(0, L - w.Sq - w.window + 1)
        kv_bytes += (L - lo) * w.Hkv * w.d * 2 * 2
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    res = {"ms": round(ms, 4), "kv_GBps": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic("c4f_paged64/head-major"),
                        "kernel": "attn_fwd_kernel<bf16, 4 waves, paged, V by DMA>" + (" + combine_kernel" if splits > 1
                                                                                      else ""),
                        "avg_ms": round(ms, 4), "algorithmic_bytes": kv_bytes},
           "ms_warm": round(ms_warm, 4), "num_splits": splits, "kv_bytes": kv_bytes, "page_size": page_size,
           "seq_lens": f"uniform in [{len_lo}, {w.Skv}], seed {seed}",
           "cache": "pages stored head-major [Hkv, page_size, d], passed as strided [page_size, Hkv, d] views",
           "token_major": {"ms": round(ms_tm, 4), "kv_GBps": round(kv_bytes / (ms_tm * 1e-3) / 1e9, 1),
                           "frac_hbm": round(kv_bytes / (ms_tm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
           "timing": "median of 50 launches, each after a 512 MiB read that evicts the caches; ms_warm: back-to-back mean"}
    del d, R, o, keep, kh, vh
    torch.cuda.empty_cache()
    return res


def prologue_leg(rba, torch, name, new_tokens, seq_lens, Skv, reps, mxfp8=False, max_new=0):
    """The attention prologue (K/V ShortConv W=4, Q/K RMSNorm, cache write) for a
    batch of new tokens with 64 query / 8 kv heads; HBM-bound.  max_new > 0 passes
    that bound on the new tokens per sequence (one launch); the launch without it
    (new tokens in chunks, a second launch for the conv states) is timed beside."""
    from workloads import make_prologue_inputs
    inp = make_prologue_inputs(new_tokens, seq_lens, Hq=64, Hkv=8, W=4)
    d = {k: v.to("cuda") for k, v in inp.items()}
    B, T = len(new_tokens), int(sum(new_tokens))
    # the decode legs' cache layout: head-major storage behind [B, Skv, Hkv, ...] views
    def cache(n, dt):
        return torch.zeros(B, 8, Skv, n, dtype=dt, device="cuda").transpose(1, 2)

    if mxfp8:
        kc, vc = cache(128, torch.uint8), cache(128, torch.uint8)
        ks, vs = cache(4, torch.uint8), cache(4, torch.uint8)
    else:
        kc, vc = cache(128, torch.bfloat16), cache(128, torch.bfloat16)
        ks = vs = None
    qo = torch.empty_like(d["q"])
    # the call once through the binding (checks), then the C entry point with prebuilt arguments
    rba.attn_prologue(d["q"], d["k"], d["v"], d["cu_new"], d["seq_lens"], d["conv_wk"], d["conv_wv"], d["norm_q"],
                      d["norm_k"], d["state_k"], d["state_v"], kc, vc, k_scale=ks, v_scale=vs, q_out=qo,
                      max_new=max_new)
    a = rba._PrologueArgs()
    a.B, a.T, a.Hq, a.Hkv, a.d, a.conv_w, a.eps = B, T, 64, 8, 128, 4, 1e-6
    a.cu_new, a.seq_lens = d["cu_new"].data_ptr(), d["seq_lens"].data_ptr()
    a.q, a.k, a.v = d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr()
    for nm, t in (("q_s", d["q"]), ("k_s", d["k"]), ("v_s", d["v"]), ("q_out_s", qo)):
        getattr(a, nm)[:] = [t.stride(0), t.stride(1)]
    a.conv_wk, a.conv_wv = d["conv_wk"].data_ptr(), d["conv_wv"].data_ptr()
    a.norm_q, a.norm_k = d["norm_q"].data_ptr(), d["norm_k"].data_ptr()
    a.state_k, a.state_v, a.q_out = d["state_k"].data_ptr(), d["state_v"].data_ptr(), qo.data_ptr()
    c = rba.cache_args(kc, vc, k_scale=ks, v_scale=vs)
    a.max_new = max_new
    launch = c_launcher(rba, "rba_attn_prologue", ctypes.byref(a), ctypes.byref(c), None, rba._stream(qo.device))
    ms = time_launches(launch, reps, torch)
    ms_chunked = None
    if max_new > 0:
        a.max_new = 0
        ms_chunked = time_launches(launch, reps, torch)
        a.max_new = max_new
    row = 128 * 2
    kv_row = 132 if mxfp8 else row
    # q, k, v read once; conv-state rows read and written; q_out and the cache rows written
    nbytes = T * (64 + 16) * row + 2 * B * 3 * 8 * row * 2 + T * 64 * row + T * 16 * kv_row
    res = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "bytes": nbytes, "tokens": T,
           "cache": ("MXFP8" if mxfp8 else "bf16") + ", head-major [B, Hkv, Skv, d] storage",
           "timing": "back-to-back mean after a clock warm-up"}
    if max_new > 0:
        res["max_new"] = max_new
        res["launches"] = "one (K/V rows of a sequence in order per half wave, conv state advanced in place)"
        res["chunked_ms"] = round(ms_chunked, 4)
    del d, kc, vc, ks, vs, qo
    torch.cuda.empty_cache()
    return res


def prefill_leg(rba, torch, name, leg, steps, warmup, cpu_budget, fixed_rows=()):
    """One prefill workload: the step (relproj + attention through the binding)
    timed over `steps` steps after warm-up; the attention kernel and the
    projection alone (C ABI, prebuilt arguments, back to back); the fused
    kernel (projection computed inside the prefill); the oracle on a sample."""
    from workloads import CONFIGS, make_inputs
    w = CONFIGS[name]
    log(f"prefill {name}: generating inputs {w}")
    inp = make_inputs(w)
    d = {k: v.to("cuda") for k, v in inp.items()}
    o = torch.empty_like(d["q"])
    dev = d["q"].device

    def step():
        Rn = rba.relproj(d["r"], d["P"])
        rba.attn_prefill(d["q"], d["k"], d["v"], Rn, window=w.window, log_scale_base=w.log_scale_base, out=o)
        return Rn

    # W warm-up steps, then more untimed steps until ~100 ms have passed so that
    # the clocks have left their idle state before the timed steps
    t_w = time.perf_counter()
    warm_run = 0
    while warm_run < warmup or (time.perf_counter() - t_w) < 0.1:
        R = step()
        warm_run += 1
        if warm_run % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        R = step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps

    reps = max(steps, 10) if w.Sq * w.B <= 16384 else max(steps // 2, 5)
    a_attn = rba.make_args(d["q"], d["k"], d["v"], R, o, None, window=w.window, log_scale_base=w.log_scale_base)
    ms_attn = time_launches(c_launcher(rba, "rba_attn_prefill", ctypes.byref(a_attn), rba._stream(dev)), reps, torch)
    r2 = d["r"].reshape(-1, w.r_dim)
    ms_rp = time_launches(c_launcher(rba, "rba_relproj", 1, 1, r2.shape[0], w.Hq, w.r_dim, w.E,
                                     ctypes.c_void_p(r2.data_ptr()), r2.stride(0), 0,
                                     ctypes.c_void_p(d["P"].data_ptr()), ctypes.c_void_p(R.data_ptr()),
                                     rba._stream(dev)), reps, torch)
    flops = w.attn_flops()
    tf = flops / (ms_attn * 1e-3) / 1e12
    rp_bytes = w.B * w.Sq * w.Hq * w.E * 2 + w.B * w.Sq * w.r_dim * 2 + w.Hq * w.r_dim * w.E * 2
    res = {"workload": w.name, "step_ms": round(ms_step, 4),
           "step_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2), "steps": steps, "warmup_steps_run": warm_run,
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic(leg),
                        "kernel": "attn_prefill_pp_kernel<0>", "avg_ms": round(ms_attn, 4),
                        "algorithmic_flops": flops},
           "relproj": {"ms": round(ms_rp, 4), "GBps": round(rp_bytes / (ms_rp * 1e-3) / 1e9, 1),
                       "frac_hbm": round(rp_bytes / (ms_rp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes": rp_bytes, "flops": w.relproj_flops()},
           "timing": "step: wall clock over the timed steps after torch.cuda.synchronize; kernels: back-to-back "
                     "mean of C-ABI launches between HIP events after a clock warm-up"}
    del R
    res["fused"] = fused_prefill_leg(rba, torch, w, d, reps, ms_attn + ms_rp, leg)
    del d, o, a_attn
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        log(f"prefill {name}: oracle on a row sample ...")
        res["cpu_baseline"] = cpu_baseline(w, inp, cpu_budget, fixed=fixed_rows,
                                           sample_note="fixed rows first, then seeded random rows" if fixed_rows else "")
        res["gpu_over_cpu"] = round(tf / res["cpu_baseline"]["value"], 1)
    return res


def tiny_leg(rba, torch, cpu_budget):
    """The fp32 parity workload (B=1, S=256, Hq=4, Hkv=1, E=64): the GPU result
    against the oracle, the kernels' times and the oracle's time on all of it."""
    import numpy as np

    import oracle
    from workloads import CONFIGS, make_inputs
    w = CONFIGS["c1_tiny_fp32"]
    inp = make_inputs(w)
    d = {k: v.to("cuda") for k, v in inp.items()}
    R = rba.relproj(d["r"], d["P"])
    o, lse = rba.attn_prefill(d["q"], d["k"], d["v"], R, window=w.window, log_scale_base=w.log_scale_base,
                              return_lse=True)
    torch.cuda.synchronize()
    dev = d["q"].device
    a = rba.make_args(d["q"], d["k"], d["v"], R, o, None, window=w.window, log_scale_base=w.log_scale_base)
    ms = time_launches(c_launcher(rba, "rba_attn_prefill", ctypes.byref(a), rba._stream(dev)), 50, torch)
    flops = w.attn_flops()
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": w.name,
           "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_FP32_TFLOPS, 5), "traffic": None,
                        "kernel": "attn_fwd_kernel<float, 4 waves> (fp32 MFMA)", "avg_ms": round(ms, 4),
                        "algorithmic_flops": flops},
           "note": "parity case: 4 workgroups, far too small to fill the chip"}
    if cpu_budget > 0:
        t0 = time.perf_counter()
        wo, wl = oracle.attention(inp["q"], inp["k"], inp["v"], oracle.relproj(inp["r"], inp["P"]), window=w.window,
                                  log_scale_base=w.log_scale_base)
        t = time.perf_counter() - t0
        blas, aff = cpu_threads()
        res["cpu_baseline"] = {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas),
                               "affinity_cores": int(aff), "blas_threads": int(blas), "kind": "oracle",
                               "sample": f"the whole workload (fp64 NumPy), {t:.2f} s", "oracle_s": round(t, 3),
                               "measured_s": round(t, 3)}
        res["parity_max_abs"] = {"o": float(np.abs(o.double().cpu().numpy() - wo).max()),
                                 "lse": float(np.abs(lse.double().cpu().numpy() - wl).max()), "bound": 1e-5}
    del d, R, o, lse
    torch.cuda.empty_cache()
    return res


def fused_prefill_leg(rba, torch, w, d, reps, two_kernel_ms, leg):
    """rba_attn_prefill_fused on the same workload: relproj and attention in one
    launch, the rows of R kept in a per-workgroup workspace instead of HBM, and
    without a workspace (each banded key tile's logits computed into LDS)."""
    dev = d["q"].device
    PT = rba.relproj_pack(d["P"])
    o = torch.empty_like(d["q"])
    a = rba.make_args(d["q"], d["k"], d["v"], None, o, None, window=w.window, log_scale_base=w.log_scale_base)
    a.E = w.E
    rb = rba.make_relbias(d["r"], PT)
    need = rba._lib.rba_prefill_fused_workspace_bytes(ctypes.byref(a))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ms = time_launches(c_launcher(rba, "rba_attn_prefill_fused", ctypes.byref(a), ctypes.byref(rb),
                                  ctypes.c_void_p(ws.data_ptr()), need, rba._stream(dev)), reps, torch)
    # no workspace: each banded key tile's logits computed into LDS, no R in memory
    ms_oc = time_launches(c_launcher(rba, "rba_attn_prefill_fused", ctypes.byref(a), ctypes.byref(rb), None, 0,
                                     rba._stream(dev)), reps, torch)
    flops = w.attn_flops()
    res = {"ms": round(ms, 4), "step_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "two_kernel_ms": round(two_kernel_ms, 4), "speedup_vs_two_kernels": round(two_kernel_ms / ms, 4),
           "workspace_bytes": need, "kernel": "attn_prefill_pp_kernel<4> (rows of R per block in the workspace)",
           "traffic": traffic(leg + "_fused_workspace"),
           "on_chip": {"ms": round(ms_oc, 4), "step_tflops": round(flops / (ms_oc * 1e-3) / 1e12, 1),
                       "speedup_vs_two_kernels": round(two_kernel_ms / ms_oc, 4), "workspace_bytes": 0,
                       "traffic": traffic(leg + "_fused_on_chip"),
                       "kernel": "attn_prefill_pp_kernel<4, on-chip> (banded tiles' logits computed into LDS)"},
           "timing": "back-to-back mean after a clock warm-up"}
    del ws, o, PT
    return res


def attainable(rba, torch):
    """Streaming-read bandwidth and bf16 MFMA rate this device attains (the library's
    measurement aids, timed like the kernels)."""
    dev = torch.device("cuda")
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    st = rba._stream(dev)
    rd = c_launcher(rba, "rba_calib_read", ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), st)
    ms_rd = time_launches(rd, 10, torch)
    flops = ctypes.c_double(0.0)
    iters = 250
    mm = c_launcher(rba, "rba_calib_mfma", iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops), st)
    ms_mm = time_launches(mm, 5, torch)
    del buf, sink
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(nbytes / (ms_rd * 1e-3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops.value / (ms_mm * 1e-3) / 1e12, 1),
            "how": "rba_calib_read over 2 GiB (16-byte loads, 2 workgroups per CU) and rba_calib_mfma "
                   "(back-to-back bf16 32x32x16 MFMA, 32 waves per CU), HIP events, after a clock warm-up"}


ALL_LEGS = ("c1", "c2", "c3", "c4w", "c4f", "c5", "paged", "mxfp8", "prologue", "attainable")
C3_FIXED_ROWS = (0, 1, 511, 512, 4095, 4096, 32767)     # extent and log-scale edges, the last row
C2_FIXED_ROWS = (0, 1, 511, 512, 4095, 4096, 8191)      # extent and window edges, the last row


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default=",".join(ALL_LEGS),
                    help="comma-separated subset of " + ",".join(ALL_LEGS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time per timed workload (the headline's and each other's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              f"(every box has one GPU and the path needs no collective).", file=sys.stderr)
        sys.exit(2)
    legs = [x for x in args.legs.split(",") if x]
    bad = [x for x in legs if x not in ALL_LEGS]
    if bad:
        print(f"unknown legs {bad}; choose from {ALL_LEGS}", file=sys.stderr)
        sys.exit(2)
    budget = 0.0 if args.no_cpu_baseline else args.cpu_budget

    import torch

    import relative_position_bias_rba_amd as rba
    from workloads import CONFIGS

    out = {"metric": "rel-bias attn prefill TFLOP/s & decode KV GB/s (% of MI355X roofline)"}
    work = {}
    if "c3" in legs:
        head = prefill_leg(rba, torch, "c3_full_prefill", "c3", args.steps, args.warmup, budget, C3_FIXED_ROWS)
        w = CONFIGS["c3_full_prefill"]
        value = w.attn_flops() / (head["step_ms"] * 1e-3) / 1e12
        out.update({
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "warmup_steps_run": head["warmup_steps_run"], "ms_per_step": head["step_ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded normals)",
            "config": {"workload": "full-causal prefill B=2 S=32768 Hq=64 Hkv=8 d=128 r_dim=64 E=512, log-scale "
                                   "base 4096 (relproj + attention per step)",
                       "global_batch": w.B, "seq_len": w.Sq, "parallelism": "single GPU"},
            "roofline": head["roofline"],
            "cpu_baseline": head.get("cpu_baseline"),
        })
        work["c3_full_prefill"] = head
    if "c2" in legs:
        work["c2_swa_prefill"] = prefill_leg(rba, torch, "c2_swa_prefill", "c2", args.steps, args.warmup, budget,
                                             C2_FIXED_ROWS)
    if "c1" in legs:
        work["c1_tiny_fp32"] = tiny_leg(rba, torch, budget)
    for leg, name in (("c4w", "c4_decode_swa"), ("c4f", "c4_decode_full"), ("c5", "c5_long_decode")):
        if leg in legs:
            work[name] = decode_leg(rba, torch, name, 20, leg=leg, cpu_budget=budget)
    out["workloads"] = work
    extra = {}
    if "paged" in legs:
        extra["c4_decode_full_paged64"] = paged_decode_leg(rba, torch, "c4_decode_full", 64, 20, 8192)
        extra["c4_decode_full_paged64"]["cpu_baseline_ref"] = "workloads.c4_decode_full (same oracle and shapes)"
    if "mxfp8" in legs:
        for name, leg in (("c4_decode_full", "c4f"), ("c5_long_decode", "c5")):
            extra[name + "_mxfp8"] = decode_leg(rba, torch, name, 20, mxfp8=True, leg=leg + "_mxfp8")
            extra[name + "_mxfp8"]["cpu_baseline_ref"] = f"workloads.{name} (the oracle runs on the decoded cache)"
            extra[name + "_mxfp8_logits"] = decode_leg(rba, torch, name, 20, mxfp8=True, qk_fp8=True,
                                                       leg=leg + "_mxfp8_logits")
            extra[name + "_mxfp8_logits"]["cpu_baseline_ref"] = (f"workloads.{name} (the oracle runs on the "
                                                                 "decoded cache and the encoded q)")
    if extra:
        out["decode_variants"] = extra
    if "prologue" in legs:
        log("attention prologue ...")
        out["prologue"] = {
            "prefill_8192": prologue_leg(rba, torch, "prefill", [8192], [8192], 8192, 20),
            "decode_64x9": prologue_leg(rba, torch, "decode", [9] * 64, [9216] * 64, 9216, 50, max_new=9),
            "decode_64x9_mxfp8": prologue_leg(rba, torch, "decode", [9] * 64, [9216] * 64, 9216, 50, mxfp8=True,
                                              max_new=9),
        }
    if "attainable" in legs:
        att = attainable(rba, torch)
        out["attainable"] = att
        for wl in work.values():
            rf = wl.get("roofline")
            if rf and rf["unit"] == "TFLOP/s" and rf["peak"] == PEAK_BF16_TFLOPS:
                rf["frac_attainable"] = round(rf["achieved"] / att["mfma_bf16_TFLOPs"], 4)
            elif rf and rf["unit"] == "GB/s":
                rf["frac_attainable"] = round(rf["achieved"] / att["hbm_read_GBps"], 4)
    out["device"] = {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                     "compute_units": torch.cuda.get_device_properties(0).multi_processor_count}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
