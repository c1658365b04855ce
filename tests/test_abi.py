"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments with the documented status before touching the GPU.
No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest
import torch

import relative_position_bias_rba_amd as rba
from relative_position_bias_rba_amd import (RBA_E_INVALID, RBA_E_UNSUPPORTED, RBA_E_WORKSPACE, RBA_OK,
                                            make_args)

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "rba.h")
lib = rba._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rba_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("rba_relproj", "rba_attn_prefill", "rba_attn_decode", "rba_attn_paged", "rba_splitkv_combine",
                 "rba_mxfp8_quantize", "rba_attn_prologue",
                 "rba_num_splits", "rba_decode_workspace_bytes", "rba_status_string"):
        assert must in names


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(rba.lib_path)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings_and_version():
    for code in range(5):
        assert lib.rba_status_string(code)
    assert lib.rba_status_string(RBA_OK) == b"ok"
    assert lib.rba_version() >= 100


def _tensors(B=1, Sq=9, Skv=64, Hq=8, Hkv=2, d=128, E=16, dtype=torch.bfloat16):
    q = torch.zeros(B, Sq, Hq, d, dtype=dtype)
    k = torch.zeros(B, Skv, Hkv, d, dtype=dtype)
    v = torch.zeros(B, Skv, Hkv, d, dtype=dtype)
    R = torch.zeros(B, Sq, Hq, E, dtype=dtype)
    o = torch.zeros_like(q)
    return q, k, v, R, o


def _prefill(a):
    return lib.rba_attn_prefill(ctypes.byref(a), None)


def _decode(a, splits=4, ws=None, nbytes=0):
    return lib.rba_attn_decode(ctypes.byref(a), splits, ws, nbytes, None)


def test_validation_rejects_bad_shapes():
    q, k, v, R, o = _tensors()
    cases = []
    a = make_args(q, k, v, R, o); a.d = 64; cases.append((a, RBA_E_UNSUPPORTED))
    a = make_args(q, k, v, R, o); a.d = 0; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.Hkv = 3; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.Sq = 100; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.window = -1; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.E = 0; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.log_scale_base = 0.5; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.scale = float("nan"); cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.scale = 0.0; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.scale = -0.1; cases.append((a, RBA_E_INVALID))
    a = make_args(q, k, v, R, o); a.dt = 7; cases.append((a, RBA_E_UNSUPPORTED))
    a = make_args(q, k, v, R, o); a.Hq = 512; a.Hkv = 1; cases.append((a, RBA_E_UNSUPPORTED))
    a = make_args(q, k, v, R, o); a.B = -1; cases.append((a, RBA_E_INVALID))
    for a, want in cases:
        assert _prefill(a) == want
        assert _decode(a) == want
        assert lib.rba_num_splits(ctypes.byref(a), 256) == 0


def test_validation_rejects_bad_pointers_and_strides():
    q, k, v, R, o = _tensors()
    a = make_args(q, k, v, R, o); a.q = None
    assert _prefill(a) == RBA_E_INVALID
    a = make_args(q, k, v, R, o); a.o = None
    assert _prefill(a) == RBA_E_INVALID
    a = make_args(q, k, v, R, o); a.k = k.data_ptr() + 2
    assert _prefill(a) == RBA_E_INVALID
    a = make_args(q, k, v, R, o); a.q_s[1] = 1028      # not a 16-byte multiple for bf16
    assert _prefill(a) == RBA_E_INVALID
    a = make_args(q, k, v, R, o); a.v_s[0] = -8
    assert _prefill(a) == RBA_E_INVALID
    a = make_args(q, k, v, R, o); a.R = R.data_ptr() + 1
    assert _prefill(a) == RBA_E_INVALID
    a = make_args(q, k, v, R, o); a.lse = o.data_ptr() + 2
    assert _prefill(a) == RBA_E_INVALID
    with pytest.raises(ValueError):
        make_args(q.transpose(2, 3), k, v, R, o)


def test_empty_inputs_are_noops():
    q, k, v, R, o = _tensors(Sq=0)
    a = make_args(q, k, v, R, o); a.q = None; a.o = None
    assert _prefill(a) == RBA_OK
    assert _decode(a, splits=3) == RBA_OK
    q, k, v, R, o = _tensors(B=0)
    a = make_args(q, k, v, R, o)
    assert _prefill(a) == RBA_OK
    r = torch.zeros(0, 64)
    P = torch.zeros(4, 64, 16)
    assert lib.rba_relproj(0, 0, 0, 4, 64, 16, None, 64, 0, None, None, None) == RBA_OK


def test_decode_workspace_checks():
    q, k, v, R, o = _tensors(B=2, Sq=9, Skv=640, Hq=16, Hkv=2)
    a = make_args(q, k, v, R, o)
    need = lib.rba_decode_workspace_bytes(ctypes.byref(a), 4)
    assert need == 4 * 2 * 9 * 16 * (128 + 1) * 4
    assert lib.rba_decode_workspace_bytes(ctypes.byref(a), 1) == 0
    assert _decode(a, splits=4, ws=None, nbytes=0) == RBA_E_WORKSPACE
    buf = torch.zeros(need // 4, dtype=torch.float32)
    assert _decode(a, splits=4, ws=ctypes.c_void_p(buf.data_ptr()), nbytes=need - 4) == RBA_E_WORKSPACE
    assert _decode(a, splits=4, ws=ctypes.c_void_p(buf.data_ptr() + 4), nbytes=need) == RBA_E_WORKSPACE
    assert _decode(a, splits=-1) == RBA_E_INVALID
    assert _decode(a, splits=5000) == RBA_E_INVALID
    assert lib.rba_splitkv_combine(None, None, 4, ctypes.byref(a), None) == RBA_E_INVALID
    assert lib.rba_splitkv_combine(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(buf.data_ptr()), 0,
                                   ctypes.byref(a), None) == RBA_E_INVALID


def test_decode_noalloc_host_checks():
    """rba_attn_decode_noalloc rejects, before any launch, split partials
    larger than its scratch array, and bad arguments as rba_attn_decode does."""
    q, k, v, R, o = _tensors(B=64, Sq=9, Skv=640, Hq=64, Hkv=8)
    a = make_args(q, k, v, R, o)
    need = lib.rba_decode_workspace_bytes(ctypes.byref(a), 2)
    assert need > rba.RBA_DECODE_SCRATCH_BYTES
    assert lib.rba_attn_decode_noalloc(ctypes.byref(a), 2, None) == RBA_E_WORKSPACE
    assert lib.rba_attn_decode_noalloc(ctypes.byref(a), -1, None) == RBA_E_INVALID
    assert lib.rba_attn_decode_noalloc(ctypes.byref(a), 5000, None) == RBA_E_INVALID
    a.Hq = 7                      # not a multiple of Hkv
    assert lib.rba_attn_decode_noalloc(ctypes.byref(a), 2, None) == RBA_E_INVALID
    assert lib.rba_attn_decode_noalloc(None, 2, None) == RBA_E_INVALID


def _paged(B=2, Sq=3, ps=64, n_pages=10, Hq=8, Hkv=2, E=16, n_max=4):
    q = torch.zeros(B, Sq, Hq, 128, dtype=torch.bfloat16)
    kp = torch.zeros(n_pages, ps, Hkv, 128, dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    R = torch.zeros(B, Sq, Hq, E, dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    table = torch.zeros(B, n_max, dtype=torch.int32)
    lens = torch.full((B,), ps * n_max, dtype=torch.int32)
    a = make_args(q, kp, vp, R, o)
    a.Skv = ps * n_max
    kv = rba.make_paged(table, lens, ps, n_pages)
    return a, kv, (q, kp, vp, R, o, table, lens)


def _paged_call(a, kv, splits=1, ws=None, nbytes=0):
    return lib.rba_attn_paged(ctypes.byref(a), None if kv is None else ctypes.byref(kv), splits, ws, nbytes, None)


def test_paged_validation():
    a, kv, keep = _paged()
    assert _paged_call(a, None) == RBA_E_INVALID
    for field, val in (("page_size", 0), ("page_size", 32), ("page_size", 96), ("num_pages", 0),
                       ("bt_stride", 3), ("block_table", None), ("seq_lens", None)):
        a, kv, keep = _paged()
        setattr(kv, field, val)
        assert _paged_call(a, kv) == RBA_E_INVALID, field
    a, kv, keep = _paged()
    kv.seq_lens = keep[6].data_ptr() + 2
    assert _paged_call(a, kv) == RBA_E_INVALID
    a, kv, keep = _paged()
    a.Skv = 4 * 64 + 1               # needs a fifth table column
    assert _paged_call(a, kv) == RBA_E_INVALID
    a, kv, keep = _paged()
    assert _paged_call(a, kv, splits=-1) == RBA_E_INVALID
    assert _paged_call(a, kv, splits=4) == RBA_E_WORKSPACE
    a, kv, keep = _paged()
    a.d = 64
    assert _paged_call(a, kv) == RBA_E_UNSUPPORTED
    # a page whose K rows span 2^31 bytes cannot be addressed
    a, kv, keep = _paged()
    a.k_s[1] = 1 << 25
    assert _paged_call(a, kv) == RBA_E_UNSUPPORTED


def test_paged_empty_is_noop():
    a, kv, keep = _paged(Sq=0)
    kv.block_table = None
    kv.seq_lens = None
    assert _paged_call(a, kv, splits=3) == RBA_OK


def test_mxfp8_kv_validation():
    q, k, v, R, o = _tensors()
    kc = torch.zeros(k.shape, dtype=torch.uint8)
    ks = torch.zeros(*k.shape[:3], 4, dtype=torch.uint8)
    a = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks)
    assert a.kv_format == rba.RBA_KV_MXFP8
    a2 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks); a2.kv_format = 3
    assert _prefill(a2) == RBA_E_INVALID
    # the MXFP8-logits format takes the same cache and the same checks
    a3 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks, qk_fp8=True)
    assert a3.kv_format == rba.RBA_KV_MXFP8_QK == 2
    a3.dt = 0
    assert _prefill(a3) == RBA_E_UNSUPPORTED and _decode(a3) == RBA_E_UNSUPPORTED
    a3 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks, qk_fp8=True); a3.v_scale = None
    assert _prefill(a3) == RBA_E_INVALID and _decode(a3) == RBA_E_INVALID
    a3 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks, qk_fp8=True); a3.k_s[1] = 136
    assert _decode(a3) == RBA_E_INVALID
    with pytest.raises(ValueError):
        make_args(q, k, v, R, o, qk_fp8=True)
    a2 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks); a2.dt = 0
    assert _prefill(a2) == RBA_E_UNSUPPORTED and _decode(a2) == RBA_E_UNSUPPORTED
    a2 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks); a2.k_scale = None
    assert _prefill(a2) == RBA_E_INVALID
    a2 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks); a2.k_s[1] = 136   # bytes, not a 16-multiple
    assert _prefill(a2) == RBA_E_INVALID
    a2 = make_args(q, kc, kc, R, o, k_scale=ks, v_scale=ks); a2.v_scale_s[0] = -4
    assert _decode(a2) == RBA_E_INVALID
    with pytest.raises(ValueError):
        make_args(q, kc, kc, R, o, k_scale=ks)


def test_mxfp8_quantize_validation():
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    c = torch.zeros(4, 128, dtype=torch.uint8)
    sc = torch.zeros(4, 4, dtype=torch.uint8)
    px, pc, ps = (ctypes.c_void_p(t.data_ptr()) for t in (x, c, sc))
    f = lib.rba_mxfp8_quantize
    assert f(1, 0, 128, None, 128, None, 128, None, 4, None) == RBA_OK
    assert f(1, 4, 48, px, 128, pc, 128, ps, 4, None) == RBA_E_INVALID          # n not a multiple of 32
    assert f(1, 4, 0, px, 128, pc, 128, ps, 4, None) == RBA_E_INVALID
    assert f(1, -1, 128, px, 128, pc, 128, ps, 4, None) == RBA_E_INVALID
    assert f(1, 4, 128, px, 100, pc, 128, ps, 4, None) == RBA_E_INVALID         # x rows overlap
    assert f(1, 4, 128, px, 132, pc, 128, ps, 4, None) == RBA_E_INVALID         # x rows not 16-byte aligned
    assert f(1, 4, 128, ctypes.c_void_p(x.data_ptr() + 8), 128, pc, 128, ps, 4, None) == RBA_E_INVALID
    assert f(1, 4, 128, px, 128, pc, 126, ps, 4, None) == RBA_E_INVALID
    assert f(1, 4, 128, px, 128, ctypes.c_void_p(c.data_ptr() + 2), 128, ps, 4, None) == RBA_E_INVALID
    assert f(1, 4, 128, px, 128, pc, 128, ps, 3, None) == RBA_E_INVALID
    assert f(1, 4, 128, px, 128, pc, 128, None, 4, None) == RBA_E_INVALID
    assert f(5, 4, 128, px, 128, pc, 128, ps, 4, None) == RBA_E_UNSUPPORTED


def _prologue_abi(T=3, B=2, Hq=4, Hkv=2, W=4, f8=False):
    q = torch.zeros(T, Hq, 128, dtype=torch.bfloat16)
    k = torch.zeros(T, Hkv, 128, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    cu = torch.tensor([0, 1, T], dtype=torch.int32)
    lens = torch.tensor([5, 9], dtype=torch.int32)
    wk = torch.zeros(Hkv * 128, W)
    nq = torch.ones(128)
    st = torch.zeros(B, W - 1, Hkv, 128, dtype=torch.bfloat16)
    qo = torch.zeros_like(q)
    kc = torch.zeros(B, 16, Hkv, 128, dtype=torch.uint8 if f8 else torch.bfloat16)
    sc = torch.zeros(B, 16, Hkv, 4, dtype=torch.uint8) if f8 else None
    keep = (q, k, v, cu, lens, wk, nq, st, qo, kc, sc)
    a = rba._PrologueArgs()
    a.B, a.T, a.Hq, a.Hkv, a.d, a.conv_w, a.eps = B, T, Hq, Hkv, 128, W, 1e-6
    a.cu_new, a.seq_lens, a.q, a.k, a.v = cu.data_ptr(), lens.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.q_s[:] = [q.stride(0), q.stride(1)]
    a.k_s[:] = [k.stride(0), k.stride(1)]
    a.v_s[:] = [v.stride(0), v.stride(1)]
    a.conv_wk = a.conv_wv = wk.data_ptr()
    a.norm_q = a.norm_k = nq.data_ptr()
    a.state_k = a.state_v = st.data_ptr()
    a.q_out = qo.data_ptr()
    a.q_out_s[:] = [qo.stride(0), qo.stride(1)]
    c = rba.cache_args(kc, kc, k_scale=sc, v_scale=sc)
    return a, c, keep


def _prologue_call(a, c, kv=None):
    return lib.rba_attn_prologue(ctypes.byref(a), None if c is None else ctypes.byref(c),
                                 None if kv is None else ctypes.byref(kv), None)


def test_prologue_validation():
    cases = [
        (lambda a, c: setattr(a, "d", 64), RBA_E_UNSUPPORTED),
        (lambda a, c: setattr(a, "d", 0), RBA_E_INVALID),
        (lambda a, c: setattr(a, "conv_w", 0), RBA_E_INVALID),
        (lambda a, c: setattr(a, "conv_w", 9), RBA_E_INVALID),
        (lambda a, c: setattr(a, "eps", 0.0), RBA_E_INVALID),
        (lambda a, c: setattr(a, "eps", float("inf")), RBA_E_INVALID),
        (lambda a, c: setattr(a, "max_new", -1), RBA_E_INVALID),
        (lambda a, c: setattr(a, "Hkv", 3), RBA_E_INVALID),
        (lambda a, c: setattr(a, "B", 0), RBA_E_INVALID),
        (lambda a, c: setattr(a, "cu_new", None), RBA_E_INVALID),
        (lambda a, c: setattr(a, "state_k", None), RBA_E_INVALID),
        (lambda a, c: setattr(a, "q", a.q + 2), RBA_E_INVALID),
        (lambda a, c: a.k_s.__setitem__(0, 258), RBA_E_INVALID),
        (lambda a, c: setattr(c, "dt", 0), RBA_E_UNSUPPORTED),
        (lambda a, c: setattr(c, "kv_format", 3), RBA_E_INVALID),
        (lambda a, c: setattr(c, "Skv", 0), RBA_E_INVALID),
        (lambda a, c: c.v_s.__setitem__(1, 6), RBA_E_INVALID),
    ]
    for mutate, want in cases:
        a, c, keep = _prologue_abi()
        mutate(a, c)
        assert _prologue_call(a, c) == want
    a, c, keep = _prologue_abi()
    assert _prologue_call(a, None) == RBA_E_INVALID
    a, c, keep = _prologue_abi(f8=True)
    c.k_scale = None
    assert _prologue_call(a, c) == RBA_E_INVALID
    # paged destination: page size and table checked like the attention's
    a, c, keep = _prologue_abi()
    table = torch.zeros(2, 1, dtype=torch.int32)
    kv = rba.make_paged(table, keep[4], 32, 4)
    assert _prologue_call(a, c, kv) == RBA_E_INVALID
    kv = rba.make_paged(table, keep[4], 64, 4)
    c.Skv = 65                                  # two pages needed, one table column
    assert _prologue_call(a, c, kv) == RBA_E_INVALID
    # nothing to do
    a, c, keep = _prologue_abi()
    a.T = 0
    a.q = a.k = a.v = a.q_out = None
    assert _prologue_call(a, c) == RBA_OK


def test_calib_validation():
    buf = torch.zeros(16384, dtype=torch.uint8)
    sink = torch.zeros(4, dtype=torch.float32)
    pb, ps = ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(sink.data_ptr())
    assert lib.rba_calib_read(pb, 0, ps, None) == RBA_OK
    assert lib.rba_calib_read(pb, 1000, ps, None) == RBA_E_INVALID
    assert lib.rba_calib_read(None, 16384, ps, None) == RBA_E_INVALID
    assert lib.rba_calib_read(pb, 16384, None, None) == RBA_E_INVALID
    assert lib.rba_calib_read(ctypes.c_void_p(buf.data_ptr() + 4), 16384, ps, None) == RBA_E_INVALID
    assert lib.rba_calib_mfma(0, ps, None, None) == RBA_E_INVALID
    assert lib.rba_calib_mfma(10, None, None, None) == RBA_E_INVALID


def test_relproj_validation():
    r = torch.zeros(8, 64, dtype=torch.bfloat16)
    P = torch.zeros(4, 64, 16, dtype=torch.bfloat16)
    R = torch.zeros(8, 4, 16, dtype=torch.bfloat16)
    pr, pP, pR = (ctypes.c_void_p(t.data_ptr()) for t in (r, P, R))
    assert lib.rba_relproj(1, 1, 8, 4, 200, 16, pr, 200, 0, pP, pR, None) == RBA_E_UNSUPPORTED
    assert lib.rba_relproj(1, 1, 8, 4, 0, 16, pr, 64, 0, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, 8, 4, 64, 0, pr, 64, 0, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, -1, 4, 64, 16, pr, 64, 0, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, 8, 4, 64, 16, None, 64, 0, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, 8, 4, 64, 16, pr, 32, 0, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, 8, 4, 64, 16, ctypes.c_void_p(r.data_ptr() + 2), 64, 0, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(3, 1, 8, 4, 64, 16, pr, 64, 0, pP, pR, None) == RBA_E_UNSUPPORTED
    # per-head r: head stride below r_dim, or token stride below Hq head strides
    assert lib.rba_relproj(1, 1, 8, 4, 64, 16, pr, 256, 32, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, 8, 4, 64, 16, pr, 200, 64, pP, pR, None) == RBA_E_INVALID
    assert lib.rba_relproj(1, 1, 8, 4, 64, 16, pr, 256, -64, pP, pR, None) == RBA_E_INVALID


def test_relproj_pack_validation():
    assert lib.rba_relproj_packed_bytes(4, 64, 16) == 4 * 32 * 64 * 2      # E padded to whole 32-tiles
    assert lib.rba_relproj_packed_bytes(4, 64, 33) == 4 * 64 * 64 * 2
    assert lib.rba_relproj_packed_bytes(4, 40, 16) == 0                   # r_dim not a multiple of 16
    assert lib.rba_relproj_packed_bytes(4, 144, 16) == 0
    assert lib.rba_relproj_packed_bytes(0, 64, 16) == 0
    P = torch.zeros(4, 64, 16, dtype=torch.bfloat16)
    PT = torch.zeros(4, 32, 64, dtype=torch.bfloat16)
    pP, pT = ctypes.c_void_p(P.data_ptr()), ctypes.c_void_p(PT.data_ptr())
    assert lib.rba_relproj_pack(4, 40, 16, pP, pT, None) == RBA_E_UNSUPPORTED
    assert lib.rba_relproj_pack(0, 64, 16, pP, pT, None) == RBA_E_INVALID
    assert lib.rba_relproj_pack(4, 0, 16, pP, pT, None) == RBA_E_INVALID
    assert lib.rba_relproj_pack(4, 64, 0, pP, pT, None) == RBA_E_INVALID
    assert lib.rba_relproj_pack(4, 64, 16, None, pT, None) == RBA_E_INVALID
    assert lib.rba_relproj_pack(4, 64, 16, pP, ctypes.c_void_p(PT.data_ptr() + 2), None) == RBA_E_INVALID


def _fused_args(Sq=64, Hq=16, Hkv=2, E=64, dtype=torch.bfloat16):
    q, k, v, _, o = _tensors(B=1, Sq=Sq, Skv=Sq, Hq=Hq, Hkv=Hkv, E=E, dtype=dtype)
    a = make_args(q, k, v, None, o, None)
    a.E = E
    r = torch.zeros(1, Sq, 64, dtype=dtype)
    PT = rba.PackedProjection(torch.zeros(Hq * E * 64, dtype=dtype), Hq, 64, E)
    rb = rba.make_relbias(r, PT)
    return a, rb, (q, k, v, o, r, PT.data)


def _fused(a, rb, ws=None, nbytes=0):
    return lib.rba_attn_prefill_fused(ctypes.byref(a), None if rb is None else ctypes.byref(rb), ws, nbytes, None)


def test_prefill_fused_validation():
    """Rejections that the host decides before it asks the device anything."""
    a, rb, keep = _fused_args()
    assert _fused(a, None) == RBA_E_INVALID
    R = torch.zeros(1, 64, 16, 64, dtype=torch.bfloat16)
    a.R = R.data_ptr()                                   # the bias comes from r, not from R
    a.R_s[:] = [R.stride(0), R.stride(1), R.stride(2)]
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args()
    a.E = 0
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args()
    rb.r_dim = 40
    assert _fused(a, rb) == RBA_E_UNSUPPORTED               # r_dim must be a multiple of 16
    rb.r_dim = 144
    assert _fused(a, rb) == RBA_E_UNSUPPORTED
    rb.r_dim = 0
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args(Hq=8, Hkv=2)                  # 4 heads x 32 rows: the 4-wave kernel
    assert _fused(a, rb) == RBA_E_UNSUPPORTED
    a, rb, keep = _fused_args(dtype=torch.float32)
    assert _fused(a, rb) == RBA_E_UNSUPPORTED
    a, rb, keep = _fused_args()
    rb.r = None
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args()
    rb.PT = keep[5].data_ptr() + 2
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args()
    rb.r_s[1] = 60                                       # token stride not a multiple of 8
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args()
    rb.r_s[2] = 32                                       # per-head stride below r_dim
    assert _fused(a, rb) == RBA_E_INVALID
    a, rb, keep = _fused_args()
    a.Sq = a.B = 0
    assert _fused(a, rb) == RBA_OK                          # nothing to do
    a, rb, keep = _fused_args()
    a.Hkv = 5                                            # Hq not a multiple of Hkv
    assert _fused(a, rb) == RBA_E_INVALID


# --------------------------------------------------------------------------- split heuristic (host logic)

def _split_args(B, Sq, Skv, Hq=64, Hkv=8, window=0):
    q = torch.zeros(1, 1, 1, 1)
    a = rba._AttnArgs()
    a.dt, a.B, a.Sq, a.Skv, a.Hq, a.Hkv, a.d, a.E = 1, B, Sq, Skv, Hq, Hkv, 128, 512
    a.window, a.scale, a.log_scale_base = window, 0.088, 0.0
    fake = 1 << 20
    a.q = a.k = a.v = a.o = a.R = fake
    for name in ("q_s", "k_s", "v_s", "o_s", "R_s"):
        getattr(a, name)[:] = [8, 8, 8]
    return a


@pytest.mark.parametrize("B,Sq,Skv,window", [(64, 9, 9216, 0), (64, 9, 9216, 4096), (1, 1, 262144, 0),
                                              (1, 9, 300, 0), (4, 1, 64, 0), (1, 32, 100000, 4096)])
def test_num_splits_heuristic_properties(B, Sq, Skv, window):
    a = _split_args(B, Sq, Skv, window=window)
    s = lib.rba_num_splits(ctypes.byref(a), 256)
    assert 1 <= s <= 1024
    # never more splits than 4-tile chunks of the visible key range of a block
    lo = 0 if window == 0 else max(0, Skv - Sq - window + 1)
    tiles = (Skv - 1) // 64 - lo // 64 + 1
    assert s <= max(1, tiles // 4)
    # more compute units never means fewer splits
    assert lib.rba_num_splits(ctypes.byref(a), 512) >= s


def test_num_splits_reference_points():
    # 64 sequences x 8 kv heads already give two work items per CU: no split
    assert lib.rba_num_splits(ctypes.byref(_split_args(64, 9, 9216)), 256) == 1
    # one sequence, 8 kv heads, 256K keys: spread over the whole chip
    assert lib.rba_num_splits(ctypes.byref(_split_args(1, 1, 262144)), 256) == 64
