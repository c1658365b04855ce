"""Python binding of librba: relative-position-bias attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the gfx950
kernels of ``librba.so`` (built in-tree by ``relative_position_bias_rba_amd.build``);
torch provides device memory and the current HIP stream.  Importing this
package fails loudly if the library has not been built.

Layouts (head dim contiguous):
  q, o [B, Sq, Hq, 128]   k, v [B, Skv, Hkv, 128]   r [B, Sq, r_dim]
  P [Hq, r_dim, E]        R [B, Sq, Hq, E]          lse [B, Hq, Sq]
Query row t sits at position Skv - Sq + t.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "relproj", "attn_prefill", "attn_decode", "attn_decode_noalloc", "attn_paged", "splitkv_combine", "num_splits", "mxfp8_quantize",
    "attn_prologue", "cache_args",
    "decode_workspace_bytes", "lib_path", "RBAError",
    "RBA_OK", "RBA_E_INVALID", "RBA_E_UNSUPPORTED", "RBA_E_WORKSPACE", "RBA_E_LAUNCH",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "librba.so")

RBA_OK, RBA_E_INVALID, RBA_E_UNSUPPORTED, RBA_E_WORKSPACE, RBA_E_LAUNCH = range(5)
RBA_FP32, RBA_BF16 = 0, 1
RBA_DECODE_SCRATCH_BYTES = 16 << 20     # size of the scratch array of rba_attn_decode_noalloc
RBA_KV_PLAIN, RBA_KV_MXFP8, RBA_KV_MXFP8_QK = 0, 1, 2


class RBAError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {_lib.rba_status_string(code).decode()} (status {code})")


class _AttnArgs(ctypes.Structure):
    _fields_ = [
        ("dt", ctypes.c_int),
        ("B", ctypes.c_int), ("Sq", ctypes.c_int), ("Skv", ctypes.c_int),
        ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int), ("E", ctypes.c_int),
        ("window", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("log_scale_base", ctypes.c_float),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("R", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("q_s", ctypes.c_int64 * 3), ("k_s", ctypes.c_int64 * 3), ("v_s", ctypes.c_int64 * 3),
        ("o_s", ctypes.c_int64 * 3), ("R_s", ctypes.c_int64 * 3),
        ("kv_format", ctypes.c_int),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("k_scale_s", ctypes.c_int64 * 3), ("v_scale_s", ctypes.c_int64 * 3),
    ]


class _PagedKV(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("bt_stride", ctypes.c_int64),
        ("page_size", ctypes.c_int),
        ("num_pages", ctypes.c_int),
    ]


class _PrologueArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int),
        ("conv_w", ctypes.c_int),
        ("eps", ctypes.c_float),
        ("cu_new", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_s", ctypes.c_int64 * 2), ("k_s", ctypes.c_int64 * 2), ("v_s", ctypes.c_int64 * 2),
        ("conv_wk", ctypes.c_void_p), ("conv_wv", ctypes.c_void_p),
        ("norm_q", ctypes.c_void_p), ("norm_k", ctypes.c_void_p),
        ("state_k", ctypes.c_void_p), ("state_v", ctypes.c_void_p),
        ("q_out", ctypes.c_void_p),
        ("q_out_s", ctypes.c_int64 * 2),
        ("max_new", ctypes.c_int),
    ]


class _RelBias(ctypes.Structure):
    """rba_relbias: relative features and the packed projection of the fused prefill."""
    _fields_ = [
        ("r_dim", ctypes.c_int),
        ("r", ctypes.c_void_p),
        ("r_s", ctypes.c_int64 * 3),
        ("PT", ctypes.c_void_p),
    ]


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(
            f"librba.so not found at {lib_path}; build it with "
            "`python relative_position_bias_rba_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(lib_path)
    P = ctypes.POINTER(_AttnArgs)
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rba_relproj.argtypes = [ci, ci, i64, ci, ci, ci, vp, i64, i64, vp, vp, vp]
    lib.rba_relproj.restype = ci
    lib.rba_attn_prefill.argtypes = [P, vp]
    lib.rba_attn_prefill.restype = ci
    lib.rba_relproj_packed_bytes.argtypes = [ci, ci, ci]
    lib.rba_relproj_packed_bytes.restype = ctypes.c_size_t
    lib.rba_relproj_pack.argtypes = [ci, ci, ci, vp, vp, vp]
    lib.rba_relproj_pack.restype = ci
    lib.rba_prefill_fused_workspace_bytes.argtypes = [P]
    lib.rba_prefill_fused_workspace_bytes.restype = ctypes.c_size_t
    lib.rba_attn_prefill_fused.argtypes = [P, ctypes.POINTER(_RelBias), vp, ctypes.c_size_t, vp]
    lib.rba_attn_prefill_fused.restype = ci
    lib.rba_num_splits.argtypes = [P, ci]
    lib.rba_num_splits.restype = ci
    lib.rba_decode_workspace_bytes.argtypes = [P, ci]
    lib.rba_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.rba_attn_decode.argtypes = [P, ci, vp, ctypes.c_size_t, vp]
    lib.rba_attn_decode.restype = ci
    lib.rba_attn_decode_noalloc.argtypes = [P, ci, vp]
    lib.rba_attn_decode_noalloc.restype = ci
    lib.rba_attn_paged.argtypes = [P, ctypes.POINTER(_PagedKV), ci, vp, ctypes.c_size_t, vp]
    lib.rba_attn_paged.restype = ci
    lib.rba_attn_prologue.argtypes = [ctypes.POINTER(_PrologueArgs), P, ctypes.POINTER(_PagedKV), vp]
    lib.rba_attn_prologue.restype = ci
    lib.rba_splitkv_combine.argtypes = [vp, vp, ci, P, vp]
    lib.rba_splitkv_combine.restype = ci
    lib.rba_status_string.argtypes = [ci]
    lib.rba_status_string.restype = ctypes.c_char_p
    lib.rba_mxfp8_quantize.argtypes = [ci, i64, ci, vp, i64, vp, i64, vp, i64, vp]
    lib.rba_mxfp8_quantize.restype = ci
    lib.rba_calib_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.rba_calib_read.restype = ci
    lib.rba_calib_mfma.argtypes = [ci, vp, ctypes.POINTER(ctypes.c_double), vp]
    lib.rba_calib_mfma.restype = ci
    lib.rba_version.argtypes = []
    lib.rba_version.restype = ci
    return lib


_lib = _load()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RBA_BF16
    if t.dtype == torch.float32:
        return RBA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(fn: str, code: int):
    if code != RBA_OK:
        raise RBAError(fn, code)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_args(q, k, v, R=None, o=None, lse=None, *, window=0, scale=None, log_scale_base=0.0,
              dt=None, k_scale=None, v_scale=None, qk_fp8=False) -> _AttnArgs:
    """Fill the C argument struct from tensors (shapes and strides only).

    With k_scale / v_scale given, k and v are MXFP8 codes (uint8) and the
    scales their E8M0 codes [..., 128/32]; qk_fp8=True also encodes q and
    runs the logits in MXFP8 (rba_kv_format RBA_KV_MXFP8_QK)."""
    a = _AttnArgs()
    B, Sq, Hq, d = q.shape
    a.dt = _dt(q) if dt is None else dt
    a.B, a.Sq, a.Skv, a.Hq, a.Hkv, a.d = B, Sq, k.shape[1], Hq, k.shape[2], d
    a.E = 0 if R is None else R.shape[3]
    a.window = int(window)
    a.scale = float(1.0 / math.sqrt(d) if scale is None else scale)
    a.log_scale_base = float(log_scale_base or 0.0)
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.R = None if R is None else R.data_ptr()
    a.o = None if o is None else o.data_ptr()
    a.lse = None if lse is None else lse.data_ptr()
    for name, t in (("q_s", q), ("k_s", k), ("v_s", v), ("o_s", o), ("R_s", R)):
        if t is not None:
            if t.stride(3) != 1:
                raise ValueError(f"{name[0]}: innermost dimension must be contiguous")
            getattr(a, name)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    if (k_scale is None) != (v_scale is None):
        raise ValueError("give both k_scale and v_scale, or neither")
    if qk_fp8 and k_scale is None:
        raise ValueError("qk_fp8 needs an MXFP8 cache (k_scale, v_scale)")
    if k_scale is not None:
        a.kv_format = RBA_KV_MXFP8_QK if qk_fp8 else RBA_KV_MXFP8
        a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
        for name, t in (("k_scale_s", k_scale), ("v_scale_s", v_scale)):
            if t.dtype != torch.uint8 or t.stride(3) != 1:
                raise ValueError(f"{name}: uint8 with contiguous codes per row expected")
            getattr(a, name)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    return a


def _check_attn_inputs(q, k, v, R, k_scale=None, v_scale=None):
    for t in (q, k, v) + (() if R is None else (R,)) + tuple(x for x in (k_scale, v_scale) if x is not None):
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
    if R is not None and R.dtype != q.dtype:
        raise TypeError("q and R must share one dtype")
    if k_scale is not None:
        if k.dtype != torch.uint8 or v.dtype != torch.uint8 or q.dtype != torch.bfloat16:
            raise TypeError("MXFP8 K/V: k and v are uint8 codes and q is bfloat16")
    elif k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v and R must share one dtype")


def relproj(r: torch.Tensor, P: torch.Tensor, out_dtype=None, per_head: bool = False) -> torch.Tensor:
    """R[..., h, e] = sum_c r[..., c] P[h, c, e] on the GPU (MFMA kernel).

    per_head=True: r is [..., Hq, r_dim], one feature per head, and
    R[..., h, e] = sum_c r[..., h, c] P[h, c, e]."""
    if not (r.is_cuda and P.is_cuda):
        raise ValueError("tensors must live on the GPU")
    Hq, r_dim, E = P.shape
    if r.shape[-1] != r_dim:
        raise ValueError("r_dim mismatch")
    P = P.contiguous()
    if per_head:
        if r.dim() < 2 or r.shape[-2] != Hq:
            raise ValueError("per-head r must be [..., Hq, r_dim]")
        lead = r.shape[:-2]
        r3 = r.reshape(-1, Hq, r_dim)
        if r3.stride(2) != 1 or r3.stride(0) < Hq * r3.stride(1):
            r3 = r3.contiguous()
        rp, n, st, sh = r3, r3.shape[0], r3.stride(0), r3.stride(1)
    else:
        lead = r.shape[:-1]
        r2 = r.reshape(-1, r_dim)
        if r2.stride(1) != 1:
            r2 = r2.contiguous()
        rp, n, st, sh = r2, r2.shape[0], r2.stride(0), 0
    out_dtype = r.dtype if out_dtype is None else out_dtype
    R = torch.empty(*lead, Hq, E, dtype=out_dtype, device=r.device)
    code = _lib.rba_relproj(_dt(r), _dt(R), n, Hq, r_dim, E, _ptr(rp), st, sh,
                            _ptr(P), _ptr(R), _stream(r.device))
    _check("rba_relproj", code)
    return R


def attn_prefill(q, k, v, R=None, *, window=0, scale=None, log_scale_base=0.0, return_lse=False,
                 out=None, k_scale=None, v_scale=None, qk_fp8=False):
    """Attention of every query row over its visible keys (one pass).
    k_scale / v_scale: K and V are MXFP8 (see mxfp8_quantize); qk_fp8: the
    logits in MXFP8 too (q encoded, QK^T on the scaled FP8 matrix unit)."""
    _check_attn_inputs(q, k, v, R, k_scale, v_scale)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device) \
        if return_lse else None
    a = make_args(q, k, v, R, o, lse, window=window, scale=scale, log_scale_base=log_scale_base,
                  k_scale=k_scale, v_scale=v_scale, qk_fp8=qk_fp8)
    _check("rba_attn_prefill", _lib.rba_attn_prefill(ctypes.byref(a), _stream(q.device)))
    return (o, lse) if return_lse else o


class PackedProjection:
    """A projection P [Hq, r_dim, E] repacked by rba_relproj_pack: `data` is the
    packed bf16 buffer (opaque layout), the shape is kept beside it."""

    def __init__(self, data: torch.Tensor, Hq: int, r_dim: int, E: int):
        self.data, self.Hq, self.r_dim, self.E = data, Hq, r_dim, E


def relproj_pack(P: torch.Tensor) -> PackedProjection:
    """Repack a bf16 projection P [Hq, r_dim, E] (r_dim a multiple of 16, at
    most 128) on the GPU into the layout attn_prefill_fused reads.  Pack a
    weight once and keep the result."""
    if not P.is_cuda or P.dtype != torch.bfloat16 or P.dim() != 3:
        raise ValueError("P must be a bf16 [Hq, r_dim, E] GPU tensor")
    P = P.contiguous()
    Hq, r_dim, E = P.shape
    n = _lib.rba_relproj_packed_bytes(Hq, r_dim, E)
    if n == 0:
        _check("rba_relproj_pack", RBA_E_UNSUPPORTED)
    PT = torch.empty(n // 2, dtype=P.dtype, device=P.device)
    _check("rba_relproj_pack", _lib.rba_relproj_pack(Hq, r_dim, E, _ptr(P), _ptr(PT), _stream(P.device)))
    return PackedProjection(PT, Hq, r_dim, E)


def make_relbias(r: torch.Tensor, PT: PackedProjection, per_head: bool = False) -> _RelBias:
    """Fill the C relative-feature struct: r [B, Sq, r_dim] shared by the heads,
    or [B, Sq, Hq, r_dim] with per_head=True; PT from relproj_pack."""
    if r.stride(-1) != 1:
        raise ValueError("r: channels must be contiguous")
    if r.shape[-1] != PT.r_dim:
        raise ValueError("r_dim mismatch")
    rb = _RelBias()
    rb.r_dim = PT.r_dim
    rb.r, rb.PT = r.data_ptr(), PT.data.data_ptr()
    rb.r_s[:] = [r.stride(0), r.stride(1), r.stride(2) if per_head else 0]
    return rb


def prefill_fused_workspace_bytes(q, k, v, E: int, *, window=0) -> int:
    a = make_args(q, k, v, None, q, None, window=window)
    a.E = int(E)
    return _lib.rba_prefill_fused_workspace_bytes(ctypes.byref(a))


def attn_prefill_fused(q, k, v, r, PT: PackedProjection, *, per_head=False, window=0, scale=None,
                       log_scale_base=0.0, return_lse=False, out=None, workspace=None, on_chip=False):
    """relproj + attn_prefill in one launch, the relative logits computed inside
    the attention kernel from r and the packed projection PT (relproj_pack):
    by default each workgroup keeps the rows of R of its query block in its
    region of a workspace; on_chip=True (r_dim <= 64) computes each banded key
    tile's logits straight into LDS, with no workspace and no R in memory."""
    _check_attn_inputs(q, k, v, None)
    if not (r.is_cuda and PT.data.is_cuda) or r.dtype != q.dtype or PT.data.dtype != q.dtype:
        raise TypeError("r and PT must be GPU tensors of q's dtype")
    if PT.Hq != q.shape[2]:
        raise ValueError("PT was packed for another number of query heads")
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device) \
        if return_lse else None
    a = make_args(q, k, v, None, o, lse, window=window, scale=scale, log_scale_base=log_scale_base)
    a.E = PT.E
    rb = make_relbias(r, PT, per_head)
    if on_chip:
        if workspace is not None:
            raise ValueError("on_chip takes no workspace")
        code = _lib.rba_attn_prefill_fused(ctypes.byref(a), ctypes.byref(rb), None, 0, _stream(q.device))
        _check("rba_attn_prefill_fused", code)
        return (o, lse) if return_lse else o
    need = _lib.rba_prefill_fused_workspace_bytes(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    code = _lib.rba_attn_prefill_fused(ctypes.byref(a), ctypes.byref(rb), ctypes.c_void_p(workspace.data_ptr()),
                                       ws_bytes, _stream(q.device))
    _check("rba_attn_prefill_fused", code)
    return (o, lse) if return_lse else o


def num_splits(q, k, v, R=None, *, window=0, num_cus=0, log_scale_base=0.0) -> int:
    a = make_args(q, k, v, R, q, None, window=window, log_scale_base=log_scale_base)
    return _lib.rba_num_splits(ctypes.byref(a), int(num_cus))


def decode_workspace_bytes(q, k, v, R=None, *, window=0, splits=0) -> int:
    a = make_args(q, k, v, R, q, None, window=window)
    return _lib.rba_decode_workspace_bytes(ctypes.byref(a), int(splits))


def attn_decode(q, k, v, R=None, *, window=0, scale=None, log_scale_base=0.0, num_splits=0,
                return_lse=False, out=None, workspace=None, k_scale=None, v_scale=None, qk_fp8=False):
    """Split-KV attention of a few query rows against a long KV cache.
    k_scale / v_scale: K and V are MXFP8 (see mxfp8_quantize); qk_fp8: the
    logits in MXFP8 too."""
    _check_attn_inputs(q, k, v, R, k_scale, v_scale)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device) \
        if return_lse else None
    a = make_args(q, k, v, R, o, lse, window=window, scale=scale, log_scale_base=log_scale_base,
                  k_scale=k_scale, v_scale=v_scale, qk_fp8=qk_fp8)
    splits = int(num_splits)
    if splits == 0:
        splits = _lib.rba_num_splits(ctypes.byref(a), 0)
        if splits <= 0:
            _check("rba_num_splits", RBA_E_INVALID)
    need = _lib.rba_decode_workspace_bytes(ctypes.byref(a), splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _lib.rba_attn_decode(ctypes.byref(a), splits, ws_ptr, ws_bytes, _stream(q.device))
    _check("rba_attn_decode", code)
    return (o, lse) if return_lse else o


def attn_decode_noalloc(q, k, v, R=None, *, window=0, scale=None, log_scale_base=0.0, num_splits=0,
                        out=None, lse=None, k_scale=None, v_scale=None, qk_fp8=False):
    """attn_decode with the split partials in the library's own device
    scratch array (rba_attn_decode_noalloc): the C call allocates nothing.
    Pass `out` (and `lse` [B, Hq, Sq] fp32, optional) to keep this wrapper
    from allocating them.  Calls that overlap on one device race."""
    _check_attn_inputs(q, k, v, R, k_scale, v_scale)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    a = make_args(q, k, v, R, o, lse, window=window, scale=scale, log_scale_base=log_scale_base,
                  k_scale=k_scale, v_scale=v_scale, qk_fp8=qk_fp8)
    code = _lib.rba_attn_decode_noalloc(ctypes.byref(a), int(num_splits), _stream(q.device))
    _check("rba_attn_decode_noalloc", code)
    return (o, lse) if lse is not None else o


def make_paged(block_table, seq_lens, page_size: int, num_pages: int) -> _PagedKV:
    """Fill the C paged-cache struct (pointers and sizes only)."""
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [B, n] with contiguous rows")
    kv = _PagedKV()
    kv.block_table = block_table.data_ptr()
    kv.seq_lens = seq_lens.data_ptr()
    kv.bt_stride = block_table.stride(0)
    kv.page_size = int(page_size)
    kv.num_pages = int(num_pages)
    return kv


def attn_paged(q, k_pool, v_pool, block_table, seq_lens, R=None, *, max_seq_len=None, window=0, scale=None,
               log_scale_base=0.0, num_splits=0, return_lse=False, out=None, workspace=None, k_scale=None,
               v_scale=None, qk_fp8=False):
    """Attention of each sequence's last Sq query rows over its own keys in a
    paged pool k_pool / v_pool [num_pages, page_size, Hkv, 128].

    block_table int32 [B, n] (device) lists each sequence's pages; seq_lens
    int32 [B] (device) its key count.  max_seq_len (default n * page_size)
    bounds seq_lens and drives the split heuristic."""
    _check_attn_inputs(q, k_pool, v_pool, R, k_scale, v_scale)
    if not (block_table.is_cuda and seq_lens.is_cuda):
        raise ValueError("block_table and seq_lens must live on the GPU")
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device) \
        if return_lse else None
    num_pages, page_size = k_pool.shape[0], k_pool.shape[1]
    if v_pool.shape[:2] != k_pool.shape[:2]:
        raise ValueError("k_pool and v_pool must have the same pages")
    a = make_args(q, k_pool, v_pool, R, o, lse, window=window, scale=scale, log_scale_base=log_scale_base,
                  k_scale=k_scale, v_scale=v_scale, qk_fp8=qk_fp8)
    a.Skv = int(block_table.shape[1] * page_size if max_seq_len is None else max_seq_len)
    kv = make_paged(block_table, seq_lens, page_size, num_pages)
    splits = int(num_splits)
    if splits == 0:
        splits = _lib.rba_num_splits(ctypes.byref(a), 0)
        if splits <= 0:
            _check("rba_num_splits", RBA_E_INVALID)
    need = _lib.rba_decode_workspace_bytes(ctypes.byref(a), splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _lib.rba_attn_paged(ctypes.byref(a), ctypes.byref(kv), splits, ws_ptr, ws_bytes, _stream(q.device))
    _check("rba_attn_paged", code)
    return (o, lse) if return_lse else o


def mxfp8_quantize(x: torch.Tensor):
    """MXFP8 codes and E8M0 scales of x [..., n] (n a multiple of 32) along its
    last axis: (uint8 [..., n], uint8 [..., n/32])."""
    if not x.is_cuda:
        raise ValueError("tensors must live on the GPU")
    n = x.shape[-1]
    x2 = x.reshape(-1, n)
    if x2.stride(1) != 1 or (x2.stride(0) * x2.element_size()) % 16 or x2.data_ptr() % 16:
        x2 = x2.contiguous()
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(*x.shape[:-1], n // 32, dtype=torch.uint8, device=x.device)
    code = _lib.rba_mxfp8_quantize(_dt(x), x2.shape[0], n, _ptr(x2), x2.stride(0), _ptr(codes), n,
                                   _ptr(scales), n // 32, _stream(x.device))
    _check("rba_mxfp8_quantize", code)
    return codes, scales


def cache_args(k_cache, v_cache, *, k_scale=None, v_scale=None, max_seq_len=None) -> _AttnArgs:
    """The C description of a KV cache alone (dense [B, Skv, Hkv, d] or a page
    pool [num_pages, page_size, Hkv, d]; bf16, or MXFP8 codes with scales)."""
    a = _AttnArgs()
    a.dt, a.d, a.Hkv = RBA_BF16, k_cache.shape[3], k_cache.shape[2]
    a.Skv = k_cache.shape[1] if max_seq_len is None else int(max_seq_len)
    a.k, a.v = k_cache.data_ptr(), v_cache.data_ptr()
    a.k_s[:] = [k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)]
    a.v_s[:] = [v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)]
    if k_scale is not None:
        a.kv_format = RBA_KV_MXFP8
        a.k_scale, a.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
        a.k_scale_s[:] = [k_scale.stride(0), k_scale.stride(1), k_scale.stride(2)]
        a.v_scale_s[:] = [v_scale.stride(0), v_scale.stride(1), v_scale.stride(2)]
    return a


def attn_prologue(q, k, v, cu_new, seq_lens, conv_wk, conv_wv, norm_q, norm_k, state_k, state_v, k_cache, v_cache,
                  *, eps=1e-6, k_scale=None, v_scale=None, block_table=None, max_seq_len=None, q_out=None,
                  max_new=0):
    """Attention prologue for T new tokens: returns q_out = RMSNorm(q) and writes
    RMSNorm(ShortConv(k)) and ShortConv(v) into the cache at each sequence's new
    positions, then advances the conv states (see rba.h for the layouts).
    block_table (int32 [B, n]) makes k_cache / v_cache page pools.  max_new (a
    bound on any sequence's new tokens, 0 = none) selects the one-launch path."""
    T, Hq, d = q.shape
    W = conv_wk.shape[1]
    for t in (q, k, v, cu_new, seq_lens, conv_wk, conv_wv, norm_q, norm_k, k_cache, v_cache):
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("projections are bfloat16")
    for t in (conv_wk, conv_wv, norm_q, norm_k):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError("conv taps and norm weights are contiguous float32")
    out = torch.empty(T, Hq, d, dtype=torch.bfloat16, device=q.device) if q_out is None else q_out
    a = _PrologueArgs()
    a.B, a.T, a.Hq, a.Hkv, a.d, a.conv_w, a.eps = seq_lens.shape[0], T, Hq, k.shape[1], d, W, float(eps)
    a.max_new = int(max_new)
    a.cu_new, a.seq_lens = cu_new.data_ptr(), seq_lens.data_ptr()
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    for name, t in (("q_s", q), ("k_s", k), ("v_s", v), ("q_out_s", out)):
        if t.stride(2) != 1:
            raise ValueError(f"{name}: innermost dimension must be contiguous")
        getattr(a, name)[:] = [t.stride(0), t.stride(1)]
    a.conv_wk, a.conv_wv = conv_wk.data_ptr(), conv_wv.data_ptr()
    a.norm_q, a.norm_k = norm_q.data_ptr(), norm_k.data_ptr()
    a.state_k = None if state_k is None else state_k.data_ptr()
    a.state_v = None if state_v is None else state_v.data_ptr()
    a.q_out = out.data_ptr()
    if block_table is not None:
        ms = block_table.shape[1] * k_cache.shape[1] if max_seq_len is None else max_seq_len
        c = cache_args(k_cache, v_cache, k_scale=k_scale, v_scale=v_scale, max_seq_len=ms)
        kv = make_paged(block_table, seq_lens, k_cache.shape[1], k_cache.shape[0])
        kvp = ctypes.byref(kv)
    else:
        c = cache_args(k_cache, v_cache, k_scale=k_scale, v_scale=v_scale)
        kvp = None
    code = _lib.rba_attn_prologue(ctypes.byref(a), ctypes.byref(c), kvp, _stream(q.device))
    _check("rba_attn_prologue", code)
    return out


def splitkv_combine(o_part, lse_part, q_like, k_like, *, out=None, return_lse=False):
    """Merge split partials o_part [S, B, Sq, Hq, d] / lse_part [S, B, Sq, Hq] (fp32)."""
    S, B, Sq, Hq, d = o_part.shape
    o = torch.empty(B, Sq, Hq, d, dtype=q_like.dtype, device=o_part.device) if out is None else out
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=o_part.device) if return_lse else None
    a = make_args(q_like, k_like, k_like, None, o, lse)
    code = _lib.rba_splitkv_combine(ctypes.c_void_p(o_part.data_ptr()), ctypes.c_void_p(lse_part.data_ptr()),
                                    S, ctypes.byref(a), _stream(o_part.device))
    _check("rba_splitkv_combine", code)
    return (o, lse) if return_lse else o
