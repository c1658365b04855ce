"""Guards around every buffer the library writes, and run-to-run determinism.

Outputs, lse and the split-KV workspace are carved out of larger buffers whose
surrounding bytes hold a canary; after prefill, decode (split), paged and
MXFP8 calls and the attention prologue the canaries must be intact (no write
outside a destination).  The kernels use no atomics, so two identical calls
must agree bit for bit.
"""
import ctypes
import sys

import pytest
import torch

from workloads import CONFIGS, make_inputs, make_paged_inputs, make_prologue_inputs
from workloads.configs import scaled

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAD = 4096          # guard elements on each side


def rba():
    import relative_position_bias_rba_amd as m  # fails loudly if librba.so is missing
    return m


def guarded(shape, dtype, fill):
    """A tensor of `shape` inside a buffer with PAD canary elements on each side."""
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + 2 * PAD,), fill, dtype=dtype, device=DEV)
    return buf, buf[PAD:PAD + n].view(*shape)


def intact(buf, n, fill):
    return bool(torch.all(buf[:PAD] == fill)) and bool(torch.all(buf[PAD + n:] == fill))


def test_attention_writes_stay_inside_their_buffers():
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], B=3, Sq=9, Skv=700, Hq=16, Hkv=2, E=64, window=0)
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    for name, splits in (("prefill", None), ("decode", 1), ("decode", 5)):
        ob, o = guarded(tuple(d["q"].shape), torch.bfloat16, 7.0)
        lb, lse = guarded((w.B, w.Hq, w.Sq), torch.float32, 7.0)
        a = m.make_args(d["q"], d["k"], d["v"], R, o, lse)
        if splits is None:
            assert m._lib.rba_attn_prefill(ctypes.byref(a), m._stream(torch.device(DEV))) == 0
        else:
            need = m._lib.rba_decode_workspace_bytes(ctypes.byref(a), splits)
            wb, ws = guarded((max(need, 16),), torch.uint8, 0xA5)
            assert m._lib.rba_attn_decode(ctypes.byref(a), splits, ctypes.c_void_p(ws.data_ptr()), need,
                                          m._stream(torch.device(DEV))) == 0
        torch.cuda.synchronize()
        assert intact(ob, o.numel(), 7.0), (name, splits, "o")
        assert intact(lb, lse.numel(), 7.0), (name, splits, "lse")
        if splits is not None:
            assert intact(wb, max(need, 16), 0xA5), (name, splits, "workspace")
        print(f"{name}/{splits}: guards intact", flush=True)


def test_paged_mxfp8_and_prologue_are_deterministic():
    m = rba()
    w = scaled(CONFIGS["c4_decode_full"], B=3, Sq=9, Skv=640, Hq=16, Hkv=2, E=64, window=0)
    inp = make_paged_inputs(w, 64, seq_lens=[640, 100, 300])
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    kc, ks = m.mxfp8_quantize(d["k_pool"])
    vc, vs = m.mxfp8_quantize(d["v_pool"])
    outs = []
    for _ in range(2):
        o1, l1 = m.attn_paged(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_lens"], R,
                              max_seq_len=640, num_splits=3, return_lse=True)
        o2, l2 = m.attn_paged(d["q"], kc, vc, d["block_table"], d["seq_lens"], R, max_seq_len=640, num_splits=0,
                              return_lse=True, k_scale=ks, v_scale=vs)
        c2, s2 = m.mxfp8_quantize(d["k_pool"])
        outs.append((o1, l1, o2, l2, c2, s2))
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    pi = make_prologue_inputs([1, 9, 20], [300, 9, 100], Hq=16, Hkv=2, W=4)
    pd = {k: v.to(DEV) for k, v in pi.items()}
    for max_new in (0, 20):          # chunked, and one launch
        res = []
        for _ in range(2):
            kcache = torch.zeros(3, 320, 2, 128, dtype=torch.bfloat16, device=DEV)
            vcache = torch.zeros_like(kcache)
            sk, sv = pd["state_k"].clone(), pd["state_v"].clone()
            qo = m.attn_prologue(pd["q"], pd["k"], pd["v"], pd["cu_new"], pd["seq_lens"], pd["conv_wk"],
                                 pd["conv_wv"], pd["norm_q"], pd["norm_k"], sk, sv, kcache, vcache, max_new=max_new)
            res.append((qo, kcache, vcache, sk, sv))
        torch.cuda.synchronize()
        for x, y in zip(*res):
            assert torch.equal(x, y)


@pytest.mark.parametrize("max_new", [0, 20], ids=["chunked", "one_launch"])
def test_prologue_writes_stay_inside_their_buffers(max_new):
    m = rba()
    pi = make_prologue_inputs([1, 9, 20], [300, 9, 100], Hq=16, Hkv=2, W=4, seed=5)
    pd = {k: v.to(DEV) for k, v in pi.items()}
    qb, qo = guarded((30, 16, 128), torch.bfloat16, 3.0)
    kb, kcache = guarded((3, 320, 2, 128), torch.bfloat16, 3.0)
    vb, vcache = guarded((3, 320, 2, 128), torch.bfloat16, 3.0)
    skb, sk = guarded(tuple(pd["state_k"].shape), torch.bfloat16, 3.0)
    svb, sv = guarded(tuple(pd["state_v"].shape), torch.bfloat16, 3.0)
    sk.copy_(pd["state_k"])
    sv.copy_(pd["state_v"])
    m.attn_prologue(pd["q"], pd["k"], pd["v"], pd["cu_new"], pd["seq_lens"], pd["conv_wk"], pd["conv_wv"],
                    pd["norm_q"], pd["norm_k"], sk, sv, kcache, vcache, q_out=qo, max_new=max_new)
    torch.cuda.synchronize()
    for name, b, t in (("q_out", qb, qo), ("k cache", kb, kcache), ("v cache", vb, vcache), ("state k", skb, sk),
                       ("state v", svb, sv)):
        assert intact(b, t.numel(), 3.0), name
