"""rba_attn_decode_noalloc (split partials in the library's device scratch
array) against rba_attn_decode (caller workspace) through the C ABI: two
calls in a row, the second smaller, each bit-identical to the workspace path
and within the bf16 tolerances of the fp64 oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_inputs
from workloads.configs import scaled

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_call(m, w, splits):
    inp = make_inputs(w)
    d = {k: v.to(DEV) for k, v in inp.items()}
    R = m.relproj(d["r"], d["P"])
    kw = dict(window=w.window, log_scale_base=w.log_scale_base, num_splits=splits)
    o_ref, l_ref = m.attn_decode(d["q"], d["k"], d["v"], R, return_lse=True, **kw)
    o = torch.full_like(d["q"], float("nan"))
    lse = torch.full((w.B, w.Hq, w.Sq), float("nan"), dtype=torch.float32, device=DEV)
    m.attn_decode_noalloc(d["q"], d["k"], d["v"], R, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    n = m.num_splits(d["q"], d["k"], d["v"], R, window=w.window) if splits == 0 else splits
    need = m.decode_workspace_bytes(d["q"], d["k"], d["v"], R, window=w.window, splits=n)
    say(f"no-alloc decode {w.name} B={w.B} Sq={w.Sq} Skv={w.Skv} Hq={w.Hq} splits={n} partials={need} B")
    assert n > 1 and 0 < need <= m.RBA_DECODE_SCRATCH_BYTES
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    wo, wl = oracle.attention(inp["q"], inp["k"], inp["v"], oracle.relproj(inp["r"], inp["P"]), window=w.window,
                              log_scale_base=w.log_scale_base)
    g = o.double().cpu().numpy()
    dd = np.abs(g - wo)
    rel = float(np.linalg.norm(g - wo) / np.linalg.norm(wo))
    say(f"  max|d|={dd.max():.3e} mean|d|={dd.mean():.3e} rel_l2={rel:.3e}")
    assert dd.max() <= 2e-2 and dd.mean() <= 2e-3 and rel <= 1e-2
    assert np.abs(lse.cpu().numpy() - wl).max() <= 2e-2


def test_decode_noalloc_two_calls_second_smaller():
    import relative_position_bias_rba_amd as m
    big = scaled(CONFIGS["c5_long_decode"], Skv=20000)                    # heuristic splits, 64 rows
    one_call(m, big, 0)
    small = scaled(CONFIGS["c4_decode_swa"], B=2, Sq=9, Skv=1500, Hq=16, Hkv=2, E=64, window=256)
    one_call(m, small, 3)
