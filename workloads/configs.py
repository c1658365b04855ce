"""The five workload shapes of the relative-position-bias attention path.

Layouts (row-major, head dim contiguous):
  q, o : [B, Sq, Hq, d]        k, v : [B, Skv, Hkv, d]
  r    : [B, Sq, r_dim]        P    : [Hq, r_dim, E]       R : [B, Sq, Hq, E]
A query row t sits at absolute position p = Skv - Sq + t (bottom-right aligned),
so a decode step of Sq new tokens sees a cache of Skv positions that already
holds those tokens.

The shapes follow the serving setting the Inkling pages describe: GQA with
head size 128 in every layer, sliding-window layers mixed with full-attention
layers that may apply a length-dependent log-scale, and up to 9 tokens per
forward step under MTP ("vLLM TML Inkling サポート", section
"TML Inkling モデルアーキテクチャ").  Prefill length 8192 and cache length
8192 + 1024 stand in for the 8K-input / 1K-output prompts the pages measure
on; 262144 is the 256K context window offered by the hosted service
("vLLM hỗ trợ TML Inkling ...", feature list).  Values are synthetic normals.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "fp32" or "bf16": the arithmetic type the path computes in
    B: int
    Sq: int
    Skv: int
    Hq: int
    Hkv: int
    d: int
    r_dim: int
    E: int                # rel_extent: bias entries for distances 0..E-1
    window: int           # 0 = full causal; else key visible iff 0 <= p - j < window
    log_scale_base: float # 0 = off; else logits multiplied by ln(p+1)/ln(base)
    qk_std: float         # std of q and k draws
    v_std: float
    r_std: float
    p_std: float          # std of the learned projection P
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def visible_pairs(self) -> int:
        """Number of visible (query, key) pairs per (batch, head) summed over batch."""
        tot = 0
        for t in range(self.Sq):
            p = self.Skv - self.Sq + t
            lo = 0 if self.window == 0 else max(0, p - self.window + 1)
            tot += p - lo + 1
        return tot * self.B

    def attn_flops(self) -> int:
        """Algorithmic flops: 4*d per visible (query, key) pair per query head."""
        return 4 * self.d * self.Hq * self.visible_pairs()

    def kv_bytes(self) -> int:
        """K+V bytes of the union of visible key positions per (batch, kv head)."""
        esz = 4 if self.dtype == "fp32" else 2
        p_lo = self.Skv - self.Sq
        p_hi = self.Skv - 1
        lo = 0 if self.window == 0 else max(0, p_lo - self.window + 1)
        n = p_hi - lo + 1
        return self.B * self.Hkv * n * 2 * self.d * esz

    def relproj_flops(self) -> int:
        return 2 * self.B * self.Sq * self.Hq * self.r_dim * self.E


_D = 128
_QK_SMALL = 1.0 / (_D ** 0.25)   # "N(0,1)/sqrt(d)^0.5" read as N(0,1)/d^(1/4)

CONFIGS = {
    "c1_tiny_fp32": Workload("c1_tiny_fp32", "fp32", 1, 256, 256, 4, 1, _D, 32, 64, 0, 0.0,
                             1.0, 1.0, 1.0, 0.02, 1001),
    "c2_swa_prefill": Workload("c2_swa_prefill", "bf16", 1, 8192, 8192, 64, 8, _D, 64, 512, 4096, 0.0,
                               _QK_SMALL, 1.0, 1.0, 0.02, 1002),
    "c3_full_prefill": Workload("c3_full_prefill", "bf16", 2, 32768, 32768, 64, 8, _D, 64, 512, 0, 4096.0,
                                _QK_SMALL, 1.0, 1.0, 0.02, 1003),
    "c4_decode_swa": Workload("c4_decode_swa", "bf16", 64, 9, 9216, 64, 8, _D, 64, 512, 4096, 0.0,
                              1.0, 1.0, 1.0, 0.02, 1004),
    "c4_decode_full": Workload("c4_decode_full", "bf16", 64, 9, 9216, 64, 8, _D, 64, 512, 0, 0.0,
                               1.0, 1.0, 1.0, 0.02, 1004),
    "c5_long_decode": Workload("c5_long_decode", "bf16", 1, 1, 262144, 64, 8, _D, 64, 512, 0, 4096.0,
                               1.0, 1.0, 1.0, 0.02, 1005),
}


def get(name: str) -> Workload:
    return CONFIGS[name]


def scaled(w: Workload, **over) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **over)
