"""fp64 CPU oracle (test infrastructure only; see rba_oracle.py)."""
from .rba_oracle import (attention, attention_paged, attention_partial, attention_rows, brute_attention,
                         e4m3_value, gather_pages, log_scale_factor, lse_combine, mxfp8_dequantize,
                         mxfp8_quantize, relproj, short_conv, rms_norm, attention_prologue,
                         attention_mxfp8_logits)

__all__ = ["attention", "attention_paged", "attention_partial", "gather_pages", "attention_rows", "brute_attention",
           "log_scale_factor", "lse_combine", "relproj", "e4m3_value", "mxfp8_quantize", "mxfp8_dequantize",
           "short_conv", "rms_norm", "attention_prologue", "attention_mxfp8_logits"]
