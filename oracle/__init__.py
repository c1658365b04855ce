"""fp64 CPU oracle (test infrastructure only; see rba_oracle.py)."""
from .rba_oracle import (attention, attention_paged, attention_partial, attention_rows, brute_attention,
                         gather_pages, log_scale_factor, lse_combine, relproj)

__all__ = ["attention", "attention_paged", "attention_partial", "gather_pages", "attention_rows", "brute_attention",
           "log_scale_factor", "lse_combine", "relproj"]
