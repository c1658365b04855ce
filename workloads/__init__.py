"""Seeded synthetic inputs for the relative-position-bias attention path.

This package holds shapes and random draws only: no step of the attention
method is computed here.  Both the fp64 oracle (``oracle/``) and the HIP path
(``relative_position_bias_rba_amd``) take their inputs from it, so the two
sides see the same values without sharing any arithmetic.
"""
from .configs import CONFIGS, Workload, get
from .gen import make_inputs, make_paged_inputs, make_prologue_inputs, randn

__all__ = ["CONFIGS", "Workload", "get", "make_inputs", "make_paged_inputs", "make_prologue_inputs", "randn"]
