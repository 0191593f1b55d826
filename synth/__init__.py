"""Seeded synthetic workloads for the CSA2 decode path.

This package only draws random inputs (queries, merge inputs, page tables,
context lengths) and describes the workload shapes.  It holds none of the
method's arithmetic: no merging, quantisation, scoring, selection or
attention.  Both the HIP path's tests and the CPU oracle's tests feed from it.
"""
from .configs import CONFIGS, DecodeConfig, PrefillConfig, LayerSpec, small_decode, small_prefill
from .gen import Gen, DecodeCase, PrefillCase, make_decode_case, make_prefill_case

__all__ = [
    "CONFIGS", "DecodeConfig", "PrefillConfig", "LayerSpec", "small_decode", "small_prefill",
    "Gen", "DecodeCase", "PrefillCase", "make_decode_case", "make_prefill_case",
]
