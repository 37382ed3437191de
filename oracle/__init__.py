"""CPU oracle for the RMSNorm forward/backward path (and LayerNorm / GroupNorm / softmax) — TEST INFRASTRUCTURE, NOT PRODUCT CODE.

A plain, slow, directly checkable NumPy implementation of what the GPU library computes: float64
reductions, float32 elementwise arithmetic emulated with NumPy float32 operations, and
round-to-nearest-even to bfloat16 / binary16 written from the IEEE 754 definition.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. The GPU library and its Python binding never import it, and it imports nothing from
them: the two share no code. Every function is pinned by CPU tests to values the pages print,
closed forms, invariants, library conversions and float64 finite differences.
"""
from .rounding import round_to_format, rne_bf16, rne_f16, rne_f32, rne_fp8, rne_to, ulp_of
from .rmsnorm import (CASTS, DTYPES, ROUNDINGS, apply_gain, gain, rmsnorm_bwd, rmsnorm_dw, rmsnorm_fwd,
                      rmsnorm_fwd_fp8, rstd_of)
from .layernorm import groupnorm_bwd, groupnorm_fwd, layernorm_bwd, layernorm_fwd, row_stats
from .softmax import rmsnorm_bwd_f64, rmsnorm_fwd_f64, softmax_bwd, softmax_fwd

__all__ = [
    "round_to_format", "rne_bf16", "rne_f16", "rne_f32", "rne_fp8", "rne_to", "ulp_of",
    "CASTS", "DTYPES", "ROUNDINGS", "apply_gain", "gain", "rmsnorm_bwd", "rmsnorm_dw", "rmsnorm_fwd",
    "rmsnorm_fwd_fp8", "rstd_of",
    "groupnorm_bwd", "groupnorm_fwd", "layernorm_bwd", "layernorm_fwd", "row_stats",
    "rmsnorm_bwd_f64", "rmsnorm_fwd_f64", "softmax_bwd", "softmax_fwd",
]
