"""Plain CPU softmax over the last dimension, forward and backward, and the float64 RMSNorm.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle (see ``oracle/__init__.py``).

Source: "Add backward passes to the fused rms_norm, layer_norm and softmax_last_dim ops" (candle
pull request 4059), Conversation:

* the softmax backward is dx = y * (dy - sum(dy * y)), the sum taken in float32 for the 16-bit
  types and in float64 for float64 inputs;
* the fused softmax forward computes in float32 for bf16 / f16 and rounds once at the store (before
  the change it stored exp in bf16 and scaled it, rounding twice); float32 and float64 compute in
  their own type;
* the float64 norm kernels accumulate their statistics in float64 (they used float before, so the
  forward's statistics differed from the backward's), checked against the composed formulation to
  1e-10.

Forward (the definition, correctly rounded): with m the row maximum,

    y_j = RNE_T( exp(x_j - m) / sum_k exp(x_k - m) )        evaluated in float64, rounded once

(for T = float64 the float64 value itself). Subtracting the maximum does not change the real
result; it keeps exp from overflowing. A row of -inf only has no defined softmax (NaN).

Backward, from the forward's output y (T values) and the upstream gradient dy:

    s  = RNE_f32( sum_j dy_j * y_j )          (float64 sum; float64 result for T = float64)
    dx = RNE_T( fl( y * fl(dy - s) ) )        each operation one float32 (float64) operation

This is the exact derivative of softmax: d y_i / d x_j = y_i (delta_ij - y_j).

The float64 RMSNorm (``rmsnorm_fwd_f64`` / ``rmsnorm_bwd_f64``) is the RMSNorm of
``oracle.rmsnorm`` evaluated entirely in float64 with epsilon the given float64 value (the backward
is that module's ``exact`` mode), the composed formulation the candle page checks against.
"""
from __future__ import annotations

import numpy as np

from .rmsnorm import rmsnorm_bwd
from .rounding import rne_f32, rne_to

DTYPES = ("f32", "f16", "bf16", "f64")


def _check(dtype: str) -> None:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")


def _round(v, dtype: str):
    if dtype == "f64":
        return np.asarray(v, np.float64)
    if dtype == "f32":
        return rne_f32(v)
    return rne_to(v, dtype)


def softmax_fwd(x, *, dtype: str = "bf16", exact: bool = False):
    """Softmax over the last axis. Returns T values (float32 array; float64 for "f64" or exact)."""
    _check(dtype)
    x64 = np.asarray(x, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m = np.max(x64, axis=-1, keepdims=True)
        e = np.exp(x64 - m)
        y = e / np.sum(e, axis=-1, keepdims=True)
    return y if exact else _round(y, dtype)


def softmax_bwd(dy, y, *, dtype: str = "bf16", exact: bool = False):
    """dx = y * (dy - sum(dy * y)) over the last axis, from the forward's output y."""
    _check(dtype)
    wide = exact or dtype == "f64"
    F = np.float64 if wide else np.float32
    y = np.asarray(y, F)
    dy = np.asarray(dy, F)
    with np.errstate(invalid="ignore", over="ignore"):
        s = np.sum(dy.astype(np.float64) * y.astype(np.float64), axis=-1, keepdims=True)
        if not wide:
            s = rne_f32(s)
        dx = y * (dy - s.astype(F))
    return dx if exact else _round(dx, dtype)


def rmsnorm_fwd_f64(x, w, *, eps: float, offset: float = 0.0):
    """RMSNorm in float64 throughout, epsilon the given float64 value: ``(y, rstd)``.

    rstd = 1 / sqrt(sum(x^2) / N + eps), y = (x * rstd) * (offset + w), each a float64 operation
    (the sum in NumPy's float64 order)."""
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        rstd = 1.0 / np.sqrt(np.sum(x * x, axis=-1) / n + np.float64(eps))
        y = (x * rstd[..., None]) * (np.float64(offset) + np.asarray(w, np.float64))
    return y, rstd


def rmsnorm_bwd_f64(dy, x, w, rstd, *, offset: float = 0.0):
    """Backward of ``rmsnorm_fwd_f64``: ``(dx, dw)`` as float64 arrays."""
    return rmsnorm_bwd(np.asarray(dy, np.float64), np.asarray(x, np.float64),
                       np.asarray(w, np.float64), np.asarray(rstd, np.float64), offset=offset,
                       dtype="f32", exact=True)
