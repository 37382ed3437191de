"""Plain CPU LayerNorm and GroupNorm forward and backward, float32 statistics.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle (see ``oracle/__init__.py``).

Sources (pages, by title):

* "Add backward passes to the fused rms_norm, layer_norm and softmax_last_dim ops" (candle pull
  request 4059): the layer_norm backward is the composed rule (the derivative of the formula) with
  the statistics in float32 for the 16-bit types; the fused forward keeps two partial sums per row
  and stores once at the end.
* "fix(group_norm): keep the backward statistics and reductions in fp32" (Liger-Kernel pull
  request 1608), Summary and commit message: Mean and RSTD are stored in float32 (as layer_norm
  already did), and the backward upcasts W, X and the upstream gradient to float32 on load and
  runs its reductions in float32. Its Details table compares the input, weight and bias gradients
  of GroupNorm with float32 autograd; its issue snippets expect an input gradient of exactly zero
  for an upstream gradient of ones.

Neither page prints the formulas; they are the textbook definitions (the plainest reading):

LayerNorm, per row r of an [M, N] matrix (``fl`` one float32 operation, sums in float64 then one
rounding to float32, ``RNE_T`` round-to-nearest-even to the I/O dtype):

    mean_r = RNE_f32( (sum_j x_rj) / N )
    rstd_r = RNE_f32( 1 / sqrt( (sum_j (x_rj - mu_r)^2) / N + eps ) )   mu_r the float64 mean
    xhat   = fl( fl(x - mean) * rstd )                                    from the float32 caches
    y      = RNE_T( fl( fl(xhat * w) + b ) )       (y = RNE_T(fl(xhat * w)) without a bias)

The variance is taken about the mean (not as E[x^2] - mean^2), so a large common offset of the
row does not cancel it away. One cast at the store, as the candle page describes for its fused
forward.

Backward, from the forward's float32 mean and rstd:

    xhat = fl( fl(x - mean) * rstd ),   gdy = fl(w * dy)
    c1   = RNE_f32( (sum_j gdy_j) / N ),   c2 = RNE_f32( (sum_j gdy_j * xhat_j) / N )
    dx   = RNE_T( fl( rstd * fl( fl(gdy - c1) - fl(xhat * c2) ) ) )
    dw_j = RNE_f32( sum_r dy_rj * xhat_rj ),   db_j = RNE_f32( sum_r dy_rj )     (float32 outputs)

This is the exact derivative of y = (x - mu) * r * w + b with r = (var + eps)^(-1/2):
dL/dx_i = r * (g_i - mean_j g_j - xhat_i * mean_j(g_j xhat_j)) for g = w * dy.

GroupNorm: x is [B, C, S] (S the flattened spatial size), C split into G groups of Cg = C / G
adjacent channels. The statistics are those of LayerNorm over each (batch, group) row of
n = Cg * S elements; the affine weight and bias are per channel, w_c and b_c for every element of
channel c. The backward uses the row constants c1, c2 over the n elements of the group, and
dW_c = sum over batch and space of dy * xhat, dB_c = sum over batch and space of dy.

``exact=True`` evaluates the same formulas in float64 with no rounding (the real-number function).
"""
from __future__ import annotations

import numpy as np

from .rounding import rne_f32, rne_to

DTYPES = ("f32", "f16", "bf16")


def _check(dtype: str) -> None:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")


def row_stats(x, eps: float, exact: bool = False):
    """Per-row mean and rstd of the last axis (float64 sums; float32 results unless exact)."""
    x64 = np.asarray(x, np.float64)
    n = x64.shape[-1]
    mu = np.sum(x64, axis=-1) / n
    var = np.sum((x64 - mu[..., None]) ** 2, axis=-1) / n
    eps64 = np.float64(eps) if exact else np.float64(np.float32(eps))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = 1.0 / np.sqrt(var + eps64)
    if exact:
        return mu, r
    return rne_f32(mu), rne_f32(r)


def normalize(x, mean, rstd, exact: bool = False):
    """xhat = fl(fl(x - mean) * rstd), mean and rstd broadcast over the last axis."""
    F = np.float64 if exact else np.float32
    with np.errstate(invalid="ignore", over="ignore"):
        return (np.asarray(x, F) - np.asarray(mean, F)[..., None]) * np.asarray(rstd, F)[..., None]


def affine(xhat, w, b, *, dtype: str, exact: bool = False):
    """y = RNE_T(fl(fl(xhat * w) + b)); b may be None (no bias). w, b broadcast against xhat."""
    F = np.float64 if exact else np.float32
    with np.errstate(invalid="ignore", over="ignore"):
        y = xhat * np.asarray(w, F)
        if b is not None:
            y = y + np.asarray(b, F)
    return y if exact else rne_to(y, dtype)


def layernorm_fwd(x, w, b=None, *, eps: float, dtype: str = "bf16", exact: bool = False):
    """LayerNorm over the last axis. Returns ``(y, mean, rstd)``; y holds T values (float32 array),
    mean and rstd are the float32 caches (float64 arrays if exact)."""
    _check(dtype)
    mean, rstd = row_stats(x, eps, exact)
    y = affine(normalize(x, mean, rstd, exact), w, b, dtype=dtype, exact=exact)
    return y, mean, rstd


def _bwd_rows(dy, x, w, mean, rstd, *, dtype: str, exact: bool):
    """dx of the row-wise normalization with per-element weights w (broadcast against x), and the
    per-element products dy * xhat whose sums make the weight gradient."""
    F = np.float64 if exact else np.float32
    x = np.asarray(x, F)
    dy = np.asarray(dy, F)
    r = np.asarray(rstd, F)[..., None]
    n = x.shape[-1]
    with np.errstate(invalid="ignore", over="ignore"):
        xhat = normalize(x, mean, rstd, exact)
        gdy = np.asarray(w, F) * dy
        c1 = np.sum(gdy.astype(np.float64), axis=-1) / n
        c2 = np.sum(gdy.astype(np.float64) * xhat.astype(np.float64), axis=-1) / n
        if not exact:
            c1, c2 = rne_f32(c1), rne_f32(c2)
        c1 = c1.astype(F)[..., None]
        c2 = c2.astype(F)[..., None]
        dx = r * ((gdy - c1) - xhat * c2)
    if not exact:
        dx = rne_to(dx, dtype)
    return dx, xhat


def layernorm_bwd(dy, x, w, mean, rstd, *, dtype: str = "bf16", exact: bool = False):
    """LayerNorm backward from the forward's caches. Returns ``(dx, dw, db)``: dx [M, N] (T values
    in float32), dw and db [N] float32 (float64 if exact)."""
    _check(dtype)
    dx, xhat = _bwd_rows(dy, x, w, mean, rstd, dtype=dtype, exact=exact)
    dy64 = np.asarray(dy, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        dw = np.sum(dy64 * xhat.astype(np.float64), axis=0)
        db = np.sum(dy64, axis=0)
    if not exact:
        dw, db = rne_f32(dw), rne_f32(db)
    return dx, dw, db


def _group_rows(x, G: int):
    """[B, C, S] -> [B, G, Cg * S]: the rows GroupNorm normalizes (groups of adjacent channels)."""
    x = np.asarray(x)
    B, C, S = x.shape
    if G < 1 or C % G:
        raise ValueError(f"C = {C} is not a multiple of the group count G = {G}")
    return x.reshape(B, G, (C // G) * S)


def _channel_rows(v, G: int, S: int):
    """Per-channel values [C] -> [G, Cg * S]: each channel's value repeated over its S elements."""
    v = np.asarray(v)
    C = v.shape[0]
    return np.repeat(v.reshape(G, C // G), S, axis=1)


def groupnorm_fwd(x, w, b=None, *, G: int, eps: float, dtype: str = "bf16",
                  exact: bool = False):
    """GroupNorm of x [B, C, S] with G groups and per-channel affine w, b [C] (b may be None).
    Returns ``(y [B, C, S], mean [B, G], rstd [B, G])``."""
    _check(dtype)
    B, C, S = np.shape(x)
    rows = _group_rows(x, G)
    mean, rstd = row_stats(rows, eps, exact)
    wr = _channel_rows(w, G, S)
    br = None if b is None else _channel_rows(b, G, S)
    y = affine(normalize(rows, mean, rstd, exact), wr, br, dtype=dtype, exact=exact)
    return y.reshape(B, C, S), mean, rstd


def groupnorm_bwd(dy, x, w, mean, rstd, *, G: int, dtype: str = "bf16", exact: bool = False):
    """GroupNorm backward from the forward's caches. Returns ``(dx [B, C, S], dw [C], db [C])``."""
    _check(dtype)
    B, C, S = np.shape(x)
    rows = _group_rows(x, G)
    drows = _group_rows(dy, G)
    dx, xhat = _bwd_rows(drows, rows, _channel_rows(w, G, S), mean, rstd, dtype=dtype,
                         exact=exact)
    dy64 = np.asarray(dy, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        dw = np.sum(dy64 * xhat.astype(np.float64).reshape(B, C, S), axis=(0, 2))
        db = np.sum(dy64, axis=(0, 2))
    if not exact:
        dw, db = rne_f32(dw), rne_f32(db)
    return dx.reshape(B, C, S), dw, db
