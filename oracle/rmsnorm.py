"""Plain CPU RMSNorm forward and backward with the rounding conventions spelled out.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle (see ``oracle/__init__.py``).

Sources (pages, by title):

* "Den dolda avrundningen i RMSNorm" (precisit.com blog post):
  section "En välbekant operation" gives the operation: each element divided by the root of the
  mean of the squares plus a small epsilon under the root, then multiplied by a learned gain;
  section "Två ställen att avrunda" gives the two places the result can be rounded to the 16-bit
  type: once (gain product in float32, one cast at the store) or twice (the normalized value is
  cast first, then the product is cast again); section "Vilken konvention hör till modellen?"
  ties the first to Gemma (which also uses ``1 + gamma`` as the gain) and the second to Llama;
  footnote 6 states the comparison assumes weights stored in the input dtype.
* "feat: correct casts in RMSNorm to match references" (Liger-Kernel pull request 92): forward and
  backward upcast to float32, the per-row inverse RMS is cached in float32 for the backward and the
  weight gradient is kept in float32.
* "fix(group_norm): keep the backward statistics and reductions in fp32" (Liger-Kernel pull
  request 1608), Summary: the backward upcasts weight, input and upstream gradient on load and
  reduces in float32; statistics are stored in float32.
* "Add backward passes to the fused rms_norm, layer_norm and softmax_last_dim ops" (candle pull
  request 4059): the RMSNorm backward is the derivative of the composed formula, with float32
  statistics for the 16-bit types.

Precision model. ``fl(.)`` below is one IEEE float32 operation with round-to-nearest-even; NumPy's
float32 elementwise arithmetic is exactly that. Row and column sums are taken in float64 (the GPU
is free to pick its own fp32 summation order; the comparison tolerances absorb that freedom) and
then rounded once to float32. ``RNE_T`` is round-to-nearest-even to the I/O dtype T, from
``oracle.rounding``.

Forward, per row r (gain ``g_j = fl(offset + w_j)``, so offset 0 is Llama's gain, offset 1 Gemma's):

    rstd_r = RNE_f32( 1 / sqrt( (sum_j x_rj^2) / N + eps ) )      (sum and root in float64)
    xhat   = fl(x * rstd)                                            (normalized value formed first)
    twice:  y = RNE_T( fl( RNE_T(xhat) * g ) )
    once:   y = RNE_T( fl( xhat * g ) )

For T = float32 every RNE_T is the identity and the two conventions coincide.

Backward (one reading, documented as such: the whole backward runs in float32 on upcast inputs with
the one cast at the store of dx, the same in both rounding conventions; the pages do not print the
per-convention casts of a backward):

    xhat = fl(x * rstd)            with rstd read from the forward's float32 cache
    gdy  = fl(g * dy)
    c_r  = RNE_f32( (sum_j gdy_rj * xhat_rj) / N )                   (sum in float64)
    dx   = RNE_T( fl( rstd * fl( gdy - fl(xhat * c) ) ) )
    dw_j = RNE_f32( sum_r dy_rj * xhat_rj )                           (sum in float64, output fp32)

This is the exact derivative of y = x * r(x) * g with r = (mean(x^2) + eps)^(-1/2):
dL/dx_i = r * (g_i dy_i - xhat_i * mean_j(g_j dy_j xhat_j)) and dL/dw_j = sum_rows dy_j xhat_j.

Second backward (``casts="autograd"``; only differs for round twice with a 16-bit T): the casts an
autograd engine makes when it differentiates the round-twice forward computed in T, as the Liger
pull request describes for matching the references. The forward multiplies the gain by the
T-rounded xhat in T, so the gradient reaching xhat is the T product of the upstream gradient and the
gain, and the gain's gradient multiplies the upstream gradient by the T-rounded xhat:

    gdy  = RNE_T( fl(g * dy) )
    dw_j = RNE_f32( sum_r dy_rj * RNE_T(xhat_rj) )
    c and dx as above (the normalization itself runs in float32).

``exact=True`` evaluates the same formulas entirely in float64 with no rounding to T or float32; it
is the real-number function, used for finite-difference and closed-form checks.
"""
from __future__ import annotations

import numpy as np

from .rounding import rne_f32, rne_fp8, rne_to

DTYPES = ("f32", "f16", "bf16")
ROUNDINGS = ("once", "twice")
CASTS = ("float32", "autograd")


def _check(dtype: str, rounding: str) -> None:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    if rounding not in ROUNDINGS:
        raise ValueError(f"rounding must be one of {ROUNDINGS}, got {rounding!r}")


def gain(w, offset: float, exact: bool = False) -> np.ndarray:
    """g_j = fl(offset + w_j): the multiplier applied after normalization (offset 1 = Gemma style)."""
    if exact:
        return np.float64(offset) + np.asarray(w, np.float64)
    return np.float32(offset) + np.asarray(w, np.float32)


def apply_gain(xhat, g, *, rounding: str, dtype: str, exact: bool = False) -> np.ndarray:
    """The store step of the forward: the two rounding conventions.

    round twice: RNE_T(fl(RNE_T(xhat) * g)); round once: RNE_T(fl(xhat * g)).
    ("Den dolda avrundningen i RMSNorm", section "Två ställen att avrunda".)
    """
    _check(dtype, rounding)
    if exact:
        return np.asarray(xhat, np.float64) * np.asarray(g, np.float64)
    xhat = np.asarray(xhat, np.float32)
    g = np.asarray(g, np.float32)
    if rounding == "twice":
        return rne_to(rne_to(xhat, dtype) * g, dtype)
    return rne_to(xhat * g, dtype)


def rstd_of(x, eps: float, exact: bool = False) -> np.ndarray:
    """Per-row 1/sqrt(mean(x^2) + eps), epsilon inside the root, in float64, rounded to float32.

    ``eps`` is taken at its float32 value, the value that crosses the C interface.
    ("Den dolda avrundningen i RMSNorm", section "En välbekant operation".)
    """
    x64 = np.asarray(x, np.float64)
    n = x64.shape[-1]
    ms = np.sum(x64 * x64, axis=-1) / n
    eps64 = np.float64(np.float32(eps))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = 1.0 / np.sqrt(ms + eps64)
    return r if exact else rne_f32(r)


def rmsnorm_fwd(x, w, *, eps: float, offset: float = 0.0, rounding: str = "twice",
                dtype: str = "bf16", exact: bool = False):
    """Forward of RMSNorm over the rows of ``x`` ([M, N], values already representable in T).

    Returns ``(y, rstd)``: ``y`` [M, N] (float32 array holding T values, or float64 if exact) and
    the per-row ``rstd`` [M] cache (float32, or float64 if exact).
    """
    _check(dtype, rounding)
    x = np.asarray(x)
    rstd = rstd_of(x, eps, exact)
    F = np.float64 if exact else np.float32
    with np.errstate(invalid="ignore", over="ignore"):
        xhat = np.asarray(x, F) * np.asarray(rstd, F)[..., None]
        y = apply_gain(xhat, gain(w, offset, exact), rounding=rounding, dtype=dtype, exact=exact)
    return y, rstd


def _autograd_casts(casts: str, rounding: str, dtype: str, exact: bool) -> bool:
    if casts not in CASTS:
        raise ValueError(f"casts must be one of {CASTS}, got {casts!r}")
    _check(dtype, rounding)
    return casts == "autograd" and rounding == "twice" and dtype != "f32" and not exact


def rmsnorm_fwd_fp8(x, w, *, eps: float, scale: float, fmt: str = "e4m3", offset: float = 0.0,
                    dtype: str = "bf16"):
    """Forward with an 8-bit float output: normalization, gain and the per-tensor output scale all
    in float32, then one cast to the OCP 8-bit format (the blog post "Den dolda avrundningen i
    RMSNorm", section "Var implementationerna skiljer sig" and its footnote 3, on Transformer
    Engine's FP8 output path):

        y8 = RNE_fmt( fl( fl(xhat * g) * scale ) )

    Returns ``(y8, rstd)`` with ``y8`` a float32 array holding 8-bit values (NaN where e4m3
    overflows, +-inf where e5m2 does).
    """
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}, got {dtype!r}")
    x = np.asarray(x)
    rstd = rstd_of(x, eps)
    with np.errstate(invalid="ignore", over="ignore"):
        xhat = np.asarray(x, np.float32) * rstd[..., None]
        yg = xhat * gain(w, offset)
        y8 = rne_fp8(yg * np.float32(scale), fmt)
    return y8, rstd


def rmsnorm_bwd(dy, x, w, rstd, *, offset: float = 0.0, dtype: str = "bf16", exact: bool = False,
                rounding: str = "twice", casts: str = "float32"):
    """Backward of RMSNorm given the forward's per-row ``rstd`` cache.

    Returns ``(dx, dw)``: ``dx`` [M, N] (float32 holding T values, or float64 if exact) and
    ``dw`` [N] (float32, or float64 if exact). With ``casts="float32"`` it does not depend on the
    forward's rounding convention; ``casts="autograd"`` reproduces the casts of differentiating the
    round-twice forward in T (see the module docstring).
    """
    ag = _autograd_casts(casts, rounding, dtype, exact)
    F = np.float64 if exact else np.float32
    x = np.asarray(x, F)
    dy = np.asarray(dy, F)
    r = np.asarray(rstd, F)[..., None]
    n = x.shape[-1]
    with np.errstate(invalid="ignore", over="ignore"):
        xhat = x * r
        gdy = gain(w, offset, exact).astype(F) * dy
        if ag:
            gdy = rne_to(gdy, dtype)
        c = np.sum(gdy.astype(np.float64) * xhat.astype(np.float64), axis=-1) / n
        c = (c if exact else rne_f32(c))[..., None]
        dx = r * (gdy - xhat * c)
        xw = rne_to(xhat, dtype) if ag else xhat
        dw = np.sum(dy.astype(np.float64) * xw.astype(np.float64), axis=0)
    if exact:
        return dx, dw
    return rne_to(dx, dtype), rne_f32(dw)


def rmsnorm_dw(dy, x, rstd, *, dtype: str = "bf16", rounding: str = "twice",
               casts: str = "float32") -> np.ndarray:
    """Only the weight gradient of ``rmsnorm_bwd``: dw_j = RNE_f32(sum_r dy_rj * fl(x_rj * rstd_r))
    (with RNE_T applied to the normalized value for the autograd casts).

    The same formula as the backward's dw (the tests hold the two equal bit for bit); it skips the
    input gradient so that full-size matrices stay cheap to check.
    """
    ag = _autograd_casts(casts, rounding, dtype, False)
    xhat = np.asarray(x, np.float32) * np.asarray(rstd, np.float32)[..., None]
    if ag:
        xhat = rne_to(xhat, dtype)
    dw = np.sum(np.asarray(dy, np.float32).astype(np.float64) * xhat.astype(np.float64), axis=0)
    return rne_f32(dw)
