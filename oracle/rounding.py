"""Round-to-nearest-even onto the bfloat16, binary16 and OCP 8-bit grids, written from the IEEE 754
definition.

TEST INFRASTRUCTURE ONLY: part of the CPU oracle (see ``oracle/__init__.py``).

Each format of the path is a binary floating-point format described by three numbers:
the significand precision ``p`` (hidden bit included), the smallest normal exponent ``emin`` and the
largest exponent ``emax``. Rounding a real value ``v`` to such a format with ties-to-even means:

* find the spacing of the format's grid at ``v``: ``2**(E - p + 1)`` where ``E`` is the exponent of
  the leading bit of ``v``, clamped below at ``emin`` (values under the normal range share the
  subnormal spacing ``2**(emin - p + 1)``);
* take the nearest multiple of that spacing, and on an exact tie the multiple whose quotient is even;
* if the result's magnitude exceeds the largest finite value ``(2 - 2**(1-p)) * 2**emax`` the
  result is an infinity of the same sign (IEEE overflow under round-to-nearest).

NaN stays NaN, infinities and signed zeros are kept.

The bfloat16 blog post ("Den dolda avrundningen i RMSNorm", precisit.com, section "En skillnad du
kan återskapa") rounds with an integer trick on the float32 bit pattern that only covers finite
inputs; this module instead rounds from the definition above, in float64 arithmetic that is exact
for every float32 input, so NaN, infinity, overflow and subnormal results are covered too. The
tests pin it to the values that post prints and to the conversions of independent libraries.
"""
from __future__ import annotations

import numpy as np

# (significand bits incl. hidden bit, smallest normal exponent, largest exponent)
FORMATS = {
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
    "f32": (24, -126, 127),
    # OCP 8-bit formats. e5m2 follows the IEEE pattern (infinities at the top exponent). e4m3 has no
    # infinities: its top exponent holds normal values except the all-ones code, which is NaN, so
    # the largest finite value is 1.75 * 2^8 = 448 and anything that rounds beyond it is NaN.
    "e4m3": (4, -6, 8),
    "e5m2": (3, -14, 15),
}
# Largest finite value and what overflow becomes, where they differ from the IEEE pattern.
_MAX_FINITE = {"e4m3": 448.0}
_OVERFLOW_NAN = {"e4m3"}


def round_to_format(v, fmt: str) -> np.ndarray:
    """Round each element of ``v`` (float32 or float64 input) to the nearest value of ``fmt``.

    Ties go to the even neighbour. Returns a float32 array whose values are exactly representable
    in ``fmt`` (NaN, +-Inf and +-0 included). ``fmt`` is one of "bf16", "f16", "f32", "e4m3",
    "e5m2".
    For "f32" the input is expected in float64 and the result is the correctly rounded float32.
    """
    p, emin, emax = FORMATS[fmt]
    a = np.asarray(v, dtype=np.float64)
    out = np.array(a, dtype=np.float64, copy=True)
    finite = np.isfinite(a) & (a != 0.0)
    if np.any(finite):
        af = a[finite]
        # frexp: af = m * 2**e with 0.5 <= |m| < 1, so the leading bit has exponent e - 1.
        _, e = np.frexp(af)
        lead = np.maximum(e.astype(np.int64) - 1, emin)
        spacing = np.ldexp(1.0, lead - (p - 1))
        # af / spacing is exact (power-of-two scaling in float64); rint rounds half to even.
        q = np.rint(af / spacing) * spacing
        big = _MAX_FINITE.get(fmt, (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax)
        over = np.nan if fmt in _OVERFLOW_NAN else np.inf
        q = np.where(np.abs(q) > big, np.copysign(over, af), q)
        out[finite] = q
    if fmt in _OVERFLOW_NAN:
        out[np.isinf(a)] = np.nan
    return out.astype(np.float32)


def rne_bf16(v) -> np.ndarray:
    """Round to bfloat16 (8-bit significand, float32 exponent range); result held in float32."""
    return round_to_format(v, "bf16")


def rne_f16(v) -> np.ndarray:
    """Round to IEEE binary16 (11-bit significand, subnormals down to 2**-24, overflow to Inf)."""
    return round_to_format(v, "f16")


def rne_f32(v) -> np.ndarray:
    """Round float64 values to float32 (nearest, ties to even)."""
    return round_to_format(v, "f32")


def rne_fp8(v, fmt: str) -> np.ndarray:
    """Round to an OCP 8-bit float format ("e4m3" or "e5m2"): nearest, ties to even; beyond the
    largest finite value e5m2 gives an infinity and e4m3 (which has none) gives NaN."""
    if fmt not in ("e4m3", "e5m2"):
        raise ValueError(f"unknown 8-bit format {fmt!r}")
    return round_to_format(v, fmt)


def rne_to(v, dtype: str) -> np.ndarray:
    """Round to the I/O dtype of the path: "bf16", "f16" or "f32" (identity for float32 input)."""
    if dtype == "f32":
        return np.asarray(v, dtype=np.float32)
    return round_to_format(v, dtype)


def ulp_of(v, dtype: str) -> np.ndarray:
    """Spacing of the ``dtype`` grid at |v| (the gap to the next value away from zero), float64."""
    p, emin, _ = FORMATS[dtype]
    a = np.abs(np.asarray(v, dtype=np.float64))
    safe = np.where(np.isfinite(a) & (a > 0), a, 1.0)
    _, e = np.frexp(safe)
    lead = np.maximum(e.astype(np.int64) - 1, emin)
    return np.ldexp(1.0, lead - (p - 1))
