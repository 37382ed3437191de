"""Seeded synthetic inputs for the RMSNorm forward/backward workloads.

This module holds no RMSNorm arithmetic: it only names the workloads (shape, dtype, convention,
epsilon, value distributions) and draws their inputs. Both the GPU library's tests/benchmark and
the CPU oracle's tests take their inputs from here; it imports neither of them.

Recipe (the same for every workload): ``numpy.random.default_rng(seed)`` draws x, then w, then dy
(in that order; an all-ones tensor draws nothing) as float64, which are cast to float32 and then
rounded to the I/O dtype with an independent library conversion (torch's CPU bfloat16 cast, NumPy's
float16 cast). Both sides therefore receive the same already-rounded values, as the blog post
"Den dolda avrundningen i RMSNorm" (section "Ge testet samma precision som modellen") recommends
for comparing implementations.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("f32", "f16", "bf16", "f64")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" | "f16" | "bf16": dtype of x, w, y, dy, dx
    M: int              # rows
    N: int              # row width (hidden size)
    rounding: str       # "once" | "twice"
    offset: float       # gain = offset + w
    eps: float
    x_dist: tuple       # ("normal", mean, std) | ("uniform", lo, hi) | ("ones",)
    w_dist: tuple
    dy_dist: tuple
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def itemsize(self) -> int:
        return {"f32": 4, "f64": 8}.get(self.dtype, 2)

    def fwd_bytes(self) -> int:
        """Algorithmic bytes of one forward: read x, write y, read w once, write the fp32 rstd."""
        s = self.itemsize
        return 2 * self.M * self.N * s + self.N * s + 4 * self.M

    def bwd_bytes(self) -> int:
        """Algorithmic bytes of one backward: read dy and x, write dx, read w and rstd, write dw."""
        s = self.itemsize
        return 3 * self.M * self.N * s + self.N * s + 4 * self.M + 4 * self.N


_STD = ("normal", 0.0, 1.0)
_GAIN = ("uniform", 0.9, 1.1)

WORKLOADS = {
    # fp32 I/O, tiny: the two conventions coincide; checked against the oracle in full.
    "fp32_64x1024": Workload("fp32_64x1024", "f32", 64, 1024, "twice", 0.0, 1e-6,
                             _STD, _GAIN, _STD, 0),
    # bf16 I/O, Llama-style (round twice), the headline measurement.
    "bf16_4096x4096": Workload("bf16_4096x4096", "bf16", 4096, 4096, "twice", 0.0, 1e-6,
                               _STD, _GAIN, _STD, 0),
    # fp16 I/O with x ~ N(0, 8^2): the sum of squares of a row overflows binary16.
    "fp16_8192x8192": Workload("fp16_8192x8192", "f16", 8192, 8192, "twice", 0.0, 1e-5,
                               ("normal", 0.0, 8.0), _GAIN, ("ones",), 0),
    # bf16 Gemma-style: round once with gain 1 + w, w ~ N(0, 0.1) read as variance 0.1.
    "bf16_16384x3072_gemma": Workload("bf16_16384x3072_gemma", "bf16", 16384, 3072, "once", 1.0,
                                      1e-6, _STD, ("normal", 0.0, math.sqrt(0.1)), _STD, 0),
}
# Hidden-size sweep at M = 4096, bf16, round twice.
for _n in (1024, 2048, 4096, 8192, 16384, 32768):
    WORKLOADS[f"bf16_sweep_4096x{_n}"] = Workload(f"bf16_sweep_4096x{_n}", "bf16", 4096, _n, "twice",
                                                  0.0, 1e-6, _STD, _GAIN, _STD, 0)
HEADLINE = "bf16_4096x4096"


def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape)
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "ones":
        return np.ones(shape, dtype=np.float64)
    raise ValueError(f"unknown distribution {dist!r}")


def to_dtype_values(a, dtype: str) -> np.ndarray:
    """float32 array holding the values of ``a`` converted to ``dtype`` by a library cast
    (float64 array, the values as drawn, for "f64")."""
    if dtype == "f64":
        return np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if dtype == "f32":
        return a32
    if dtype == "f16":
        return a32.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(a32).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(wl: Workload, M: int | None = None, N: int | None = None,
                seed: int | None = None) -> dict:
    """Draw ``x`` [M, N], ``w`` [N], ``dy`` [M, N] for a workload (float32 arrays of T values).

    ``M``, ``N`` and ``seed`` override the workload's own, for smaller parity cases that keep the
    workload's distributions.
    """
    M = wl.M if M is None else M
    N = wl.N if N is None else N
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = _draw(rng, wl.x_dist, (M, N))
    w = _draw(rng, wl.w_dist, (N,))
    dy = _draw(rng, wl.dy_dist, (M, N))
    return {
        "x": to_dtype_values(x, wl.dtype),
        "w": to_dtype_values(w, wl.dtype),
        "dy": to_dtype_values(dy, wl.dtype),
    }


def make_device_inputs(wl: Workload, device: str, seed: int | None = None) -> dict:
    """Timing inputs drawn on the device: ``x`` [M, N], ``w`` [N], ``dy`` [M, N] as tensors of
    dtype T, with the workload's distributions (float32 draws from torch's device generator, seeded,
    x then w then dy, then cast to T). The values differ from make_inputs' (another generator);
    they serve benchmarks of large shapes, where drawing on the host takes minutes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)

    def draw(dist, shape):
        kind = dist[0]
        if kind == "normal":
            t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            return t.mul_(dist[2]).add_(dist[1])
        if kind == "uniform":
            t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
            return t.mul_(dist[2] - dist[1]).add_(dist[1])
        if kind == "ones":
            return torch.ones(shape, device=device, dtype=torch.float32)
        raise ValueError(f"unknown distribution {dist!r}")

    td = torch_dtype(wl.dtype)
    x = draw(wl.x_dist, (wl.M, wl.N)).to(td)
    w = draw(wl.w_dist, (wl.N,)).to(td)
    dy = draw(wl.dy_dist, (wl.M, wl.N)).to(td)
    return {"x": x, "w": w, "dy": dy}


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "f64": torch.float64}[dtype]


def to_device(a: np.ndarray, dtype: str, device: str):
    """Copy an array of T values (float32, or float64 for "f64") to a ``device`` tensor of dtype T
    (exact conversion)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch_dtype(dtype)).to(device)


# ---- LayerNorm / GroupNorm inputs -----------------------------------------------------------------
# Same recipe; the bias is drawn after x, w and dy (so x, w and dy equal the RMSNorm workload's),
# as b ~ N(0, 0.1^2). ``x_dist`` overrides the workload's, e.g. ("normal", 16.0, 1.0) for rows whose
# mean is large against their spread (the group_norm page's test cases with an input offset).
_BIAS = ("normal", 0.0, 0.1)


def make_norm_inputs(wl: Workload, M: int | None = None, N: int | None = None,
                     seed: int | None = None, x_dist: tuple | None = None,
                     b_dist: tuple = _BIAS) -> dict:
    """Draw ``x`` [M, N], ``w`` [N], ``dy`` [M, N], then ``b`` [N] (float32 arrays of T values)."""
    M = wl.M if M is None else M
    N = wl.N if N is None else N
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = _draw(rng, x_dist or wl.x_dist, (M, N))
    w = _draw(rng, wl.w_dist, (N,))
    dy = _draw(rng, wl.dy_dist, (M, N))
    b = _draw(rng, b_dist, (N,))
    return {
        "x": to_dtype_values(x, wl.dtype),
        "w": to_dtype_values(w, wl.dtype),
        "dy": to_dtype_values(dy, wl.dtype),
        "b": to_dtype_values(b, wl.dtype),
    }


# LayerNorm at the RMSNorm headline shape: bf16 4096 x 4096, eps 1e-5 (the usual LayerNorm eps).
LN_WORKLOADS = {
    "ln_bf16_4096x4096": Workload("ln_bf16_4096x4096", "bf16", 4096, 4096, "once", 0.0, 1e-5,
                                  _STD, _GAIN, _STD, 0),
    "ln_fp32_64x1024": Workload("ln_fp32_64x1024", "f32", 64, 1024, "once", 0.0, 1e-5,
                                _STD, _GAIN, _STD, 0),
    "ln_fp16_8192x8192": Workload("ln_fp16_8192x8192", "f16", 8192, 8192, "once", 0.0, 1e-5,
                                  ("normal", 0.0, 8.0), _GAIN, ("ones",), 0),
}


# GroupNorm: x [B, C, S] (S the flattened spatial size), G groups. Shapes from the group_norm
# page's Details table (Liger-Kernel pull request 1608, its backward timings and accuracy cases).
@dataclasses.dataclass(frozen=True)
class GnWorkload:
    name: str
    dtype: str
    B: int
    C: int
    S: int
    G: int
    eps: float
    x_dist: tuple
    w_dist: tuple
    dy_dist: tuple
    b_dist: tuple = _BIAS
    seed: int = 0

    def with_(self, **kw) -> "GnWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def numel(self) -> int:
        return self.B * self.C * self.S

    def fwd_bytes(self) -> int:
        """Read x, write y, read w and b, write the float32 mean and rstd."""
        s = self.itemsize
        return 2 * self.numel * s + 2 * self.C * s + 8 * self.B * self.G

    def bwd_bytes(self) -> int:
        """Read dy and x, write dx, read w, mean and rstd, write the float32 dw and db."""
        s = self.itemsize
        return 3 * self.numel * s + self.C * s + 8 * self.B * self.G + 8 * self.C


GN_WORKLOADS = {
    w.name: w for w in [
        GnWorkload("gn_bf16_1x16x256x256_g4", "bf16", 1, 16, 256 * 256, 4, 1e-5, _STD, _GAIN,
                   _STD),
        GnWorkload("gn_bf16_16x32x256x256_g8", "bf16", 16, 32, 256 * 256, 8, 1e-5, _STD, _GAIN,
                   _STD),
        GnWorkload("gn_bf16_16x512x64x64_g32", "bf16", 16, 512, 64 * 64, 32, 1e-5, _STD, _GAIN,
                   _STD),
        GnWorkload("gn_bf16_64x64x8192_g8", "bf16", 64, 64, 8192, 8, 1e-5, _STD, _GAIN, _STD),
        # many channels of a small spatial size (20 channels of 32 x 32 a group): 20480-element
        # (batch, group) rows
        GnWorkload("gn_bf16_8x640x32x32_g32", "bf16", 8, 640, 32 * 32, 32, 1e-5, _STD, _GAIN,
                   _STD),
        GnWorkload("gn_f16_1x16x256x256_g4_ones", "f16", 1, 16, 256 * 256, 4, 1e-5, _STD,
                   ("ones",), ("ones",), ("normal", 0.0, 0.0)),
        GnWorkload("gn_bf16_2x64x32x32_g8_offset16", "bf16", 2, 64, 32 * 32, 8, 1e-5,
                   ("normal", 16.0, 1.0), _GAIN, _STD),
        GnWorkload("gn_f32_2x8x16_g4", "f32", 2, 8, 16, 4, 1e-5, _STD, _GAIN, _STD),
    ]
}
GN_HEADLINE = "gn_bf16_16x32x256x256_g8"


def make_gn_inputs(wl: GnWorkload, B: int | None = None, C: int | None = None,
                   S: int | None = None, seed: int | None = None) -> dict:
    """Draw ``x`` [B, C, S], ``w`` [C], ``dy`` [B, C, S], then ``b`` [C] (T values in float32)."""
    B = wl.B if B is None else B
    C = wl.C if C is None else C
    S = wl.S if S is None else S
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = _draw(rng, wl.x_dist, (B, C, S))
    w = _draw(rng, wl.w_dist, (C,))
    dy = _draw(rng, wl.dy_dist, (B, C, S))
    b = _draw(rng, wl.b_dist, (C,))
    return {k: to_dtype_values(v, wl.dtype) for k, v in (("x", x), ("w", w), ("dy", dy), ("b", b))}


# Softmax over the last dimension: logits x ~ N(0, 2^2) (a spread that gives peaked rows), dy ~
# N(0, 1), at the RMSNorm headline shape; and the float64 RMSNorm at the same shape.
SM_WORKLOADS = {
    "sm_bf16_4096x4096": Workload("sm_bf16_4096x4096", "bf16", 4096, 4096, "once", 0.0, 0.0,
                                  ("normal", 0.0, 2.0), _GAIN, _STD, 0),
    "sm_f32_64x1024": Workload("sm_f32_64x1024", "f32", 64, 1024, "once", 0.0, 0.0,
                               ("normal", 0.0, 2.0), _GAIN, _STD, 0),
    "sm_f16_4096x4096": Workload("sm_f16_4096x4096", "f16", 4096, 4096, "once", 0.0, 0.0,
                                 ("normal", 0.0, 2.0), _GAIN, _STD, 0),
    "sm_f64_1024x4096": Workload("sm_f64_1024x4096", "f64", 1024, 4096, "once", 0.0, 0.0,
                                 ("normal", 0.0, 2.0), _GAIN, _STD, 0),
}
F64_WORKLOADS = {
    "f64_4096x4096": Workload("f64_4096x4096", "f64", 4096, 4096, "once", 0.0, 1e-6, _STD, _GAIN,
                              _STD, 0),
}
