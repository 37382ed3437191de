"""RMSNorm forward/backward on AMD Instinct MI355X (gfx950): Python binding of ``librmsnorm``.

The binding only marshals arguments: it checks tensor shapes, dtypes, devices and strides, allocates
outputs with torch (device memory and streams are all torch provides here) and calls the C
interface in ``librmsnorm.so`` on torch's current stream. Every step of the computation runs in the
library's HIP kernels; there is no fallback. If the library has not been built the first call
raises ``LibraryMissing`` (build it with ``python -m bwd_precision_numerics_amd.build``).

    y, rstd = fwd(x, w, eps=1e-6, offset=0.0, rounding="twice")
    dx, dw  = bwd(dy, x, w, rstd, offset=0.0)
    y       = rms_norm(x, w, eps, offset, rounding)        # autograd-aware
    y8, rstd = fwd_fp8(x, w, scale=1.0, fmt="e4m3")        # OCP 8-bit output
    y, mean, rstd = layernorm_fwd(x, w, b, eps=1e-5)       # LayerNorm (b may be None)
    dx, dw, db    = layernorm_bwd(dy, x, w, mean, rstd, bias=True)
    y, mean, rstd = groupnorm_fwd(x, G, w, b, eps=1e-5)    # GroupNorm of [B, C, *spatial]
    dx, dw, db    = groupnorm_bwd(dy, x, G, w, mean, rstd)
    y = softmax_fwd(x); dx = softmax_bwd(dy, y)             # softmax over the last dimension
    layer_norm(x, w, b), group_norm(x, G, w, b), softmax(x) # autograd-aware versions
    y, rstd = fwd_f64(x64, w64); dx, dw = bwd_f64(dy64, x64, w64, rstd)   # float64 RMSNorm

``rounding="twice"`` is the Llama convention T(float(T(xhat)) * g); ``"once"`` is the Gemma
convention T(xhat * g); the gain is ``g = offset + w`` (offset 1 for Gemma).
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librmsnorm.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "librmsnorm.h")
HEADER_PATHS = [HEADER_PATH] + [os.path.join(os.path.dirname(HERE), "include", f)
                               for f in ("libnorms.h", "libsoftmax.h")]

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
ROUNDING_CODES = {"once": 0, "twice": 1}
BWD_AUTOGRAD_CASTS = 0x10  # flag OR-ed into the backward's rounding argument
CASTS = ("float32", "autograd")
VARIANT_CODES = {"auto": 0, "registers": 1, "lds": 2, "streaming": 3}
FP8_CODES = {"e4m3": 0, "e5m2": 1}
PROBE_CODES = {"read": 0, "write": 1, "copy": 2, "sum2": 3, "launch": 4}
PROBE_CACHED_STORES = 0x100  # OR-ed into a probe kind: plain stores instead of non-temporal
STATUS_NAMES = {0: "OK", 1: "ERR_INVALID_ARG", 2: "ERR_UNSUPPORTED", 3: "ERR_MISALIGNED",
                4: "ERR_WORKSPACE", 5: "ERR_HIP"}


class LibraryMissing(RuntimeError):
    """librmsnorm.so is not built (or cannot be loaded)."""


class RMSNormError(RuntimeError):
    """A librmsnorm call returned a non-OK status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({message})")
        self.status = status


_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_f = ctypes.c_float
_i = ctypes.c_int
_sz = ctypes.c_size_t
_d = ctypes.c_double
SIGNATURES = {
    "rmsnorm_fwd": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i, _f, _f, _i, _p]),
    "rmsnorm_fwd_variant": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i, _f, _f, _i, _i, _p]),
    "rmsnorm_fwd_fp8": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i, _f, _f, _f, _i, _i,
                             _p]),
    "rmsnorm_bwd_workspace_bytes": (_sz, [_i64, _i64, _i]),
    "rmsnorm_bwd": (_i, [_p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _p, _sz, _i64, _i64, _i, _f,
                         _f, _i, _p]),
    "rmsnorm_bwd_variant": (_i, [_p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _p, _sz, _i64, _i64,
                                 _i, _f, _f, _i, _i, _p]),
    "rmsnorm_bwd_noalloc": (_i, [_p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _i64, _i64, _i, _f,
                                 _f, _i, _p]),
    "rmsnorm_bwd_rows": (_i, [_p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _sz, _i64, _i64, _i, _f,
                              _i, _i, _p]),
    "rmsnorm_bwd_dw_reduce": (_i, [_p, _sz, _p, _i64, _i64, _i, _p]),
    "layernorm_fwd": (_i, [_p, _i64, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i, _f, _i, _p]),
    "layernorm_bwd_workspace_bytes": (_sz, [_i64, _i64, _i]),
    "layernorm_bwd": (_i, [_p, _i64, _p, _i64, _p, _p, _p, _p, _i64, _p, _p, _p, _sz, _i64, _i64,
                           _i, _i, _p]),
    "groupnorm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i]),
    "groupnorm_fwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _sz, _i64, _i64, _i64, _i64, _i, _f, _p]),
    "groupnorm_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _i64, _i64, _i64, _i64, _i,
                           _p]),
    "softmax_fwd": (_i, [_p, _i64, _p, _i64, _i64, _i64, _i, _i, _p]),
    "softmax_bwd": (_i, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i, _i, _p]),
    "rmsnorm_fwd_f64": (_i, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _d, _d, _p]),
    "rmsnorm_bwd_f64_workspace_bytes": (_sz, [_i64, _i64]),
    "rmsnorm_bwd_f64": (_i, [_p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _p, _sz, _i64, _i64, _d,
                             _p]),
    "rmsnorm_bandwidth_probe_out_bytes": (_sz, [_sz]),
    "rmsnorm_bandwidth_probe": (_i, [_i, _p, _p, _p, _sz, _p]),
    "rmsnorm_status_string": (ctypes.c_char_p, [_i]),
    "rmsnorm_abi_version": (_i, []),
}


def header_text(paths=None) -> str:
    """The C headers' text without comments."""
    text = "\n".join(open(p, encoding="utf-8").read() for p in (paths or HEADER_PATHS))
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def header_functions(paths=None) -> list:
    """Names of the functions the C headers declare."""
    return sorted(set(re.findall(r"\b((?:rmsnorm|layernorm|groupnorm|softmax)_[a-z_0-9]+)\s*\(",
                                 header_text(paths))))


def library(path: str | None = None) -> ctypes.CDLL:
    """Load librmsnorm.so once and declare its signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LibraryMissing(f"{p} is not built; run `python -m bwd_precision_numerics_amd.build`")
    try:
        lib = ctypes.CDLL(p)
    except OSError as e:
        raise LibraryMissing(f"cannot load {p}: {e}") from e
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = library().rmsnorm_status_string(status).decode()
        raise RMSNormError(fn, status, msg)


# ---- tensor plumbing --------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_name(t) -> str:
    torch = _torch()
    m = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return m[t.dtype]


def _rows(t, name: str):
    """Check a 2-D device tensor with unit column stride and rows that do not overlap; return
    (ptr, row stride). A broadcast view (row stride 0) or any row stride below N is refused: the
    kernels address M rows of N elements at the row stride."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, N], got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along the last dimension")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} has overlapping rows (row stride {t.stride(0)} < {t.shape[1]}); "
                         "pass a contiguous copy")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return t.data_ptr(), ld


def _vec(t, name: str, n: int):
    if t.dim() != 1 or t.shape[0] != n:
        raise ValueError(f"{name} must be 1-D of length {n}, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if n > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _same_device(*ts):
    dev = ts[0].device
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def workspace_bytes(M: int, N: int, dtype: str) -> int:
    return int(library().rmsnorm_bwd_workspace_bytes(M, N, DTYPE_CODES[dtype]))


def fwd(x, w, eps: float = 1e-6, offset: float = 0.0, rounding: str = "twice",
        variant: str = "auto", y=None, rstd=None, want_rstd: bool = True):
    """RMSNorm forward. Returns ``(y, rstd)`` (``rstd`` is None when ``want_rstd`` is False)."""
    torch = _torch()
    dt = dtype_name(x)
    if w.dtype != x.dtype:
        raise TypeError("w must have the dtype of x")
    M, N = x.shape
    px, ldx = _rows(x, "x")
    pw = _vec(w, "w", N)
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if y.dtype != x.dtype or tuple(y.shape) != (M, N):
        raise ValueError("y must match x in shape and dtype")
    py, ldy = _rows(y, "y")
    if want_rstd and rstd is None:
        rstd = torch.empty((M,), dtype=torch.float32, device=x.device)
    prs = None
    if rstd is not None:
        if rstd.dtype != torch.float32:
            raise TypeError("rstd must be float32")
        prs = _vec(rstd, "rstd", M)
        _same_device(x, rstd)
    _same_device(x, w, y)
    st = library().rmsnorm_fwd_variant(px, ldx, pw, py, ldy, prs, M, N, DTYPE_CODES[dt], eps,
                                       offset, ROUNDING_CODES[rounding], VARIANT_CODES[variant],
                                       _stream(x.device))
    _check("rmsnorm_fwd", st)
    return y, rstd


def fp8_torch_dtype(fmt: str):
    torch = _torch()
    return {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]


def fwd_fp8(x, w, eps: float = 1e-6, offset: float = 0.0, scale: float = 1.0,
            fmt: str = "e4m3", variant: str = "auto", y=None, rstd=None, want_rstd: bool = True):
    """RMSNorm forward with an 8-bit output ``FP8(fl(xhat * g) * scale)``.

    Returns ``(y8, rstd)``; y8 is ``torch.float8_e4m3fn`` or ``torch.float8_e5m2`` (or the
    caller's ``y``, which may also be uint8). ``rstd`` equals the one ``fwd`` writes.
    """
    torch = _torch()
    dt = dtype_name(x)
    if fmt not in FP8_CODES:
        raise ValueError(f"fmt must be one of {sorted(FP8_CODES)}")
    if w.dtype != x.dtype:
        raise TypeError("w must have the dtype of x")
    M, N = x.shape
    px, ldx = _rows(x, "x")
    pw = _vec(w, "w", N)
    if y is None:
        y = torch.empty((M, N), dtype=fp8_torch_dtype(fmt), device=x.device)
    if y.dtype not in (fp8_torch_dtype(fmt), torch.uint8) or tuple(y.shape) != (M, N):
        raise ValueError(f"y must be [M, N] of {fp8_torch_dtype(fmt)} or uint8")
    py, ldy = _rows(y, "y")
    if want_rstd and rstd is None:
        rstd = torch.empty((M,), dtype=torch.float32, device=x.device)
    prs = None
    if rstd is not None:
        if rstd.dtype != torch.float32:
            raise TypeError("rstd must be float32")
        prs = _vec(rstd, "rstd", M)
        _same_device(x, rstd)
    _same_device(x, w, y)
    st = library().rmsnorm_fwd_fp8(px, ldx, pw, py, ldy, prs, M, N, DTYPE_CODES[dt], eps, offset,
                                   scale, FP8_CODES[fmt], VARIANT_CODES[variant],
                                   _stream(x.device))
    _check("rmsnorm_fwd_fp8", st)
    return y, rstd


def _bwd_common(dy, x, w, rstd, dx):
    torch = _torch()
    dt = dtype_name(x)
    if dy.dtype != x.dtype or w.dtype != x.dtype:
        raise TypeError("dy and w must have the dtype of x")
    if tuple(dy.shape) != tuple(x.shape):
        raise ValueError("dy must have the shape of x")
    if rstd is None or rstd.dtype != torch.float32:
        raise TypeError("rstd (float32, from fwd) is required")
    M, N = x.shape
    if dx is None:
        dx = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if dx.dtype != x.dtype or tuple(dx.shape) != (M, N):
        raise ValueError("dx must match x in shape and dtype")
    _same_device(dy, x, w, rstd, dx)
    return dt, M, N, dx


def _ws_buffer(t, device, name: str = "workspace"):
    """Pointer and byte size of a caller-provided workspace. It must be a contiguous GPU tensor on
    the inputs' device; the size reported to the library is the tensor's extent, bounded by what
    its storage holds from the tensor's first byte (so a view cannot claim memory it does not own).
    The library checks that size against what the call needs."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    nbytes = t.numel() * t.element_size()
    avail = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    return t.data_ptr(), max(0, min(nbytes, avail))


def _workspace(M, N, dt, device, workspace):
    torch = _torch()
    need = workspace_bytes(M, N, dt)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=device)
    return _ws_buffer(workspace, device)


def bwd_rounding_code(rounding: str, casts: str) -> int:
    """The backward's rounding argument: the convention, plus the autograd-casts flag."""
    if casts not in CASTS:
        raise ValueError(f"casts must be one of {CASTS}, got {casts!r}")
    return ROUNDING_CODES[rounding] | (BWD_AUTOGRAD_CASTS if casts == "autograd" else 0)


def bwd(dy, x, w, rstd, eps: float = 1e-6, offset: float = 0.0, rounding: str = "twice",
        variant: str = "auto", dx=None, dw=None, workspace=None, casts: str = "float32"):
    """RMSNorm backward. Returns ``(dx, dw)``; ``dw`` is float32.

    ``casts="autograd"`` reproduces the casts of differentiating the round-twice forward in T
    (no effect for round once or float32); the default is the float32 backward."""
    torch = _torch()
    dt, M, N, dx = _bwd_common(dy, x, w, rstd, dx)
    if dw is None:
        dw = torch.empty((N,), dtype=torch.float32, device=x.device)
    if dw.dtype != torch.float32:
        raise TypeError("dw must be float32")
    pdy, lddy = _rows(dy, "dy")
    px, ldx = _rows(x, "x")
    pdx, lddx = _rows(dx, "dx")
    pws, wsb = _workspace(M, N, dt, x.device, workspace)
    _same_device(x, dw)
    st = library().rmsnorm_bwd_variant(pdy, lddy, px, ldx, _vec(w, "w", N), _vec(rstd, "rstd", M),
                                       pdx, lddx, _vec(dw, "dw", N), pws, wsb, M,
                                       N, DTYPE_CODES[dt], eps, offset,
                                       bwd_rounding_code(rounding, casts),
                                       VARIANT_CODES[variant], _stream(x.device))
    _check("rmsnorm_bwd", st)
    return dx, dw


def bwd_rows(dy, x, w, rstd, workspace, offset: float = 0.0, variant: str = "auto", dx=None,
             rounding: str = "twice", casts: str = "float32"):
    """First backward stage: dx and the per-block dw partials (in ``workspace``)."""
    dt, M, N, dx = _bwd_common(dy, x, w, rstd, dx)
    pdy, lddy = _rows(dy, "dy")
    px, ldx = _rows(x, "x")
    pdx, lddx = _rows(dx, "dx")
    pws, wsb = _ws_buffer(workspace, x.device)
    st = library().rmsnorm_bwd_rows(pdy, lddy, px, ldx, _vec(w, "w", N), _vec(rstd, "rstd", M),
                                    pdx, lddx, pws, wsb, M, N, DTYPE_CODES[dt],
                                    offset, bwd_rounding_code(rounding, casts),
                                    VARIANT_CODES[variant], _stream(x.device))
    _check("rmsnorm_bwd_rows", st)
    return dx


def dw_reduce(workspace, dw, M: int, N: int, dtype: str):
    """Second backward stage: dw = fixed-order sum of the partials in ``workspace``."""
    if dw.dtype != _torch().float32:
        raise TypeError("dw must be float32")
    if dtype not in DTYPE_CODES:
        raise ValueError(f"dtype must be one of {sorted(DTYPE_CODES)}")
    pdw = _vec(dw, "dw", N)
    pws, wsb = _ws_buffer(workspace, dw.device)
    st = library().rmsnorm_bwd_dw_reduce(pws, wsb, pdw, M, N,
                                         DTYPE_CODES[dtype], _stream(dw.device))
    _check("rmsnorm_bwd_dw_reduce", st)
    return dw


# ---- LayerNorm --------------------------------------------------------------------------------------

def layernorm_workspace_bytes(M: int, N: int, dtype: str) -> int:
    return int(library().layernorm_bwd_workspace_bytes(M, N, DTYPE_CODES[dtype]))


def _opt_vec(t, name, n, dtype):
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}")
    return _vec(t, name, n)


def layernorm_fwd(x, w, b=None, eps: float = 1e-5, variant: str = "auto", y=None, mean=None,
                  rstd=None, want_stats: bool = True):
    """LayerNorm over the last dimension of a 2-D ``x``. Returns ``(y, mean, rstd)`` (the float32
    caches are None when ``want_stats`` is False)."""
    torch = _torch()
    dt = dtype_name(x)
    M, N = x.shape
    px, ldx = _rows(x, "x")
    pw = _opt_vec(w, "w", N, x.dtype)
    pb = _opt_vec(b, "b", N, x.dtype)
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if y.dtype != x.dtype or tuple(y.shape) != (M, N):
        raise ValueError("y must match x in shape and dtype")
    py, ldy = _rows(y, "y")
    if want_stats:
        mean = torch.empty((M,), dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty((M,), dtype=torch.float32, device=x.device) if rstd is None else rstd
    pm = _opt_vec(mean, "mean", M, torch.float32)
    pr = _opt_vec(rstd, "rstd", M, torch.float32)
    _same_device(*[t for t in (x, w, b, y, mean, rstd) if t is not None])
    st = library().layernorm_fwd(px, ldx, pw, pb, py, ldy, pm, pr, M, N, DTYPE_CODES[dt], eps,
                                 VARIANT_CODES[variant], _stream(x.device))
    _check("layernorm_fwd", st)
    return y, mean, rstd


def layernorm_bwd(dy, x, w, mean, rstd, bias: bool = True, variant: str = "auto", dx=None,
                  dw=None, db=None, workspace=None):
    """LayerNorm backward. Returns ``(dx, dw, db)``; dw, db float32 (db None if not ``bias``)."""
    torch = _torch()
    dt = dtype_name(x)
    if dy.dtype != x.dtype or w.dtype != x.dtype:
        raise TypeError("dy and w must have the dtype of x")
    if tuple(dy.shape) != tuple(x.shape):
        raise ValueError("dy must have the shape of x")
    M, N = x.shape
    if dx is None:
        dx = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if dx.dtype != x.dtype or tuple(dx.shape) != (M, N):
        raise ValueError("dx must match x in shape and dtype")
    if dw is None:
        dw = torch.empty((N,), dtype=torch.float32, device=x.device)
    if bias and db is None:
        db = torch.empty((N,), dtype=torch.float32, device=x.device)
    pdy, lddy = _rows(dy, "dy")
    px, ldx = _rows(x, "x")
    pdx, lddx = _rows(dx, "dx")
    need = layernorm_workspace_bytes(M, N, dt)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=x.device)
    pws, wsb = _ws_buffer(workspace, x.device)
    _same_device(*[t for t in (dy, x, w, mean, rstd, dx, dw, db, workspace) if t is not None])
    st = library().layernorm_bwd(pdy, lddy, px, ldx, _vec(w, "w", N),
                                 _opt_vec(mean, "mean", M, torch.float32),
                                 _opt_vec(rstd, "rstd", M, torch.float32), pdx, lddx,
                                 _opt_vec(dw, "dw", N, torch.float32),
                                 _opt_vec(db, "db", N, torch.float32) if bias else None,
                                 pws, wsb, M, N, DTYPE_CODES[dt],
                                 VARIANT_CODES[variant], _stream(x.device))
    _check("layernorm_bwd", st)
    return dx, dw, (db if bias else None)


# ---- GroupNorm --------------------------------------------------------------------------------------

def groupnorm_workspace_bytes(B: int, C: int, S: int, G: int, dtype: str) -> int:
    return int(library().groupnorm_workspace_bytes(B, C, S, G, DTYPE_CODES[dtype]))


def _contig(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _gn_shape(x):
    if x.dim() < 2:
        raise ValueError("x must be [B, C, *spatial]")
    B, C = x.shape[0], x.shape[1]
    S = 1
    for d in x.shape[2:]:
        S *= d
    return B, C, S


def _gn_workspace(B, C, S, G, dt, device, workspace):
    torch = _torch()
    need = groupnorm_workspace_bytes(B, C, S, G, dt)
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 3) // 4, dtype=torch.float32, device=device)
    pws, wsb = _ws_buffer(workspace, device)
    return workspace, pws, wsb


def groupnorm_fwd(x, G: int, w, b=None, eps: float = 1e-5, y=None, mean=None, rstd=None,
                  workspace=None):
    """GroupNorm of a contiguous ``x`` [B, C, *spatial] with G groups. Returns ``(y, mean, rstd)``
    (mean and rstd float32 [B, G])."""
    torch = _torch()
    dt = dtype_name(x)
    B, C, S = _gn_shape(x)
    px = _contig(x, "x")
    pw = _opt_vec(w, "w", C, x.dtype)
    pb = _opt_vec(b, "b", C, x.dtype)
    if y is None:
        y = torch.empty_like(x)
    if y.dtype != x.dtype or y.shape != x.shape:
        raise ValueError("y must match x in shape and dtype")
    mean = torch.empty((B, G), dtype=torch.float32, device=x.device) if mean is None else mean
    rstd = torch.empty((B, G), dtype=torch.float32, device=x.device) if rstd is None else rstd
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t.dtype != torch.float32 or t.numel() != B * G:
            raise ValueError(f"{n} must be float32 with B * G elements")
    workspace, pws, wsb = _gn_workspace(B, C, S, G, dt, x.device, workspace)
    _same_device(*[t for t in (x, w, b, y, mean, rstd, workspace) if t is not None])
    st = library().groupnorm_fwd(px, pw, pb, _contig(y, "y"), _contig(mean, "mean"),
                                 _contig(rstd, "rstd"), pws, wsb, B, C, S, G,
                                 DTYPE_CODES[dt], eps, _stream(x.device))
    _check("groupnorm_fwd", st)
    return y, mean, rstd


def groupnorm_bwd(dy, x, G: int, w, mean, rstd, bias: bool = True, dx=None, dw=None, db=None,
                  workspace=None):
    """GroupNorm backward. Returns ``(dx, dw, db)``; dw, db float32 [C] (db None if not ``bias``)."""
    torch = _torch()
    dt = dtype_name(x)
    if dy.dtype != x.dtype or w.dtype != x.dtype:
        raise TypeError("dy and w must have the dtype of x")
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    B, C, S = _gn_shape(x)
    if dx is None:
        dx = torch.empty_like(x)
    if dx.dtype != x.dtype or dx.shape != x.shape:
        raise ValueError("dx must match x in shape and dtype")
    for t, n in ((mean, "mean"), (rstd, "rstd")):
        if t.dtype != torch.float32 or t.numel() != B * G:
            raise ValueError(f"{n} must be float32 with B * G elements")
    if dw is None:
        dw = torch.empty((C,), dtype=torch.float32, device=x.device)
    if bias and db is None:
        db = torch.empty((C,), dtype=torch.float32, device=x.device)
    workspace, pws, wsb = _gn_workspace(B, C, S, G, dt, x.device, workspace)
    _same_device(*[t for t in (dy, x, w, mean, rstd, dx, dw, db, workspace) if t is not None])
    st = library().groupnorm_bwd(_contig(dy, "dy"), _contig(x, "x"), _vec(w, "w", C),
                                 _contig(mean, "mean"), _contig(rstd, "rstd"), _contig(dx, "dx"),
                                 _opt_vec(dw, "dw", C, torch.float32),
                                 _opt_vec(db, "db", C, torch.float32) if bias else None,
                                 pws, wsb, B, C, S, G, DTYPE_CODES[dt],
                                 _stream(x.device))
    _check("groupnorm_bwd", st)
    return dx, dw, (db if bias else None)


# ---- softmax and float64 RMSNorm -------------------------------------------------------------------

def _any_dtype_name(t) -> str:
    """dtype name for the entry points that also take float64."""
    torch = _torch()
    return "f64" if t.dtype == torch.float64 else dtype_name(t)


def softmax_fwd(x, variant: str = "auto", y=None):
    """Softmax over the last dimension of a 2-D ``x`` (float32 / float16 / bfloat16 / float64)."""
    torch = _torch()
    dt = _any_dtype_name(x)
    M, N = x.shape
    px, ldx = _rows(x, "x")
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if y.dtype != x.dtype or tuple(y.shape) != (M, N):
        raise ValueError("y must match x in shape and dtype")
    py, ldy = _rows(y, "y")
    _same_device(x, y)
    st = library().softmax_fwd(px, ldx, py, ldy, M, N, DTYPE_CODES[dt], VARIANT_CODES[variant],
                               _stream(x.device))
    _check("softmax_fwd", st)
    return y


def softmax_bwd(dy, y, variant: str = "auto", dx=None):
    """dx = y * (dy - sum(dy * y)) over the last dimension, from the forward's output ``y``."""
    torch = _torch()
    dt = _any_dtype_name(y)
    if dy.dtype != y.dtype or dy.shape != y.shape:
        raise ValueError("dy must match y in shape and dtype")
    M, N = y.shape
    if dx is None:
        dx = torch.empty((M, N), dtype=y.dtype, device=y.device)
    if dx.dtype != y.dtype or tuple(dx.shape) != (M, N):
        raise ValueError("dx must match y in shape and dtype")
    pdy, lddy = _rows(dy, "dy")
    py, ldy = _rows(y, "y")
    pdx, lddx = _rows(dx, "dx")
    _same_device(dy, y, dx)
    st = library().softmax_bwd(pdy, lddy, py, ldy, pdx, lddx, M, N, DTYPE_CODES[dt],
                               VARIANT_CODES[variant], _stream(y.device))
    _check("softmax_bwd", st)
    return dx


def fwd_f64(x, w, eps: float = 1e-6, offset: float = 0.0, y=None, rstd=None):
    """RMSNorm with float64 I/O and float64 statistics. Returns ``(y, rstd)`` (rstd float64)."""
    torch = _torch()
    if x.dtype != torch.float64 or w.dtype != torch.float64:
        raise TypeError("x and w must be float64")
    M, N = x.shape
    y = torch.empty_like(x) if y is None else y
    if y.dtype != x.dtype or tuple(y.shape) != (M, N):
        raise ValueError("y must match x in shape and dtype")
    rstd = torch.empty((M,), dtype=torch.float64, device=x.device) if rstd is None else rstd
    if rstd.dtype != torch.float64:
        raise TypeError("rstd must be float64")
    px, ldx = _rows(x, "x")
    py, ldy = _rows(y, "y")
    _same_device(x, w, y, rstd)
    st = library().rmsnorm_fwd_f64(px, ldx, _vec(w, "w", N), py, ldy, _vec(rstd, "rstd", M), M,
                                   N, eps, offset, _stream(x.device))
    _check("rmsnorm_fwd_f64", st)
    return y, rstd


def bwd_f64(dy, x, w, rstd, offset: float = 0.0, dx=None, dw=None, workspace=None):
    """Backward of ``fwd_f64``. Returns ``(dx, dw)``, both float64."""
    torch = _torch()
    if x.dtype != torch.float64 or dy.dtype != torch.float64 or w.dtype != torch.float64:
        raise TypeError("dy, x and w must be float64")
    if tuple(dy.shape) != tuple(x.shape):
        raise ValueError("dy must have the shape of x")
    M, N = x.shape
    dx = torch.empty_like(x) if dx is None else dx
    if dx.dtype != x.dtype or tuple(dx.shape) != (M, N):
        raise ValueError("dx must match x in shape and dtype")
    if rstd.dtype != torch.float64 or dw is not None and dw.dtype != torch.float64:
        raise TypeError("rstd and dw must be float64")
    dw = torch.empty((N,), dtype=torch.float64, device=x.device) if dw is None else dw
    need = int(library().rmsnorm_bwd_f64_workspace_bytes(M, N))
    if workspace is None:
        workspace = torch.empty((max(need, 16) + 7) // 8, dtype=torch.float64, device=x.device)
    pws, wsb = _ws_buffer(workspace, x.device)
    pdy, lddy = _rows(dy, "dy")
    px, ldx = _rows(x, "x")
    pdx, lddx = _rows(dx, "dx")
    _same_device(dy, x, w, rstd, dx, dw, workspace)
    st = library().rmsnorm_bwd_f64(pdy, lddy, px, ldx, _vec(w, "w", N), _vec(rstd, "rstd", M), pdx,
                                   lddx, _vec(dw, "dw", N), pws, wsb, M, N, offset,
                                   _stream(x.device))
    _check("rmsnorm_bwd_f64", st)
    return dx, dw


def _as_rows(t, n: int):
    """``t`` as a 2-D [rows, n] view the kernels can address (unit column stride, rows that do not
    overlap), copying only when it is not: gradients often arrive as broadcast views."""
    t2 = t.reshape(-1, n)
    if (n > 1 and t2.stride(-1) != 1) or (t2.shape[0] > 1 and t2.stride(0) < n):
        t2 = t2.contiguous()
    return t2


def _make_autograd():
    torch = _torch()

    class RMSNormFunction(torch.autograd.Function):
        """y = RMSNorm(x) * (offset + w) over the last dimension; backward through librmsnorm."""

        @staticmethod
        def forward(ctx, x, w, eps, offset, rounding, casts):
            shape = x.shape
            x2 = _as_rows(x, shape[-1])
            y, rstd = fwd(x2, w, eps=eps, offset=offset, rounding=rounding)
            ctx.save_for_backward(x2, w, rstd)
            ctx.cfg = (eps, offset, rounding, shape, casts)
            return y.reshape(shape)

        @staticmethod
        def backward(ctx, gy):
            x2, w, rstd = ctx.saved_tensors
            eps, offset, rounding, shape, casts = ctx.cfg
            gy2 = _as_rows(gy, shape[-1])
            dx, dw = bwd(gy2, x2, w, rstd, eps=eps, offset=offset, rounding=rounding, casts=casts)
            return dx.reshape(shape), dw.to(w.dtype), None, None, None, None

    return RMSNormFunction


_autograd_fn = None


def rms_norm(x, w, eps: float = 1e-6, offset: float = 0.0, rounding: str = "twice",
             casts: str = "float32"):
    """Autograd-aware RMSNorm over the last dimension of ``x``."""
    global _autograd_fn
    if _autograd_fn is None:
        _autograd_fn = _make_autograd()
    return _autograd_fn.apply(x, w, eps, offset, rounding, casts)


def _make_autograd_widened():
    torch = _torch()

    class LayerNormFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, w, b, eps):
            shape = x.shape
            x2 = _as_rows(x, shape[-1])
            y, mean, rstd = layernorm_fwd(x2, w, b, eps=eps)
            ctx.save_for_backward(x2, w, mean, rstd)
            ctx.cfg = (shape, b is not None)
            return y.reshape(shape)

        @staticmethod
        def backward(ctx, gy):
            x2, w, mean, rstd = ctx.saved_tensors
            shape, has_b = ctx.cfg
            dx, dw, db = layernorm_bwd(_as_rows(gy, shape[-1]), x2, w, mean, rstd, bias=has_b)
            return (dx.reshape(shape), dw.to(w.dtype), db.to(w.dtype) if has_b else None,
                    None)

    class GroupNormFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, G, w, b, eps):
            xc = x.contiguous()
            y, mean, rstd = groupnorm_fwd(xc, G, w, b, eps=eps)
            ctx.save_for_backward(xc, w, mean, rstd)
            ctx.cfg = (G, b is not None)
            return y

        @staticmethod
        def backward(ctx, gy):
            xc, w, mean, rstd = ctx.saved_tensors
            G, has_b = ctx.cfg
            dx, dw, db = groupnorm_bwd(gy.contiguous(), xc, G, w, mean, rstd, bias=has_b)
            return dx, None, dw.to(w.dtype), db.to(w.dtype) if has_b else None, None

    class SoftmaxFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x):
            shape = x.shape
            y = softmax_fwd(_as_rows(x, shape[-1]))
            ctx.save_for_backward(y)
            ctx.shape = shape
            return y.reshape(shape)

        @staticmethod
        def backward(ctx, gy):
            (y,) = ctx.saved_tensors
            return softmax_bwd(_as_rows(gy, ctx.shape[-1]), y).reshape(ctx.shape)

    return LayerNormFunction, GroupNormFunction, SoftmaxFunction


_widened = None


def _widened_fns():
    global _widened
    if _widened is None:
        _widened = _make_autograd_widened()
    return _widened


def layer_norm(x, w, b=None, eps: float = 1e-5):
    """Autograd-aware LayerNorm over the last dimension of ``x`` (weight required, bias optional);
    the gradients of w and b come back in w's dtype (computed in float32)."""
    return _widened_fns()[0].apply(x, w, b, eps)


def group_norm(x, G: int, w, b=None, eps: float = 1e-5):
    """Autograd-aware GroupNorm of ``x`` [B, C, *spatial] with G groups."""
    return _widened_fns()[1].apply(x, G, w, b, eps)


def softmax(x):
    """Autograd-aware softmax over the last dimension of ``x``."""
    return _widened_fns()[2].apply(x)
