"""GPU parity on seeded random shapes: every entry point (RMSNorm in all three backward modes, its
FP8-output forward and its float64 entry points, LayerNorm with and without bias, softmax,
GroupNorm) against the CPU oracle on shapes drawn
log-uniformly, so that widths land on every kernel family (lane segments, one or more wavefronts a
row, register, LDS-staged and streaming rows, element-wise rows that are not 16-byte aligned) and
row counts are ragged against the blocks. Each case is small enough for the oracle to finish in
about a second; the draws are fixed by the seed below, and each case prints its shape before it
runs.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from test_gpu_groupnorm import BASE as GN_BASE, run_gn  # noqa: E402
from test_gpu_layernorm import run_ln  # noqa: E402
from test_gpu_parity import run_case  # noqa: E402
from test_gpu_fp8 import run_fp8  # noqa: E402
from test_gpu_softmax import run_f64, run_sm  # noqa: E402

MAX_ELEMS = 1_200_000
CASES = 40


def _rows(rng, N):
    """A log-uniform row count in [1, 3000], cut so that the case stays within MAX_ELEMS."""
    M = int(np.exp(rng.uniform(0.0, np.log(3000.0))))
    return max(1, min(M, MAX_ELEMS // N))


def _width(rng, lo=1.0, hi=24000.0):
    return int(np.exp(rng.uniform(np.log(lo), np.log(hi))))


def _stride(rng, N):
    """None (contiguous rows) or a padded row stride of N + 1 .. N + 16 elements."""
    return None if rng.uniform() < 0.6 else N + int(rng.integers(1, 17))


def _rms_cases():
    rng = np.random.default_rng(20260101)
    out = []
    for i in range(CASES):
        N = _width(rng)
        M = _rows(rng, N)
        dtype = ["bf16", "f16", "f32"][int(rng.integers(3))]
        mode = ["twice", "once", "autograd"][int(rng.integers(3))]
        offset = float(rng.integers(2)) if mode == "once" else 0.0
        out.append((i, dtype, M, N, _stride(rng, N), mode, offset))
    return out


def _ln_cases():
    rng = np.random.default_rng(20260102)
    out = []
    for i in range(CASES):
        N = _width(rng, 3.0)  # two-value rows cancel dx to rounding noise: a test of their own
        M = _rows(rng, N)
        out.append((i, ["bf16", "f16", "f32"][int(rng.integers(3))], M, N, _stride(rng, N),
                    bool(rng.integers(2))))
    return out


def _sm_cases():
    rng = np.random.default_rng(20260103)
    out = []
    for i in range(CASES):
        N = _width(rng)
        M = _rows(rng, N)
        out.append((i, ["bf16", "f16", "f32", "f64"][int(rng.integers(4))], M, N,
                    _stride(rng, N)))
    return out


def _gn_cases():
    rng = np.random.default_rng(20260104)
    out = []
    for i in range(CASES):
        G = int(rng.choice([1, 2, 3, 4, 8, 32]))
        Cg = int(np.exp(rng.uniform(0.0, np.log(40.0))))
        S = _width(rng, 1.0, 20000.0)
        B = int(rng.integers(1, 5))
        C = G * Cg
        B = max(1, min(B, MAX_ELEMS // (C * S)))
        if B * C * S > MAX_ELEMS:  # a single batch too large: fewer channels a group
            Cg = max(1, MAX_ELEMS // (G * S))
            C = G * Cg
        out.append((i, ["bf16", "f16", "f32"][int(rng.integers(3))], B, C, S, G,
                    bool(rng.integers(2))))
    return out


def _fp8_cases():
    rng = np.random.default_rng(20260105)
    out = []
    for i in range(CASES // 2):
        N = _width(rng)
        out.append((i, ["bf16", "f16", "f32"][int(rng.integers(3))], _rows(rng, N), N,
                    ["e4m3", "e5m2"][int(rng.integers(2))], float(2.0 ** rng.integers(-4, 5)),
                    float(rng.integers(2))))
    return out


def _f64_cases():
    rng = np.random.default_rng(20260106)
    out = []
    for i in range(CASES // 2):
        N = _width(rng)
        out.append((i, _rows(rng, N), N, _stride(rng, N), float(rng.integers(2))))
    return out


@pytest.mark.parametrize("i,dtype,M,N,ld,mode,offset", _rms_cases())
def test_sweep_rmsnorm(i, dtype, M, N, ld, mode, offset):
    if mode == "autograd":
        run_case(dtype, M, N, rounding="twice", ld=ld, casts="autograd", seed=100 + i)
    else:
        run_case(dtype, M, N, rounding=mode, offset=offset, ld=ld, seed=100 + i)


@pytest.mark.parametrize("i,dtype,M,N,ld,bias", _ln_cases())
def test_sweep_layernorm(i, dtype, M, N, ld, bias):
    run_ln(dtype, M, N, ld=ld, bias=bias, seed=200 + i)


@pytest.mark.parametrize("i,dtype,M,N,ld", _sm_cases())
def test_sweep_softmax(i, dtype, M, N, ld):
    run_sm(dtype, M, N, seed=300 + i, ld=ld)


@pytest.mark.parametrize("i,dtype,B,C,S,G,bias", _gn_cases())
def test_sweep_groupnorm(i, dtype, B, C, S, G, bias):
    run_gn(GN_BASE[dtype], B=B, C=C, S=S, G=G, seed=400 + i, bias=bias)


@pytest.mark.parametrize("i,dtype,M,N,fmt,scale,offset", _fp8_cases())
def test_sweep_fp8_forward(i, dtype, M, N, fmt, scale, offset):
    run_fp8(dtype, M, N, fmt=fmt, scale=scale, offset=offset, seed=500 + i)


@pytest.mark.parametrize("i,M,N,ld,offset", _f64_cases())
def test_sweep_rmsnorm_f64(i, M, N, ld, offset):
    run_f64(M, N, seed=600 + i, offset=offset, ld=ld)
