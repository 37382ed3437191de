"""Pins for the oracle's RMSNorm forward and backward (CPU only).

Each pin ties the oracle to something other than itself: closed forms (unit RMS of the output at
gain 1 and epsilon 0; the x . dx identity), exact invariants (power-of-two scaling, N = 1),
identities between the two rounding conventions the blog post "Den dolda avrundningen i RMSNorm"
states (section "Två ställen att avrunda": the conventions coincide for float32 I/O), float64 central
finite differences of the forward, torch float64 autograd of the composed formula, and torch's CPU
RMSNorm for the round-once convention. A final test plants plausible mistakes in a copy of the
oracle and checks that the pins catch every one.
"""
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.rmsnorm as oracle_rmsnorm
from oracle import rne_bf16, rmsnorm_bwd, rmsnorm_fwd
from workloads import WORKLOADS, make_inputs, to_dtype_values

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed, dtype="f32", scale=1.0):
    rng = np.random.default_rng(seed)
    return to_dtype_values(rng.standard_normal(shape) * scale, dtype)


# --------------------------------------------------------------------------------------------
# Pin suite, parameterised by the oracle module so the mutation test can run it on planted bugs.
# --------------------------------------------------------------------------------------------

def pin_unit_rms(mod):
    """gain 1, offset 0, eps 0: every output row has RMS exactly 1 (float64) / within 2^-9 (bf16)."""
    x = _rand((6, 40), 11)
    w = np.ones(40, np.float32)
    y, _ = mod.rmsnorm_fwd(x, w, eps=0.0, dtype="f32", exact=True)
    rms = np.sqrt(np.mean(np.asarray(y, np.float64) ** 2, axis=1))
    assert np.allclose(rms, 1.0, rtol=1e-12, atol=0)
    xb = _rand((6, 40), 12, "bf16")
    for rounding in ("once", "twice"):
        yb, _ = mod.rmsnorm_fwd(xb, w, eps=0.0, dtype="bf16", rounding=rounding)
        rms = np.sqrt(np.mean(np.asarray(yb, np.float64) ** 2, axis=1))
        assert np.all(np.abs(rms - 1.0) <= 2.0**-9)


def pin_worked_example(mod):
    """Blog post "Den dolda avrundningen i RMSNorm", section "En skillnad du kan återskapa"."""
    g = rne_bf16(np.float32(1.05))
    assert float(mod.apply_gain(np.float32(1.1), g, rounding="once", dtype="bf16")) == 1.1484375
    assert float(mod.apply_gain(np.float32(1.1), g, rounding="twice", dtype="bf16")) == 1.15625


def _loss(mod, x, w, dy, eps, offset):
    y, _ = mod.rmsnorm_fwd(x, w, eps=eps, offset=offset, dtype="f32", exact=True)
    return float(np.sum(np.asarray(dy, np.float64) * y))


def pin_finite_differences(mod, M=3, N=8, eps=1e-6, offset=0.0, seed=0, h=1e-6):
    """Backward (float64) equals central differences of L = sum(dy * y) of the forward (float64)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, N))
    w = rng.uniform(0.5, 1.5, N)
    dy = rng.standard_normal((M, N))
    _, rstd = mod.rmsnorm_fwd(x, w, eps=eps, offset=offset, dtype="f32", exact=True)
    dx, dw = mod.rmsnorm_bwd(dy, x, w, rstd, offset=offset, dtype="f32", exact=True)
    fdx = np.zeros_like(x)
    for i in range(M):
        for j in range(N):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fdx[i, j] = (_loss(mod, xp, w, dy, eps, offset) - _loss(mod, xm, w, dy, eps, offset)) / (2 * h)
    fdw = np.zeros_like(w)
    for j in range(N):
        wp = w.copy(); wp[j] += h
        wm = w.copy(); wm[j] -= h
        fdw[j] = (_loss(mod, x, wp, dy, eps, offset) - _loss(mod, x, wm, dy, eps, offset)) / (2 * h)
    sx = max(np.max(np.abs(fdx)), 1.0)
    sw = max(np.max(np.abs(fdw)), 1.0)
    assert np.max(np.abs(dx - fdx)) <= 1e-6 * sx + 1e-8, (dx, fdx)
    assert np.max(np.abs(dw - fdw)) <= 1e-6 * sw + 1e-8, (dw, fdw)


def pin_x_dot_dx(mod, eps=0.0):
    """sum_j x_j dx_j = eps/(ms+eps) * sum_j g_j dy_j xhat_j per row (0 at eps = 0)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 33))
    w = rng.uniform(0.9, 1.1, 33)
    dy = rng.standard_normal((4, 33))
    _, rstd = mod.rmsnorm_fwd(x, w, eps=eps, dtype="f32", exact=True)
    dx, _ = mod.rmsnorm_bwd(dy, x, w, rstd, dtype="f32", exact=True)
    lhs = np.sum(x * dx, axis=1)
    ms = np.mean(x * x, axis=1)
    eps64 = float(np.float32(eps))
    xhat = x / np.sqrt(ms + eps64)[:, None]
    rhs = eps64 / (ms + eps64) * np.sum(w * dy * xhat, axis=1)
    scale = np.sum(np.abs(x * dx), axis=1) + np.abs(rhs)
    assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale + 1e-300)


def pin_gemma_identity(mod):
    """Gain 1 + w with w = 0 equals gain w = 1 with no offset (float32 path and float64 path)."""
    x = _rand((4, 64), 52, "bf16")
    for exact in (False, True):
        for rounding in ("once", "twice"):
            a, _ = mod.rmsnorm_fwd(x, np.zeros(64, np.float32), eps=1e-6, offset=1.0, dtype="bf16",
                                   rounding=rounding, exact=exact)
            b, _ = mod.rmsnorm_fwd(x, np.ones(64, np.float32), eps=1e-6, offset=0.0, dtype="bf16",
                                   rounding=rounding, exact=exact)
            assert np.array_equal(a, b)
    dy = _rand((4, 64), 53, "bf16")
    _, r = mod.rmsnorm_fwd(x, np.zeros(64, np.float32), eps=1e-6, offset=1.0)
    for exact in (False, True):
        a, _ = mod.rmsnorm_bwd(dy, x, np.zeros(64, np.float32), r, offset=1.0, exact=exact)
        b, _ = mod.rmsnorm_bwd(dy, x, np.ones(64, np.float32), r, offset=0.0, exact=exact)
        assert np.array_equal(a, b)


def _torch_llama_autograd(x, w, dy, eps, dtype):
    """torch autograd of the round-twice (Llama) graph computed in T: returns (dx, dw) as float32,
    plus dw recomputed with a float32 weight over the T-rounded normalized value."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    xt = torch.tensor(x, dtype=tdt, requires_grad=True)
    wt = torch.tensor(w, dtype=tdt, requires_grad=True)
    x32 = xt.float()
    xhat = x32 * torch.rsqrt(x32.pow(2).mean(-1, keepdim=True) + float(np.float32(eps)))
    h = xhat.to(tdt)
    (wt * h).backward(torch.tensor(dy, dtype=tdt))
    w32 = torch.tensor(w, dtype=torch.float32, requires_grad=True)
    (w32 * h.detach().float()).backward(torch.tensor(dy, dtype=torch.float32))
    return xt.grad.float().numpy(), w32.grad.numpy()


def pin_autograd_casts(mod, dtype="bf16"):
    """The autograd-cast backward reproduces torch's T autograd of the round-twice graph: dx on
    >= 99.9 % of elements and within one step of T elsewhere (the float32 backward matches only
    about three quarters; the remaining differences come from torch's own float32 order of the
    normalization's derivative), dw as the sum of dy * T(xhat) (a float32 weight gradient over the
    forward's rounded normalized value)."""
    inp = make_inputs(WORKLOADS["bf16_4096x4096"], M=96, N=512, seed=77)
    x, w, dy = (to_dtype_values(inp[k], dtype) for k in ("x", "w", "dy"))
    _, r = mod.rmsnorm_fwd(x, w, eps=1e-6, dtype=dtype)
    dxB, dwB = mod.rmsnorm_bwd(dy, x, w, r, dtype=dtype, rounding="twice", casts="autograd")
    dxA, dwA = mod.rmsnorm_bwd(dy, x, w, r, dtype=dtype, rounding="twice", casts="float32")
    dxT, dwT = _torch_llama_autograd(x, w, dy, 1e-6, dtype)
    assert np.mean(dxB == dxT) >= 0.999, np.mean(dxB == dxT)
    rms = np.sqrt(np.mean(dxT.astype(np.float64) ** 2, axis=1, keepdims=True))
    steps = np.abs(dxB.astype(np.float64) - dxT) / oracle.ulp_of(
        np.maximum(np.abs(dxT), 2.0**-12 * rms), dtype)
    assert steps.max() <= 1.0
    assert np.mean(dxA == dxT) < 0.95
    nrm = np.linalg.norm(dwT)
    assert np.linalg.norm(dwB - dwT) / nrm <= 1e-6
    assert np.linalg.norm(dwA - dwT) / nrm > 1e-4


PIN_SUITE = [
    pin_unit_rms,
    pin_autograd_casts,
    pin_gemma_identity,
    pin_worked_example,
    lambda m: pin_finite_differences(m, M=3, N=8, eps=0.1, offset=1.0),
    lambda m: pin_finite_differences(m, M=2, N=5, eps=0.0),
    lambda m: pin_x_dot_dx(m, eps=0.0),
    lambda m: pin_x_dot_dx(m, eps=0.05),
]


# --------------------------------------------------------------------------------------------
# The pins on the real oracle
# --------------------------------------------------------------------------------------------

def test_unit_rms_output():
    pin_unit_rms(oracle_rmsnorm)


def test_worked_example_through_forward_store_step():
    pin_worked_example(oracle_rmsnorm)


@pytest.mark.parametrize("N", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.1])
@pytest.mark.parametrize("offset", [0.0, 1.0])
def test_backward_matches_finite_differences(N, eps, offset):
    if N == 1 and eps == 0.0:
        pytest.skip("N=1, eps=0 is covered by test_single_column_rows (dx vanishes exactly)")
    pin_finite_differences(oracle_rmsnorm, M=min(4, 1 + N % 4), N=N, eps=eps, offset=offset, seed=N)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.1])
def test_x_dot_dx_closed_form(eps):
    pin_x_dot_dx(oracle_rmsnorm, eps)


def test_x_dot_dx_vanishes_in_float32_path():
    x = _rand((8, 512), 21, "bf16")
    w = to_dtype_values(np.random.default_rng(22).uniform(0.9, 1.1, 512), "bf16")
    dy = _rand((8, 512), 23, "bf16")
    _, rstd = rmsnorm_fwd(x, w, eps=0.0, dtype="bf16")
    dx, _ = rmsnorm_bwd(dy, x, w, rstd, dtype="f32")
    lhs = np.sum(x.astype(np.float64) * dx, axis=1)
    scale = np.sum(np.abs(x.astype(np.float64) * dx), axis=1)
    assert np.all(np.abs(lhs) <= 1e-5 * scale)


def test_matches_torch_float64_autograd_of_composed_formula():
    rng = np.random.default_rng(7)
    for (M, N, eps, offset) in [(3, 7, 1e-6, 0.0), (2, 16, 0.1, 1.0), (4, 1, 1e-3, 0.5)]:
        x = rng.standard_normal((M, N))
        w = rng.uniform(-1, 1, N)
        dy = rng.standard_normal((M, N))
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
        e = float(np.float32(eps))
        yt = xt * torch.rsqrt(xt.pow(2).mean(-1, keepdim=True) + e) * (offset + wt)
        (yt * torch.tensor(dy)).sum().backward()
        y, rstd = rmsnorm_fwd(x, w, eps=eps, offset=offset, dtype="f32", exact=True)
        dx, dw = rmsnorm_bwd(dy, x, w, rstd, offset=offset, dtype="f32", exact=True)
        assert np.allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-14)
        assert np.allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(dw, wt.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("rounding", ["once", "twice"])
def test_power_of_two_scaling_is_exact(dtype, rounding):
    """At eps = 0, y(2^k x) == y(x) and dx(2^k x) == 2^-k dx(x), bit for bit."""
    x = _rand((5, 96), 31, dtype)
    w = to_dtype_values(np.random.default_rng(32).uniform(0.9, 1.1, 96), dtype)
    dy = _rand((5, 96), 33, dtype)
    y0, r0 = rmsnorm_fwd(x, w, eps=0.0, dtype=dtype, rounding=rounding)
    dx0, dw0 = rmsnorm_bwd(dy, x, w, r0, dtype=dtype)
    for k in (-3, 4):
        xs = (x * np.float32(2.0**k)).astype(np.float32)
        y1, r1 = rmsnorm_fwd(xs, w, eps=0.0, dtype=dtype, rounding=rounding)
        dx1, dw1 = rmsnorm_bwd(dy, xs, w, r1, dtype=dtype)
        assert np.array_equal(y1, y0)
        assert np.array_equal(r1, (r0 * np.float32(2.0**-k)).astype(np.float32))
        assert np.array_equal(dx1, (dx0 * np.float32(2.0**-k)).astype(np.float32))
        assert np.array_equal(dw1, dw0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_column_rows(dtype):
    """N = 1, eps = 0: y = sign(x) * g and dx vanishes."""
    x = np.array([[3.0], [-0.5], [1e-3], [-7.0]], np.float32)
    w = np.array([1.25], np.float32)
    dy = np.array([[1.0], [2.0], [-3.0], [0.5]], np.float32)
    y, rstd = rmsnorm_fwd(x, w, eps=0.0, dtype=dtype, rounding="once")
    assert np.array_equal(y[:, 0], np.sign(x[:, 0]) * np.float32(1.25))
    _, rstd_e = rmsnorm_fwd(x, w, eps=0.0, dtype=dtype, exact=True)
    dx, _ = rmsnorm_bwd(dy, x, w, rstd_e, dtype=dtype, exact=True)
    assert np.all(np.abs(dx) <= 1e-12 * np.abs(rstd_e[:, None] * dy))
    dx32, _ = rmsnorm_bwd(dy, x, w, rstd, dtype="f32")
    assert np.all(np.abs(dx32) <= 1e-6 * np.abs(rstd[:, None] * dy * 1.25))


def test_conventions_coincide_for_float32_io():
    """Blog post, section "Två ställen att avrunda": with float32 I/O the inner cast does nothing."""
    inp = make_inputs(WORKLOADS["fp32_64x1024"])
    y1, _ = rmsnorm_fwd(inp["x"], inp["w"], eps=1e-6, dtype="f32", rounding="once")
    y2, _ = rmsnorm_fwd(inp["x"], inp["w"], eps=1e-6, dtype="f32", rounding="twice")
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_conventions_coincide_for_unit_gain(dtype):
    x = _rand((16, 256), 41, dtype)
    w = np.ones(256, np.float32)
    y1, _ = rmsnorm_fwd(x, w, eps=1e-6, dtype=dtype, rounding="once")
    y2, _ = rmsnorm_fwd(x, w, eps=1e-6, dtype=dtype, rounding="twice")
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_conventions_differ_for_general_gain(dtype):
    x = _rand((64, 512), 42, dtype)
    w = to_dtype_values(np.random.default_rng(43).uniform(0.9, 1.1, 512), dtype)
    y1, _ = rmsnorm_fwd(x, w, eps=1e-6, dtype=dtype, rounding="once")
    y2, _ = rmsnorm_fwd(x, w, eps=1e-6, dtype=dtype, rounding="twice")
    frac = np.mean(y1 != y2)
    assert 0.15 < frac < 0.35
    # every difference is one step on the dtype's grid
    d = np.abs(y1.astype(np.float64) - y2) / oracle.ulp_of(np.minimum(np.abs(y1), np.abs(y2)), dtype)
    assert np.all(d[y1 != y2] == 1.0)


def test_gemma_offset_identity():
    pin_gemma_identity(oracle_rmsnorm)


def test_round_once_agrees_with_torch_cpu_rms_norm_bf16():
    """torch's CPU RMSNorm multiplies in float32 and casts last for bf16 input (the blog post's
    footnote 2 states this for its tested inputs); the oracle's round-once convention must agree
    up to reduction-order differences in the statistic."""
    x = _rand((4096, 512), 61, "bf16")
    w = to_dtype_values(np.random.default_rng(62).uniform(0.9, 1.1, 512), "bf16")
    yo, _ = rmsnorm_fwd(x, w, eps=1e-6, dtype="bf16", rounding="once")
    xt = torch.from_numpy(x).to(torch.bfloat16)
    wt = torch.from_numpy(w).to(torch.bfloat16)
    yt = torch.nn.functional.rms_norm(xt, (512,), weight=wt, eps=1e-6).float().numpy()
    eq = np.mean(yo == yt)
    assert eq >= 0.9999, eq
    assert np.max(np.abs(yo.astype(np.float64) - yt) / oracle.ulp_of(yo, "bf16")) <= 1.0


def test_fp32_path_close_to_exact():
    inp = make_inputs(WORKLOADS["fp32_64x1024"])
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    y, r = rmsnorm_fwd(x, w, eps=1e-6, dtype="f32")
    ye, re = rmsnorm_fwd(x, w, eps=1e-6, dtype="f32", exact=True)
    assert np.max(np.abs(y - ye) / np.abs(ye)) <= 2.0**-22
    assert np.max(np.abs(r - re) / re) <= 2.0**-24
    dx, dw = rmsnorm_bwd(dy, x, w, r, dtype="f32")
    dxe, dwe = rmsnorm_bwd(dy, x, w, re, dtype="f32", exact=True)
    assert np.linalg.norm(dx - dxe) / np.linalg.norm(dxe) <= 1e-6
    assert np.linalg.norm(dw - dwe) / np.linalg.norm(dwe) <= 1e-6


def test_dw_is_additive_over_rows():
    inp = make_inputs(WORKLOADS["bf16_4096x4096"], M=64, N=256)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    _, r = rmsnorm_fwd(x, w, eps=1e-6)
    _, dw = rmsnorm_bwd(dy, x, w, r)
    _, dwa = rmsnorm_bwd(dy[:20], x[:20], w, r[:20])
    _, dwb = rmsnorm_bwd(dy[20:], x[20:], w, r[20:])
    assert np.allclose(dw, dwa.astype(np.float64) + dwb, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_autograd_casts_match_torch_autograd(dtype):
    pin_autograd_casts(oracle_rmsnorm, dtype)


def test_autograd_casts_identities():
    """The autograd casts change nothing for float32 I/O or round once, and dx is unchanged when
    g * dy is exact in T (unit gain)."""
    inp = make_inputs(WORKLOADS["bf16_4096x4096"], M=32, N=256, seed=78)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    _, r = rmsnorm_fwd(x, w, eps=1e-6)
    for kw in (dict(dtype="f32", rounding="twice"), dict(dtype="bf16", rounding="once")):
        a = rmsnorm_bwd(dy, x, w, r, casts="float32", **kw)
        b = rmsnorm_bwd(dy, x, w, r, casts="autograd", **kw)
        assert all(np.array_equal(p, q) for p, q in zip(a, b))
    ones = np.ones(256, np.float32)
    a, _ = rmsnorm_bwd(dy, x, ones, r, casts="float32")
    b, _ = rmsnorm_bwd(dy, x, ones, r, casts="autograd")
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        rmsnorm_bwd(dy, x, w, r, casts="fp64")


def test_dw_only_function_equals_backward_dw():
    for name in ("fp32_64x1024", "bf16_16384x3072_gemma", "fp16_8192x8192"):
        wl = WORKLOADS[name]
        inp = make_inputs(wl, M=48, N=200)
        _, r = rmsnorm_fwd(inp["x"], inp["w"], eps=wl.eps, offset=wl.offset, dtype=wl.dtype)
        _, dw = rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], r, offset=wl.offset, dtype=wl.dtype)
        assert np.array_equal(oracle.rmsnorm_dw(inp["dy"], inp["x"], r), dw)
    wl = WORKLOADS["bf16_4096x4096"]
    inp = make_inputs(wl, M=48, N=200)
    _, r = rmsnorm_fwd(inp["x"], inp["w"], eps=wl.eps)
    _, dw = rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], r, casts="autograd")
    assert np.array_equal(oracle.rmsnorm_dw(inp["dy"], inp["x"], r, casts="autograd"), dw)


def test_backward_independent_of_forward_convention_and_offset_derivative():
    """dw does not depend on the offset (d(offset + w)/dw = 1); dx does through the gain."""
    inp = make_inputs(WORKLOADS["bf16_16384x3072_gemma"], M=16, N=192)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    _, r = rmsnorm_fwd(x, w, eps=1e-6, offset=1.0, rounding="once")
    dx0, dw0 = rmsnorm_bwd(dy, x, w, r, offset=0.0)
    dx1, dw1 = rmsnorm_bwd(dy, x, w, r, offset=1.0)
    assert np.array_equal(dw0, dw1)
    assert not np.array_equal(dx0, dx1)


def test_fp16_sum_of_squares_overflows_but_oracle_stays_finite():
    """x ~ N(0, 8^2) with N = 8192: the running sum of squares leaves the binary16 range, which is
    the failure the fp32 statistics avoid (the GroupNorm pull request's fp16 overflow, Summary)."""
    wl = WORKLOADS["fp16_8192x8192"]
    inp = make_inputs(wl, M=4)
    x = inp["x"]
    acc = np.float16(0)
    with np.errstate(over="ignore"):
        for v in x[0].astype(np.float16):
            acc = np.float16(acc + v * v)
    assert np.isinf(acc)
    y, r = rmsnorm_fwd(x, inp["w"], eps=wl.eps, dtype="f16")
    dx, dw = rmsnorm_bwd(inp["dy"], x, inp["w"], r, dtype="f16")
    assert np.isfinite(r).all() and np.isfinite(y).all()
    assert np.isfinite(dx).all() and np.isfinite(dw).all()


def test_nan_and_zero_rows_propagate():
    x = np.zeros((3, 8), np.float32)
    x[1, 3] = np.nan
    x[2] = 1.0
    w = np.ones(8, np.float32)
    y, r = rmsnorm_fwd(x, w, eps=0.0, dtype="bf16")
    assert np.isinf(r[0]) and np.isnan(y[0]).all()      # zero row, eps = 0: 0 * inf
    assert np.isnan(r[1]) and np.isnan(y[1]).all()      # a NaN poisons its row only
    assert np.isfinite(y[2]).all() and np.all(y[2] == 1.0)
    y, r = rmsnorm_fwd(x[[0]], w, eps=1e-6, dtype="bf16")
    assert np.all(y == 0) and np.isfinite(r).all()       # zero row, eps > 0: zeros


def test_input_validation():
    with pytest.raises(ValueError):
        rmsnorm_fwd(np.zeros((1, 2)), np.zeros(2), eps=0.0, dtype="f64")
    with pytest.raises(ValueError):
        rmsnorm_fwd(np.zeros((1, 2)), np.zeros(2), eps=0.0, rounding="thrice")


# --------------------------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# --------------------------------------------------------------------------------------------

MUTATIONS = {
    "mean over N-1": ("ms = np.sum(x64 * x64, axis=-1) / n", "ms = np.sum(x64 * x64, axis=-1) / (n - 1)"),
    "eps outside the root": ("r = 1.0 / np.sqrt(ms + eps64)", "r = 1.0 / np.sqrt(ms) + eps64"),
    "sign of the projection": ("dx = r * (gdy - xhat * c)", "dx = r * (gdy + xhat * c)"),
    "dropped projection": ("dx = r * (gdy - xhat * c)", "dx = r * gdy"),
    "dropped rstd factor in dx": ("dx = r * (gdy - xhat * c)", "dx = (gdy - xhat * c)"),
    "mean of the projection not divided": (
        "axis=-1) / n\n        c = (c", "axis=-1)\n        c = (c"),
    "gain in dw": ("dw = np.sum(dy.astype(np.float64) * xw", "dw = np.sum(gdy.astype(np.float64) * xw"),
    "column sum for dw transposed": ("xw.astype(np.float64), axis=0)", "xw.astype(np.float64), axis=1)"),
    "round twice without the inner cast": (
        "return rne_to(rne_to(xhat, dtype) * g, dtype)", "return rne_to(xhat * g, dtype)"),
    "round once with an inner cast": (
        "return rne_to(xhat * g, dtype)", "return rne_to(rne_to(xhat, dtype) * g, dtype)"),
    "offset dropped from the float32 gain": (
        "return np.float32(offset) + np.asarray(w, np.float32)", "return np.asarray(w, np.float32)"),
    "offset dropped from the float64 gain": (
        "return np.float64(offset) + np.asarray(w, np.float64)", "return np.asarray(w, np.float64)"),
    "autograd casts without the gain-product rounding": (
        "gdy = rne_to(gdy, dtype)", "gdy = gdy"),
    "autograd casts without the rounded xhat in dw": (
        "xw = rne_to(xhat, dtype) if ag else xhat", "xw = xhat"),
    "xhat from the squared sum without the root": (
        "r = 1.0 / np.sqrt(ms + eps64)", "r = 1.0 / (ms + eps64)"),
}


def _mutant(src_old, src_new):
    src = open(oracle_rmsnorm.__file__, encoding="utf-8").read()
    assert src.count(src_old) >= 1, src_old
    src = src.replace(src_old, src_new, 1)
    mod = types.ModuleType("oracle._mutant")
    mod.__package__ = "oracle"
    mod.__file__ = "<mutant>"
    exec(compile(src, "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in PIN_SUITE:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake: {name}"
