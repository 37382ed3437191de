"""Pins for the oracle's softmax (forward and backward) and its float64 RMSNorm (CPU only).

Pinned to: closed forms (two-element rows are the logistic function; rows of exp values 1, 2, 3;
uniform rows), invariants (rows sum to 1; adding a constant to a row changes nothing; dx sums to
zero), logits too large for a plain exp (the maximum must be subtracted), torch's float64 softmax
and autograd, float64 central finite differences, correct rounding of the 16-bit result (the candle
pull request's "rounds once at the store": error at most half a bfloat16 ulp),
and for the float64 RMSNorm finite differences and the float64 x . dx identity. A final test plants
plausible mistakes in a copy of the oracle and checks that the pins catch every one.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.softmax as oracle_sm
from workloads import to_dtype_values

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed, dtype="f32", scale=1.0):
    rng = np.random.default_rng(seed)
    return to_dtype_values(rng.standard_normal(shape) * scale, dtype)


def pin_closed_forms(mod):
    a, b = 0.3, -1.2
    y = mod.softmax_fwd(np.array([[a, b]]), dtype="f64")
    sig = 1.0 / (1.0 + math.exp(-(a - b)))
    assert abs(y[0, 0] - sig) < 1e-15 and abs(y[0, 1] - (1 - sig)) < 1e-15
    y = mod.softmax_fwd(np.log(np.array([[1.0, 2.0, 3.0]])), dtype="f64")
    assert np.allclose(y, [[1 / 6, 2 / 6, 3 / 6]], rtol=1e-15, atol=0)
    y = mod.softmax_fwd(np.full((2, 8), 0.7, np.float32), dtype="bf16")
    assert np.all(y == 0.125)
    y = mod.softmax_fwd(np.array([[1000.0, 1000.0, -1000.0]]), dtype="f64")
    assert y.tolist() == [[0.5, 0.5, 0.0]]


def pin_invariants(mod):
    x = _rand((5, 37), 1, scale=3.0).astype(np.float64)
    y = mod.softmax_fwd(x, dtype="f64")
    assert np.allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(mod.softmax_fwd(x + 11.5, dtype="f64"), y, rtol=1e-13, atol=0)
    dy = _rand((5, 37), 2).astype(np.float64)
    dx = mod.softmax_bwd(dy, y, dtype="f64")
    assert np.allclose(dx.sum(axis=1), 0.0, atol=1e-15)


def pin_torch_autograd(mod):
    x = _rand((4, 19), 3, scale=2.0).astype(np.float64)
    dy = _rand((4, 19), 4).astype(np.float64)
    tx = torch.tensor(x, requires_grad=True)
    ty = torch.softmax(tx, dim=-1)
    ty.backward(torch.tensor(dy))
    y = mod.softmax_fwd(x, dtype="f64")
    assert np.allclose(y, ty.detach().numpy(), rtol=1e-14, atol=1e-16)
    dx = mod.softmax_bwd(dy, y, dtype="f64")
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-15)


def pin_finite_differences(mod, h=1e-6):
    x = _rand((2, 6), 5).astype(np.float64)
    dy = _rand((2, 6), 6).astype(np.float64)
    dx = mod.softmax_bwd(dy, mod.softmax_fwd(x, dtype="f64"), dtype="f64")
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        p, m = x.copy(), x.copy()
        p[idx] += h
        m[idx] -= h
        g[idx] = (np.sum(dy * mod.softmax_fwd(p, dtype="f64")) -
                  np.sum(dy * mod.softmax_fwd(m, dtype="f64"))) / (2 * h)
    assert np.allclose(dx, g, rtol=1e-6, atol=1e-9)


def pin_correct_rounding(mod):
    """16-bit outputs are the exact softmax rounded once: within half an ulp of T (relative error
    at most 2^-8, the unit roundoff of bfloat16's 8-bit significand)."""
    x = _rand((64, 1024), 7, "bf16")
    y = mod.softmax_fwd(x, dtype="bf16")
    ye = mod.softmax_fwd(x, dtype="bf16", exact=True)
    rel = np.abs(y - ye) / ye
    assert rel.max() <= 2.0**-8
    assert np.array_equal(y, oracle.rne_bf16(ye))


def pin_rmsnorm_f64(mod, eps=1e-3, h=1e-6):
    x = _rand((3, 7), 8).astype(np.float64)
    w = _rand((7,), 9).astype(np.float64) + 1.0
    dy = _rand((3, 7), 10).astype(np.float64)
    y, r = mod.rmsnorm_fwd_f64(x, w, eps=eps, offset=0.5)
    assert np.allclose(r, 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps), rtol=1e-15)
    dx, dw = mod.rmsnorm_bwd_f64(dy, x, w, r, offset=0.5)
    loss = lambda xv, wv: float(np.sum(dy * mod.rmsnorm_fwd_f64(xv, wv, eps=eps, offset=0.5)[0]))  # noqa: E731
    for arr, grad, f in ((x, dx, lambda v: loss(v, w)), (w, dw, lambda v: loss(x, v))):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            g[idx] = (f(p) - f(m)) / (2 * h)
        assert np.allclose(grad, g, rtol=1e-6, atol=1e-9)


PIN_SUITE = [pin_closed_forms, pin_invariants, pin_torch_autograd, pin_finite_differences,
             pin_correct_rounding, pin_rmsnorm_f64]


@pytest.mark.parametrize("pin", PIN_SUITE, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle_sm)


def test_half_type_backward_uses_float32_steps():
    """16-bit backward: s rounded to float32, then dx = RNE_T(fl(y * fl(dy - s)))."""
    x = _rand((8, 300), 11, "bf16")
    y = oracle.softmax_fwd(x, dtype="bf16")
    dy = _rand((8, 300), 12, "bf16")
    dx = oracle.softmax_bwd(dy, y, dtype="bf16")
    s = oracle.rne_f32(np.sum(dy.astype(np.float64) * y.astype(np.float64), axis=1, keepdims=True))
    manual = oracle.rne_bf16(y * (dy - s.astype(np.float32)))
    assert np.array_equal(dx, manual)
    dxe = oracle.softmax_bwd(dy, y, dtype="bf16", exact=True)
    assert np.linalg.norm(dx - dxe) <= 2.0**-8 * np.linalg.norm(dxe)


def test_rounding_twice_is_worse():
    """The candle page: storing exp in bf16 and then scaling rounds twice; the fused forward now
    rounds once. On random rows the twice-rounded result is off by more."""
    x = _rand((64, 1024), 13, "bf16", scale=2.0)
    ye = oracle.softmax_fwd(x, dtype="bf16", exact=True)
    once = oracle.softmax_fwd(x, dtype="bf16")
    e = oracle.rne_bf16(np.exp(x.astype(np.float64) - x.max(axis=1, keepdims=True)))
    twice = oracle.rne_bf16(e / e.astype(np.float64).sum(axis=1, keepdims=True))
    err = lambda y: float(np.max(np.abs(y - ye) / ye))  # noqa: E731
    assert err(once) <= 2.0**-8 < err(twice)


def test_float32_output_is_correctly_rounded():
    x = _rand((4, 100), 14)
    assert np.array_equal(oracle.softmax_fwd(x, dtype="f32"),
                          oracle.rne_f32(oracle.softmax_fwd(x, dtype="f32", exact=True)))


def test_float32_bar_covers_the_rounded_difference():
    """The float32 softmax bar of the GPU tests, 2^-18 + 2^-20 relative: rounding x - max to float32
    and nothing else (exact exp, sum and division, then y rounded to float32) already goes past
    2^-18 on 64-wide rows spread up to 88 below their maximum, and stays inside the bar."""
    from parity import SM_F32_REL
    rng = np.random.default_rng(11)
    rows = []
    for sp in (50.0, 86.5, 86.99, 87.0, 87.01, 88.0, 100.0):
        for _ in range(3):
            r = rng.uniform(-sp, 0.0, 64).astype(np.float32)
            rows.append(r + np.float32(rng.uniform(-5, 5)))
    x = np.stack(rows)
    d = (x - x.max(axis=1, keepdims=True)).astype(np.float32)  # the only float32 step
    e = np.exp(d.astype(np.float64))
    y = oracle.rne_f32(e / e.sum(axis=1, keepdims=True))
    y_o = oracle.softmax_fwd(x, dtype="f32", exact=True)
    rel = np.abs(y - y_o) / np.maximum(np.abs(y_o), 1e-38)
    assert rel.max() > 2.0**-18
    assert rel.max() <= SM_F32_REL


def test_rmsnorm_f64_matches_exact_mode_for_float32_eps():
    x = _rand((5, 64), 15).astype(np.float64)
    w = _rand((64,), 16).astype(np.float64)
    y, r = oracle.rmsnorm_fwd_f64(x, w, eps=0.25, offset=1.0)
    y2, r2 = oracle.rmsnorm_fwd(x, w, eps=0.25, offset=1.0, dtype="f32", exact=True)
    assert np.allclose(y, y2, rtol=1e-15, atol=0) and np.allclose(r, r2, rtol=1e-15, atol=0)


def test_rmsnorm_f64_x_dot_dx_vanishes_at_eps_zero():
    x = _rand((4, 50), 17).astype(np.float64)
    w = _rand((50,), 18).astype(np.float64)
    dy = _rand((4, 50), 19).astype(np.float64)
    _, r = oracle.rmsnorm_fwd_f64(x, w, eps=0.0)
    dx, _ = oracle.rmsnorm_bwd_f64(dy, x, w, r)
    assert np.allclose(np.sum(x * dx, axis=1), 0.0, atol=1e-12)


def test_input_validation():
    with pytest.raises(ValueError):
        oracle.softmax_fwd(np.zeros((1, 2)), dtype="f8")


MUTATIONS = {
    "max not subtracted": ("e = np.exp(x64 - m)", "e = np.exp(x64)"),
    "normalized by the sum of x": ("y = e / np.sum(e, axis=-1, keepdims=True)",
                                   "y = e / np.sum(x64, axis=-1, keepdims=True)"),
    "backward without the y factor": ("dx = y * (dy - s.astype(F))", "dx = (dy - s.astype(F))"),
    "backward sign": ("dx = y * (dy - s.astype(F))", "dx = y * (dy + s.astype(F))"),
    "backward sum of dy alone": ("s = np.sum(dy.astype(np.float64) * y.astype(np.float64)",
                                 "s = np.sum(dy.astype(np.float64)"),
    "16-bit result rounded twice": ("return y if exact else _round(y, dtype)",
                                    "return y if exact else _round(_round(y * 1.5, dtype) / 1.5, dtype)"),
    "f64 rmsnorm eps outside the root": (
        "rstd = 1.0 / np.sqrt(np.sum(x * x, axis=-1) / n + np.float64(eps))",
        "rstd = 1.0 / np.sqrt(np.sum(x * x, axis=-1) / n) + np.float64(eps)"),
    "f64 rmsnorm offset dropped": ("(np.float64(offset) + np.asarray(w, np.float64))",
                                   "np.asarray(w, np.float64)"),
    "f64 rmsnorm mean over n-1": ("np.sum(x * x, axis=-1) / n", "np.sum(x * x, axis=-1) / (n - 1)"),
}


def _mutant(src_old, src_new):
    src = open(oracle_sm.__file__, encoding="utf-8").read()
    assert src.count(src_old) >= 1, src_old
    src = src.replace(src_old, src_new, 1)
    mod = types.ModuleType("oracle._mutant_sm")
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
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"


def test_half_type_check_accepts_only_midpoint_differences():
    """The 16-bit softmax check lets a value differ from the correctly rounded one only where the
    exact value lies within the float32 bound of the midpoint between the two candidates: moving
    the element nearest a midpoint to its other candidate passes, moving the element farthest
    from one fails."""
    from parity import check_softmax_fwd
    rng = np.random.default_rng(5)
    x = np.asarray(rng.standard_normal((40, 50)), np.float16).astype(np.float32)
    v = oracle.softmax_fwd(x, dtype="f16", exact=True)
    y = oracle.softmax_fwd(x, dtype="f16").astype(np.float16)
    other = np.where(v > y, np.nextafter(y, np.float16(np.inf)),
                     np.nextafter(y, np.float16(-np.inf)))
    gap = np.abs(v - (y.astype(np.float64) + other.astype(np.float64)) / 2) / np.abs(v)
    near, far = np.unravel_index(np.argmin(gap), gap.shape), np.unravel_index(np.argmax(gap),
                                                                               gap.shape)
    assert gap[near] <= 2.0**-18 < gap[far]
    check_softmax_fwd(y.astype(np.float32), x, dtype="f16")
    ok = y.copy()
    ok[near] = other[near]
    assert check_softmax_fwd(ok.astype(np.float32), x, dtype="f16")["y_off_midpoint"] == 0
    bad = y.copy()
    bad[far] = other[far]
    with pytest.raises(AssertionError):
        check_softmax_fwd(bad.astype(np.float32), x, dtype="f16")
