"""Pins for the oracle's LayerNorm and GroupNorm (CPU only).

Each pin ties the oracle to something other than itself: closed forms (zero mean and unit variance
of the output at unit weight, zero bias and epsilon 0; the sums of dx and of xhat * dx), exact
invariants (power-of-two scaling), float64 central finite differences of the forward, torch float64
autograd of torch's own layer_norm and group_norm, and the GroupNorm facts the Liger-Kernel pull
request "fix(group_norm): keep the backward statistics and reductions in fp32" prints (Details and
the issue snippets: an input gradient of exactly zero and finite for an upstream gradient of ones,
and a bias gradient of 65536 that float16 cannot hold). A final test plants plausible mistakes in a
copy of the oracle and checks that the pins catch every one.
"""
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.layernorm as oracle_ln
from workloads import to_dtype_values

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand(shape, seed, dtype="f32", scale=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    return to_dtype_values(rng.standard_normal(shape) * scale + shift, dtype)


# --------------------------------------------------------------------------------------------
# Pin suite, parameterised by the oracle module so the mutation test can run it on planted bugs.
# --------------------------------------------------------------------------------------------

def pin_standardized_rows(mod):
    """w = 1, b = 0, eps = 0: every LayerNorm row, and every GroupNorm group, has mean 0 and
    variance 1 (float64, exact mode); the float32 statistics are the rounded float64 ones."""
    x = _rand((5, 48), 1, shift=3.0)
    y, mean, rstd = mod.layernorm_fwd(x, np.ones(48), None, eps=0.0, dtype="f32", exact=True)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-12)
    x64 = np.asarray(x, np.float64)
    assert np.allclose(mean, x64.mean(axis=1), rtol=1e-15)
    assert np.allclose(rstd, 1.0 / x64.std(axis=1), rtol=1e-12)
    xg = _rand((2, 6, 10), 2, shift=-2.0)
    yg, _, _ = mod.groupnorm_fwd(xg, np.ones(6), np.zeros(6), G=3, eps=0.0, dtype="f32",
                                 exact=True)
    rows = np.asarray(yg).reshape(2, 3, 20)
    assert np.allclose(rows.mean(axis=2), 0.0, atol=1e-12)
    assert np.allclose((rows ** 2).mean(axis=2), 1.0, rtol=1e-12)


def pin_affine(mod):
    """Constant-row check of the affine step: a row whose centred values are +-1 has rstd 1 at
    eps 0, so y = RNE_T(fl(+-w + b)) exactly."""
    x = np.array([[3.0, 1.0, 3.0, 1.0]], np.float32)  # mean 2, variance 1
    w = np.array([1.5, -2.0, 0.25, 3.0], np.float32)
    b = np.array([0.5, 0.5, -1.0, 2.0], np.float32)
    y, mean, rstd = mod.layernorm_fwd(x, w, b, eps=0.0, dtype="f32")
    assert float(mean[0]) == 2.0 and float(rstd[0]) == 1.0
    assert y.tolist() == [[2.0, 2.5, -0.75, -1.0]]
    y2, _, _ = mod.layernorm_fwd(x, w, None, eps=0.0, dtype="f32")
    assert y2.tolist() == [[1.5, 2.0, 0.25, -3.0]]


def _ln_loss(mod, x, w, b, dy, eps):
    y, _, _ = mod.layernorm_fwd(x, w, b, eps=eps, dtype="f32", exact=True)
    return float(np.sum(np.asarray(dy, np.float64) * y))


def pin_ln_finite_differences(mod, M=3, N=7, eps=1e-3, seed=3, h=1e-6):
    x = _rand((M, N), seed, shift=0.7).astype(np.float64)
    w = _rand((N,), seed + 1, shift=1.0).astype(np.float64)
    b = _rand((N,), seed + 2).astype(np.float64)
    dy = _rand((M, N), seed + 3).astype(np.float64)
    _, mean, rstd = mod.layernorm_fwd(x, w, b, eps=eps, dtype="f32", exact=True)
    dx, dw, db = mod.layernorm_bwd(dy, x, w, mean, rstd, dtype="f32", exact=True)

    def fd(arr, setter):
        g = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            g[idx] = (_ln_loss(mod, *setter(p), dy, eps) - _ln_loss(mod, *setter(m), dy, eps)) / (2 * h)
        return g

    assert np.allclose(dx, fd(x, lambda v: (v, w, b)), rtol=1e-6, atol=1e-7)
    assert np.allclose(dw, fd(w, lambda v: (x, v, b)), rtol=1e-6, atol=1e-7)
    assert np.allclose(db, fd(b, lambda v: (x, w, v)), rtol=1e-6, atol=1e-7)


def pin_gn_torch_autograd(mod, B=2, C=6, S=5, G=3, eps=1e-4, seed=7):
    """Forward and all three gradients against torch's float64 group_norm and layer_norm."""
    x = _rand((B, C, S), seed, shift=1.5).astype(np.float64)
    w = _rand((C,), seed + 1, shift=1.0).astype(np.float64)
    b = _rand((C,), seed + 2).astype(np.float64)
    dy = _rand((B, C, S), seed + 3).astype(np.float64)
    y, mean, rstd = mod.groupnorm_fwd(x, w, b, G=G, eps=eps, dtype="f32", exact=True)
    dx, dw, db = mod.groupnorm_bwd(dy, x, w, mean, rstd, G=G, dtype="f32", exact=True)
    tx, tw, tb = (torch.tensor(a, requires_grad=True) for a in (x, w, b))
    ty = torch.nn.functional.group_norm(tx, G, tw, tb, eps)
    ty.backward(torch.tensor(dy))
    assert np.allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(db, tb.grad.numpy(), rtol=1e-10, atol=1e-12)
    # LayerNorm over the last axis
    x2, dy2 = x.reshape(B * C, S), dy.reshape(B * C, S)
    w2, b2 = _rand((S,), seed + 4, shift=1.0).astype(np.float64), _rand((S,), seed + 5).astype(np.float64)
    y2, m2, r2 = mod.layernorm_fwd(x2, w2, b2, eps=eps, dtype="f32", exact=True)
    dx2, dw2, db2 = mod.layernorm_bwd(dy2, x2, w2, m2, r2, dtype="f32", exact=True)
    tx, tw, tb = (torch.tensor(a, requires_grad=True) for a in (x2, w2, b2))
    ty = torch.nn.functional.layer_norm(tx, (S,), tw, tb, eps)
    ty.backward(torch.tensor(dy2))
    assert np.allclose(y2, ty.detach().numpy(), rtol=1e-12, atol=1e-12)
    for a, t in ((dx2, tx), (dw2, tw), (db2, tb)):
        assert np.allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_dx_sums(mod, eps=0.01):
    """Per row: sum_j dx_j = 0 (shift invariance) and, for the exact function,
    sum_j xhat_j dx_j = rstd * eps / (var + eps) * sum_j w_j dy_j xhat_j (scale invariance broken
    only by eps)."""
    x = _rand((4, 33), 8, shift=-1.0).astype(np.float64)
    w = _rand((33,), 9, shift=1.0).astype(np.float64)
    dy = _rand((4, 33), 10).astype(np.float64)
    _, mean, rstd = mod.layernorm_fwd(x, w, None, eps=eps, dtype="f32", exact=True)
    dx, _, _ = mod.layernorm_bwd(dy, x, w, mean, rstd, dtype="f32", exact=True)
    assert np.allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    var = x.var(axis=1)
    xhat = (x - x.mean(axis=1, keepdims=True)) / np.sqrt(var + eps)[:, None]
    lhs = np.sum(xhat * dx, axis=1)
    rhs = (1.0 / np.sqrt(var + eps)) * eps / (var + eps) * np.sum(w * dy * xhat, axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-13)


def pin_groupnorm_ones_page_case(mod):
    """Liger-Kernel pull request "fix(group_norm): ...": (1, 16, 256, 256) in float16 with 4 groups
    and an upstream gradient of ones (weight 1, bias 0, the module's initial values). The exact
    input gradient is zero (the output sums to a constant per group); the page's issue snippets
    expect 0 and print 0.0 after the fix and 466.0 before it, with every one of the 1048576 elements
    finite. Their inputs are not printed; for x ~ N(0, 1) the float32 rounding of x - mean leaves a
    residual of at most one float16 subnormal step (2^-24), far from the broken value. The bias
    gradient is 65536 per channel, a value float16 cannot hold (Testing Done)."""
    B, C, S, G = 1, 16, 256 * 256, 4
    x = _rand((B, C, S), 12, "f16")
    w, b = np.ones(C, np.float32), np.zeros(C, np.float32)
    dy = np.ones((B, C, S), np.float32)
    _, mean, rstd = mod.groupnorm_fwd(x, w, b, G=G, eps=1e-5, dtype="f16")
    dx, dw, db = mod.groupnorm_bwd(dy, x, w, mean, rstd, G=G, dtype="f16")
    assert int(np.isfinite(dx).sum()) == 1048576
    assert float(np.abs(dx).max()) <= 2.0**-24
    assert float(np.mean(dx == 0.0)) > 0.99
    assert np.all(db == 65536.0)
    # dw_c sums xhat over channel c; over the channels of a group xhat sums to zero
    assert np.all(np.abs(dw.astype(np.float64).reshape(G, C // G).sum(axis=1)) < 0.05)


PIN_SUITE = [pin_standardized_rows, pin_affine, pin_ln_finite_differences, pin_gn_torch_autograd,
             pin_dx_sums, pin_groupnorm_ones_page_case]


def test_standardized_rows():
    pin_standardized_rows(oracle_ln)


def test_affine_step_exact():
    pin_affine(oracle_ln)


def test_layernorm_finite_differences():
    pin_ln_finite_differences(oracle_ln)


@pytest.mark.parametrize("eps", [0.0, 1e-5])
def test_layernorm_finite_differences_eps(eps):
    pin_ln_finite_differences(oracle_ln, eps=eps, N=9, seed=21)


def test_groupnorm_and_layernorm_match_torch_float64_autograd():
    pin_gn_torch_autograd(oracle_ln)


@pytest.mark.parametrize("B,C,S,G", [(1, 4, 2, 4), (3, 8, 3, 2), (2, 4, 6, 1), (2, 6, 1, 3)])
def test_groupnorm_torch_autograd_shapes(B, C, S, G):
    pin_gn_torch_autograd(oracle_ln, B=B, C=C, S=S, G=G, seed=B * 100 + C)


def test_single_element_groups():
    """One element per group: xhat = 0, so y = b and dx = 0 exactly (torch refuses this shape)."""
    x = _rand((2, 4, 1), 60, "bf16")
    w, b = _rand((4,), 61, "bf16", shift=1.0), _rand((4,), 62, "bf16")
    dy = _rand((2, 4, 1), 63, "bf16")
    y, m, r = oracle.groupnorm_fwd(x, w, b, G=4, eps=1e-5, dtype="bf16")
    assert np.array_equal(y[:, :, 0], np.broadcast_to(b, (2, 4)))
    dx, dw, db = oracle.groupnorm_bwd(dy, x, w, m, r, G=4, dtype="bf16")
    assert np.all(dx == 0.0) and np.all(dw == 0.0)
    assert np.array_equal(db, oracle.rne_f32(dy[:, :, 0].astype(np.float64).sum(axis=0)))


def test_dx_sums():
    pin_dx_sums(oracle_ln)
    pin_dx_sums(oracle_ln, eps=0.0)


def test_groupnorm_ones_page_case():
    pin_groupnorm_ones_page_case(oracle_ln)


def test_groupnorm_is_layernorm_of_group_rows():
    """G = C with S elements per channel and unit affine equals LayerNorm over each channel; G = 1
    equals LayerNorm over each whole sample (weights constant)."""
    x = _rand((3, 4, 16), 30, "bf16", shift=2.0)
    y, m, r = oracle.groupnorm_fwd(x, np.ones(4), None, G=4, eps=1e-6, dtype="bf16")
    y2, m2, r2 = oracle.layernorm_fwd(x.reshape(12, 16), np.ones(16), None, eps=1e-6, dtype="bf16")
    assert np.array_equal(y.reshape(12, 16), y2)
    assert np.array_equal(m.reshape(-1), m2) and np.array_equal(r.reshape(-1), r2)
    y3, _, _ = oracle.groupnorm_fwd(x, np.full(4, 0.5), None, G=1, eps=1e-6, dtype="bf16")
    y4, _, _ = oracle.layernorm_fwd(x.reshape(3, 64), np.full(64, 0.5), None, eps=1e-6,
                                    dtype="bf16")
    assert np.array_equal(y3.reshape(3, 64), y4)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_power_of_two_scaling_is_exact(dtype):
    """eps = 0: y(2^k x) == y(x) bit for bit; dx(2^k x) == 2^-k dx(x) (float32 dy path)."""
    x = _rand((6, 40), 31, dtype, shift=0.5)
    w = _rand((40,), 32, dtype, shift=1.0)
    b = _rand((40,), 33, dtype)
    dy = _rand((6, 40), 34, dtype)
    y, m, r = oracle.layernorm_fwd(x, w, b, eps=0.0, dtype=dtype)
    for k in (-3, 4):
        xs = (x * np.float32(2.0 ** k)).astype(np.float32)
        ys, ms, rs = oracle.layernorm_fwd(xs, w, b, eps=0.0, dtype=dtype)
        assert np.array_equal(ys, y)
        assert np.array_equal(ms, m * np.float32(2.0 ** k))
        assert np.array_equal(rs, r * np.float32(2.0 ** -k))
    if dtype == "f32":
        dx, dw, db = oracle.layernorm_bwd(dy, x, w, m, r, dtype=dtype)
        xs = (x * np.float32(8.0)).astype(np.float32)
        _, ms, rs = oracle.layernorm_fwd(xs, w, b, eps=0.0, dtype=dtype)
        dxs, dws, dbs = oracle.layernorm_bwd(dy, xs, w, ms, rs, dtype=dtype)
        assert np.array_equal(dxs, dx / np.float32(8.0))
        assert np.array_equal(dws, dw) and np.array_equal(dbs, db)


def test_float32_path_close_to_exact():
    x = _rand((16, 256), 40, "f32", shift=4.0)
    w = _rand((256,), 41, "f32", shift=1.0)
    b = _rand((256,), 42, "f32")
    dy = _rand((16, 256), 43, "f32")
    y, m, r = oracle.layernorm_fwd(x, w, b, eps=1e-5, dtype="f32")
    ye, me, re = oracle.layernorm_fwd(x, w, b, eps=1e-5, dtype="f32", exact=True)
    assert np.max(np.abs(y - ye)) < 4e-6 * np.max(np.abs(ye))
    dx, dw, db = oracle.layernorm_bwd(dy, x, w, m, r, dtype="f32")
    dxe, dwe, dbe = oracle.layernorm_bwd(dy, x, w, me, re, dtype="f32", exact=True)
    assert np.linalg.norm(dx - dxe) <= 1e-5 * np.linalg.norm(dxe)
    assert np.linalg.norm(dw - dwe) <= 1e-6 * np.linalg.norm(dwe)
    assert np.array_equal(db, oracle.rne_f32(dbe))


def test_large_offset_variance_is_not_cancelled():
    """A row with mean 4096 and spread 2^-6 (float32 values 4096 + k/64): the float64 two-pass
    variance is exact, where E[x^2] - mean^2 in float32 would lose it entirely."""
    k = np.arange(-8, 8, dtype=np.float64)
    x = (4096.0 + k / 64.0).astype(np.float32)[None, :]
    _, mean, rstd = oracle.layernorm_fwd(x, np.ones(16), None, eps=0.0, dtype="f32")
    var = np.var(k / 64.0)
    assert float(mean[0]) == 4096.0 - 0.5 / 64.0
    assert float(rstd[0]) == float(oracle.rne_f32(1.0 / np.sqrt(var)))
    x32 = x.astype(np.float32)
    naive = np.float32(np.mean(x32 * x32, dtype=np.float32) - np.mean(x32, dtype=np.float32) ** 2)
    assert abs(float(naive) - var) > 0.5 * var  # the cancellation the two-pass form avoids


def test_input_validation():
    x = _rand((2, 4, 3), 50)
    with pytest.raises(ValueError):
        oracle.groupnorm_fwd(x, np.ones(4), None, G=3, eps=0.0)
    with pytest.raises(ValueError):
        oracle.layernorm_fwd(x[0], np.ones(3), None, eps=0.0, dtype="f64")


# --------------------------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# --------------------------------------------------------------------------------------------

MUTATIONS = {
    "variance over n-1": ("** 2, axis=-1) / n", "** 2, axis=-1) / (n - 1)"),
    "variance about zero": ("(x64 - mu[..., None]) ** 2", "x64 ** 2"),
    "eps outside the root": ("r = 1.0 / np.sqrt(var + eps64)", "r = 1.0 / np.sqrt(var) + eps64"),
    "mean not subtracted in xhat": (
        "(np.asarray(x, F) - np.asarray(mean, F)[..., None])", "np.asarray(x, F)"),
    "bias dropped": ("y = y + np.asarray(b, F)", "y = y"),
    "bias added before the weight": ("y = xhat * np.asarray(w, F)\n        if b is not None:\n            y = y + np.asarray(b, F)",
                                     "y = xhat\n        if b is not None:\n            y = y + np.asarray(b, F)\n        y = y * np.asarray(w, F)"),
    "dropped mean term in dx": ("dx = r * ((gdy - c1) - xhat * c2)", "dx = r * (gdy - xhat * c2)"),
    "dropped projection in dx": ("dx = r * ((gdy - c1) - xhat * c2)", "dx = r * (gdy - c1)"),
    "sign of the projection": ("dx = r * ((gdy - c1) - xhat * c2)", "dx = r * ((gdy - c1) + xhat * c2)"),
    "rstd factor dropped": ("dx = r * ((gdy - c1) - xhat * c2)", "dx = ((gdy - c1) - xhat * c2)"),
    "c1 without the weight": ("c1 = np.sum(gdy.astype(np.float64), axis=-1) / n",
                              "c1 = np.sum(dy.astype(np.float64), axis=-1) / n"),
    "c2 without the weight": ("c2 = np.sum(gdy.astype(np.float64) * xhat",
                              "c2 = np.sum(dy.astype(np.float64) * xhat"),
    "weight gradient uses w * dy": (
        "dw = np.sum(dy64 * xhat.astype(np.float64), axis=0)",
        "dw = np.sum(dy64 * np.asarray(w, np.float64) * xhat.astype(np.float64), axis=0)"),
    "bias gradient sums xhat": ("db = np.sum(dy64, axis=0)", "db = np.sum(xhat.astype(np.float64), axis=0)"),
    "group channels interleaved": ("return np.repeat(v.reshape(G, C // G), S, axis=1)",
                                   "return np.tile(v.reshape(G, C // G), (1, S))"),
    "group weight gradient over the wrong axes": (
        "reshape(B, C, S), axis=(0, 2))", "reshape(B, C, S), axis=(0, 1)).sum() + np.zeros(C)"),
    "float32 c2 without the mean": (
        "c2 = np.sum(gdy.astype(np.float64) * xhat.astype(np.float64), axis=-1) / n",
        "c2 = np.sum(gdy.astype(np.float64) * xhat.astype(np.float64), axis=-1)"),
}


def _mutant(src_old, src_new):
    src = open(oracle_ln.__file__, encoding="utf-8").read()
    assert src.count(src_old) >= 1, src_old
    src = src.replace(src_old, src_new, 1)
    mod = types.ModuleType("oracle._mutant_ln")
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
