"""Pins for the oracle's OCP 8-bit rounding and its FP8-output forward (CPU only).

The rounding is checked against torch's float8_e4m3fn / float8_e5m2 casts over sampled float32 bit
patterns (including every tie of the sampled binades, subnormals and overflow) and hand cases; the
forward against torch's CPU RMSNorm in float32 followed by the scale and torch's float8 cast.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import rne_fp8, rmsnorm_fwd_fp8
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def _torch_cast(v, fmt):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(TORCH_FP8[fmt]).float().numpy()


def _same(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return (np.isnan(a) & np.isnan(b)) | (a.view(np.uint32) == b.view(np.uint32))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_matches_torch_cast_on_bit_sample(fmt):
    pats = np.arange(0, 2**32, 4099, dtype=np.uint64).astype(np.uint32)
    v = pats.view(np.float32)
    assert _same(rne_fp8(v, fmt), _torch_cast(v, fmt)).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_matches_torch_cast_on_ties_and_small_values(fmt):
    p = {"e4m3": 4, "e5m2": 3}[fmt]
    rng = np.random.default_rng(5)
    e = rng.integers(-20, 17, 200_000)
    m = rng.integers(0, 2**p, 200_000)
    # exact midpoints between neighbours of the 8-bit grid (and their negatives)
    ties = (np.ldexp(1.0 + (2 * m + 1) / 2.0**p, e) * rng.choice([-1, 1], 200_000)).astype(np.float32)
    small = rng.uniform(-2.0**-5, 2.0**-5, 200_000).astype(np.float32)
    for v in (ties, small):
        assert _same(rne_fp8(v, fmt), _torch_cast(v, fmt)).all()


@pytest.mark.parametrize("value,e4m3,e5m2", [
    (448.0, 448.0, 448.0),
    (464.0, 448.0, 448.0),          # e4m3: tie between 448 and the NaN code: even is 448
    (470.0, np.nan, 448.0),         # e4m3 overflow is NaN (no infinities)
    (57344.0, np.nan, 57344.0),     # largest finite e5m2
    (61440.0, np.nan, np.inf),      # e5m2: tie with 2^16, even, overflows
    (2.0**-9, 2.0**-9, 2.0**-9),    # smallest e4m3 subnormal
    (2.0**-10, 0.0, 2.0**-10),      # half of it: tie to even (zero) in e4m3
    (2.0**-16, 0.0, 2.0**-16),      # smallest e5m2 subnormal
    (-np.inf, np.nan, -np.inf),
])
def test_fp8_hand_cases(value, e4m3, e5m2):
    for fmt, want in (("e4m3", e4m3), ("e5m2", e5m2)):
        got = float(rne_fp8(np.float32(value), fmt))
        assert (np.isnan(got) and np.isnan(want)) or got == want, (fmt, value, got)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_forward_matches_torch_rms_norm_then_cast(fmt, dtype):
    """torch's CPU RMSNorm on float32 values, times the gain, times the scale, cast to 8 bits:
    equal on >= 99.9 % of elements (the rest differ by the statistic's summation order)."""
    wl = WORKLOADS["bf16_4096x4096"].with_(dtype=dtype)
    inp = make_inputs(wl, M=256, N=1024, seed=21)
    x, w = inp["x"], inp["w"]
    scale = 37.5 if fmt == "e4m3" else 1.0e3
    y8, r = rmsnorm_fwd_fp8(x, w, eps=1e-6, scale=scale, fmt=fmt, dtype=dtype)
    xt = torch.from_numpy(x)
    yt = torch.nn.functional.rms_norm(xt, (1024,), eps=1e-6) * torch.from_numpy(w)
    yt = (yt * np.float32(scale)).to(TORCH_FP8[fmt]).float().numpy()
    assert np.mean(_same(y8, yt)) >= 0.999
    # the rstd cache is the ordinary forward's
    _, r2 = oracle.rmsnorm_fwd(x, w, eps=1e-6, dtype=dtype)
    assert np.array_equal(r, r2)


def test_fp8_forward_is_the_float32_forward_scaled_and_cast():
    """With a power-of-two scale (which commutes with every float32 rounding) the FP8 output is the
    float32 forward's output (pinned separately) times the scale, cast to 8 bits."""
    inp = make_inputs(WORKLOADS["bf16_4096x4096"], M=64, N=512, seed=22)
    x, w = inp["x"], inp["w"]
    y32, _ = oracle.rmsnorm_fwd(x, w, eps=1e-6, dtype="f32")
    for fmt, k in (("e5m2", 2), ("e4m3", 5), ("e4m3", -1)):
        y8, _ = rmsnorm_fwd_fp8(x, w, eps=1e-6, scale=2.0**k, fmt=fmt)
        assert np.array_equal(y8, rne_fp8(y32 * np.float32(2.0**k), fmt), equal_nan=True)
