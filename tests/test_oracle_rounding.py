"""Pins for the oracle's round-to-nearest-even (CPU only).

The rounding functions are checked against values the blog post "Den dolda avrundningen i RMSNorm"
prints, against independent library conversions (torch's CPU bfloat16 cast, NumPy's float16 and
float32 casts) over large structured samples of bit patterns, and against hand-derived edge cases.
"""
import math

import numpy as np
import pytest
import torch

from golden.load import load
from oracle import apply_gain, rne_bf16, rne_f16, rne_f32, round_to_format, ulp_of

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_lib(a32):
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16).float().numpy()


def _same(a, b):
    """Elementwise equality that treats NaN == NaN and distinguishes +0 from -0."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return nan | ((a == b) & (np.signbit(a) == np.signbit(b)))


def _bit_sample(stride):
    """Every ``stride``-th float32 bit pattern, plus the patterns next to each power of two."""
    pats = np.arange(0, 2**32, stride, dtype=np.uint64).astype(np.uint32)
    exps = (np.arange(0, 256, dtype=np.uint32) << np.uint32(23))
    near = (exps[:, None] + np.arange(-70000, 70000, 97, dtype=np.int64)[None, :]).ravel()
    near = (near % 2**32).astype(np.uint32)
    allp = np.concatenate([pats, near, near | np.uint32(0x80000000)])
    return allp.view(np.float32)


def test_worked_example_bf16():
    g = load("worked_example.txt")
    gain = rne_bf16(np.float32(g["gain_decimal"]))
    assert float(gain) == g["gain_bf16"]
    xhat = np.float32(g["xhat_f32"])
    once = apply_gain(xhat, gain, rounding="once", dtype="bf16")
    twice = apply_gain(xhat, gain, rounding="twice", dtype="bf16")
    assert float(once) == g["round_once"]
    assert float(twice) == g["round_twice"]


def test_two_million_experiment():
    g = load("two_million_experiment.txt")
    rng = np.random.default_rng(g["seed"])
    n = g["samples"]
    xhat = rng.standard_normal(n).astype(np.float32)
    gamma = rng.uniform(g["gain_low"], g["gain_high"], n).astype(np.float32)
    gb = rne_bf16(gamma)
    once = apply_gain(xhat, gb, rounding="once", dtype="bf16")
    twice = apply_gain(xhat, gb, rounding="twice", dtype="bf16")
    diff = once != twice
    assert int(diff.sum()) == g["differing"]
    assert round(100.0 * diff.sum() / n, 2) == g["share_percent_2dp"]
    nz = once != 0
    rel = np.abs(once[nz].astype(np.float64) - twice[nz]) / np.abs(once[nz].astype(np.float64))
    assert 100.0 * rel.max() == pytest.approx(g["max_relative_percent"], abs=1e-9)
    # differing outputs are neighbours on the bf16 grid
    bo = once[diff].view(np.uint32) >> 16
    bt = twice[diff].view(np.uint32) >> 16
    same_sign = (bo >> 15) == (bt >> 15)
    steps = np.abs(bo.astype(np.int64) - bt.astype(np.int64))
    assert same_sign.all() and steps.max() == g["max_bf16_steps_apart"]


def test_bf16_matches_library_cast_on_bit_sample():
    v = _bit_sample(1021)
    ours = rne_bf16(v)
    lib = _bf16_lib(v)
    ok = _same(ours, lib)
    assert ok.all(), (v[~ok][:5], ours[~ok][:5], lib[~ok][:5])


def test_bf16_matches_library_cast_on_ties():
    # exact halfway points between adjacent bf16 values, both parities, all binades
    rng = np.random.default_rng(1)
    hi = rng.integers(0, 2**16, 2_000_000, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # drop Inf/NaN upper halves
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    ours = rne_bf16(ties)
    lib = _bf16_lib(ties)
    assert _same(ours, lib).all()
    # ties go to the even neighbour: the result's lowest kept bit is 0
    fin = np.isfinite(ours)
    assert ((ours[fin].view(np.uint32) >> 16) & 1 == 0).all()


def test_f16_matches_numpy_cast_on_bit_sample():
    v = _bit_sample(1021)
    ours = rne_f16(v)
    lib = v.astype(np.float16).astype(np.float32)
    ok = _same(ours, lib)
    assert ok.all(), (v[~ok][:5], ours[~ok][:5], lib[~ok][:5])


def test_f16_matches_numpy_cast_in_subnormal_and_overflow_ranges():
    rng = np.random.default_rng(2)
    a = np.concatenate([
        rng.uniform(-2.0**-13, 2.0**-13, 1_000_000),
        rng.uniform(65000.0, 66000.0, 200_000),
        -rng.uniform(65000.0, 66000.0, 200_000),
        np.arange(0, 2**-13, 2.0**-26),  # multiples of a quarter of the smallest subnormal
    ]).astype(np.float32)
    assert _same(rne_f16(a), a.astype(np.float16).astype(np.float32)).all()


def test_f32_matches_numpy_cast():
    rng = np.random.default_rng(3)
    a = np.concatenate([
        rng.standard_normal(1_000_000) * np.exp2(rng.integers(-140, 120, 1_000_000)),
        np.array([3.4028235677973366e38, 3.4028235e38 * 1.0000001, 1e-46, -1e-45, 2.0**-150]),
    ])
    assert _same(rne_f32(a), a.astype(np.float32)).all()


@pytest.mark.parametrize("value,expected", [
    (1.0 + 2.0**-8, 1.0),                       # tie between 1 and 1+2^-7: even is 1
    (1.0 + 3 * 2.0**-8, 1.0 + 2.0**-6),         # tie between 1+2^-7 and 1+2^-6: even is 1+2^-6
    (1.0 + 2.0**-8 + 2.0**-20, 1.0 + 2.0**-7),  # just above the tie rounds up
    (-(1.0 + 2.0**-8), -1.0),
    (float(np.finfo(np.float32).max), math.inf),  # carry out of the largest binade
    ((2 - 2.0**-7) * 2.0**127, (2 - 2.0**-7) * 2.0**127),  # largest finite bf16 is kept
    (2.0**-133, 2.0**-133),                     # smallest bf16 subnormal
    (2.0**-134, 0.0),                           # half of it: tie to even (zero)
    (3 * 2.0**-134, 2.0**-132),                 # 1.5 subnormal steps: tie to even (2 steps)
])
def test_bf16_hand_cases(value, expected):
    assert float(rne_bf16(np.float32(value))) == expected


@pytest.mark.parametrize("value,expected", [
    (65504.0, 65504.0),          # largest finite binary16
    (65519.0, 65504.0),          # below the halfway point to 2^16
    (65520.0, math.inf),         # halfway: ties to the even 2^16, which overflows
    (2.0**-24, 2.0**-24),        # smallest subnormal
    (2.0**-25, 0.0),             # half the smallest subnormal: tie to even (zero)
    (3 * 2.0**-25, 2.0**-23),    # tie between 1 and 2 subnormal steps: even is 2
    (1.0 + 2.0**-11, 1.0),       # tie between 1 and 1+2^-10
    (2049.0, 2048.0),            # spacing 2 above 2048: tie to even
    (2051.0, 2052.0),
])
def test_f16_hand_cases(value, expected):
    assert float(rne_f16(np.float32(value))) == expected


def test_special_values():
    sp = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0], np.float32)
    for f in (rne_bf16, rne_f16):
        r = f(sp)
        assert np.isnan(r[0])
        assert r[1] == np.inf and r[2] == -np.inf
        assert r[3] == 0 and not np.signbit(r[3])
        assert r[4] == 0 and np.signbit(r[4])
    # negative values that round to zero keep their sign
    assert np.signbit(rne_f16(np.float32(-2.0**-26)))
    assert np.signbit(rne_bf16(np.float32(-2.0**-140)))


def test_results_lie_on_the_grid_and_are_nearest():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 15, 200_000))).astype(np.float32)
    for fmt in ("bf16", "f16"):
        r = round_to_format(v, fmt).astype(np.float64)
        fin = np.isfinite(r)
        r, vf = r[fin], v[fin].astype(np.float64)
        # on the grid: an integer multiple of the local spacing
        assert np.all(np.mod(r, ulp_of(r, fmt)) == 0)
        # nearest: within half the spacing of the input's own binade
        assert np.all(np.abs(r - vf) <= 0.5 * ulp_of(vf, fmt))
