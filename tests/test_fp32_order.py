"""CPU pins of the float32 summation-order models behind the LayerNorm and GroupNorm dx bar.

The models (tests/fp32_order.py) reproduce the kernels' float32 order of the row sums c1 and c2;
parity.py lowers the 99.9 % bit-exact bar for a case only by what its model shows. Pinned here:
* integer inputs, whose float32 sums are exact in any order, give the exact sums;
* the order itself: one value 2^24 among ones, where each order loses a different number of
  them (sequential: all 63, the pairwise lane tree: one); for rows that are not 16-byte aligned,
  that the head element opens the even sum, and that without a head the peeled order is the
  register kernel's;
* the rates the bars rest on: >= 99.9 % on the LayerNorm and GroupNorm test inputs except the
  float16 rows of 70000 (and 9001 and 30001) elements with an upstream of ones (about 98.9 %, also
  the GPU's rates there).
"""
import numpy as np
import pytest

import oracle
from fp32_order import (gn_dx_model_bitexact, gn_row_kernel_mode, gn_segment_sums,
                        ln_dx_model_bitexact,
                        ln_row_sums, ln_row_sums_peel, row_heads)
from workloads import GN_WORKLOADS, LN_WORKLOADS, make_gn_inputs, make_norm_inputs


@pytest.mark.parametrize("V", [8, 1])
@pytest.mark.parametrize("N", [1, 7, 64, 1000, 8197, 70000])
def test_ln_row_sums_are_exact_on_integer_inputs(N, V):
    rng = np.random.default_rng(N)
    gd = rng.integers(-8, 9, size=(3, N)).astype(np.float32)
    xh = rng.integers(-8, 9, size=(3, N)).astype(np.float32)
    s1, s2 = ln_row_sums(gd, xh, V)
    assert np.array_equal(s1, gd.astype(np.float64).sum(axis=1))
    assert np.array_equal(s2, (gd.astype(np.float64) * xh).sum(axis=1))


def test_ln_row_sums_use_the_lane_tree():
    """512 bf16 elements: 64 vectors, one per lane of one wavefront, each lane's sum its vector's
    element 0. Lane 0 holds 2^24, the others 1: the pairwise tree loses only lane 1's 1 (2^24 + 1
    rounds to even), a sequential sum would lose all 63, the exact sum keeps them."""
    gd = np.zeros((1, 512), np.float32)
    gd[0, ::8] = 1.0
    gd[0, 0] = 2.0**24
    s1, _ = ln_row_sums(gd, np.ones_like(gd))
    assert s1[0] == 2.0**24 + 62


@pytest.mark.parametrize("N", [16, 17, 1027, 4097, 8199])
def test_ln_row_sums_peel_are_exact_on_integer_inputs(N):
    """Every element enters the peeled order once: integer sums are exact for rows of every
    head offset."""
    rng = np.random.default_rng(N)
    gd = rng.integers(-8, 9, size=(9, N)).astype(np.float32)
    xh = rng.integers(-8, 9, size=(9, N)).astype(np.float32)
    heads = row_heads(9, N, 2)
    assert len(set(heads.tolist())) > 1 or N % 8 == 0
    s1, s2 = ln_row_sums_peel(gd, xh, 8, heads)
    assert np.array_equal(s1, gd.astype(np.float64).sum(axis=1))
    assert np.array_equal(s2, (gd.astype(np.float64) * xh).sum(axis=1))


@pytest.mark.parametrize("N", [128, 1024, 4096, 8192])
def test_ln_row_sums_peel_without_a_head_is_the_wide_order(N):
    """Rows on a 16-byte boundary with whole vectors: one vector per lane in both mappings, so the
    peeled order is the register kernel's."""
    rng = np.random.default_rng(N + 1)
    gd = rng.standard_normal((5, N)).astype(np.float32)
    xh = rng.standard_normal((5, N)).astype(np.float32)
    a = ln_row_sums(gd, xh, 8)
    b = ln_row_sums_peel(gd, xh, 8, np.zeros(5, int))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_ln_row_sums_peel_head_opens_the_even_sum():
    """N = 17, h = 3 (bf16): lane 0 holds head element 0, whole vector 0 (elements 3..10) and tail
    element 11. With 2^24 at element 0 and ones at the vector's even positions, the head first in
    the even sum absorbs the four ones (2^24 + 1 rounds to 2^24); in the odd sum it would not."""
    gd = np.zeros((1, 17), np.float32)
    gd[0, 0] = 2.0**24
    gd[0, [3, 5, 7, 9]] = 1.0
    s1, _ = ln_row_sums_peel(gd, np.ones_like(gd), 8, np.array([3]))
    assert s1[0] == 2.0**24


LN_WL = {"bf16": LN_WORKLOADS["ln_bf16_4096x4096"], "f16": LN_WORKLOADS["ln_fp16_8192x8192"]}
LN_SHAPES = [(33, 64), (300, 1000), (257, 3072), (64, 4096), (40, 8192), (24, 16384), (12, 32768),
             (3, 70000)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,N", LN_SHAPES)
def test_ln_model_rates_on_the_test_inputs(dtype, M, N):
    wl = LN_WL[dtype]
    inp = make_norm_inputs(wl, M=M, N=N, seed=1)
    _, mean, rstd = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, dtype=dtype)
    rate = ln_dx_model_bitexact(inp["dy"], inp["x"], inp["w"], mean, rstd, dtype=dtype)
    if dtype == "f16" and N == 70000:
        # dy = 1, w in [0.9, 1.1]: w * dy - c1 cancels to about 0.05 of w; 9 vectors per thread
        # take compensated sums, yet the last bits of c1 still decide about 1 % of the roundings
        assert 0.985 <= rate < 0.995, rate
    else:
        assert rate >= 0.9995, rate


@pytest.mark.parametrize("dtype,M,N,lo,hi", [("f16", 12, 30001, 0.985, 0.995),
                                             ("f16", 129, 1027, 0.9995, 1.0),
                                             ("bf16", 12, 30001, 0.9995, 1.0)])
def test_ln_model_rates_element_wise(dtype, M, N, lo, hi):
    """Rows that are not 16-byte aligned: threads hold single elements 1024 apart (30 a thread at
    N = 30001, compensated sums). The float16 rows with unit upstream lose about 1 % as in the
    wide case."""
    wl = LN_WL[dtype]
    inp = make_norm_inputs(wl, M=M, N=N, seed=1)
    _, mean, rstd = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, dtype=dtype)
    rate = ln_dx_model_bitexact(inp["dy"], inp["x"], inp["w"], mean, rstd, dtype=dtype,
                                wide=False)
    assert lo <= rate <= hi, rate


@pytest.mark.parametrize("dtype,M,N,lo,hi", [("f16", 129, 1027, 0.985, 1.0),
                                             ("bf16", 129, 1027, 0.9995, 1.0),
                                             ("f16", 257, 4097, 0.985, 1.0)])
def test_ln_model_rates_peeled(dtype, M, N, lo, hi):
    """Rows not 16-byte aligned in the peeled register kernel's order (contiguous rows: every head
    offset occurs)."""
    wl = LN_WL[dtype]
    inp = make_norm_inputs(wl, M=M, N=N, seed=1)
    _, mean, rstd = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, dtype=dtype)
    rate = ln_dx_model_bitexact(inp["dy"], inp["x"], inp["w"], mean, rstd, dtype=dtype,
                                mapping="peel")
    assert lo <= rate <= hi, rate


GN_BASE = {"bf16": GN_WORKLOADS["gn_bf16_1x16x256x256_g4"],
           "f16": GN_WORKLOADS["gn_bf16_1x16x256x256_g4"].with_(dtype="f16")}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,C,S,G", [(2, 8, 8192, 2), (3, 6, 9000, 3), (2, 4, 20000, 2),
                                     (2, 4, 1000, 4), (4, 64, 64, 16)])
def test_gn_model_rates_on_the_test_inputs(dtype, B, C, S, G):
    wl = GN_BASE[dtype]
    inp = make_gn_inputs(wl, B=B, C=C, S=S, seed=B * 1000 + C + S)
    _, mean, rstd = oracle.groupnorm_fwd(inp["x"], inp["w"], inp["b"], G=G, eps=wl.eps,
                                         dtype=dtype)
    rate = gn_dx_model_bitexact(inp["dy"], inp["x"], inp["w"], mean, rstd, G=G, dtype=dtype)
    assert rate >= 0.999, rate


def test_gn_model_on_integer_chunks_is_exact():
    """With small integer x, dy and w, mean 0 and rstd 1 every float32 sum is exact, so the
    model's dx equals the oracle's everywhere."""
    rng = np.random.default_rng(3)
    B, C, S, G = 2, 4, 9000, 2
    x = rng.integers(-4, 5, size=(B, C, S)).astype(np.float32)
    dy = rng.integers(-4, 5, size=(B, C, S)).astype(np.float32)
    w = rng.integers(1, 4, size=C).astype(np.float32)
    mean = np.zeros((B, G), np.float32)
    rstd = np.ones((B, G), np.float32)
    assert gn_dx_model_bitexact(dy, x, w, mean, rstd, G=G, dtype="bf16") == 1.0
    # segments of at most a quarter chunk: one wavefront a chunk
    x1, dy1 = x[..., :1000], dy[..., :1000]
    for dt in ("bf16", "f32"):
        assert gn_dx_model_bitexact(dy1, x1, w, mean, rstd, G=G, dtype=dt, rows=False) == 1.0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,C,S,G", [(2, 16, 1025, 1), (1, 4096, 4, 1), (2, 1280, 1024, 32)])
def test_gn_model_rates_wavefront_chunks(dtype, B, C, S, G):
    """Chunked shapes whose segments fill at most a quarter chunk (one wavefront a chunk); the
    16-bit bar rests on these rates (float32 dx has a normwise bar)."""
    base = GN_BASE[dtype]
    inp = make_gn_inputs(base, B=B, C=C, S=S, seed=B * 1000 + C + S)
    _, mean, rstd = oracle.groupnorm_fwd(inp["x"], inp["w"], inp["b"], G=G, eps=base.eps,
                                         dtype=dtype)
    rate = gn_dx_model_bitexact(inp["dy"], inp["x"], inp["w"], mean, rstd, G=G, dtype=dtype,
                                rows=False)
    assert rate >= 0.999, rate


def test_gn_segment_sums_order():
    """65 elements: lane 0 adds elements 0 and 64, lanes 1..63 one each, then the pairwise lane tree.
    With 2^24 at element 0 and ones elsewhere, lane 0 loses element 64's one and the tree's first
    pair (2^24 + 1) loses lane 1's: 2^24 + 62 (a sequential sum would keep none of the 64 ones)."""
    p = np.ones((1, 1, 65), np.float32)
    p[0, 0, 0] = 2.0**24
    assert gn_segment_sums(p)[0, 0] == 2.0**24 + 62


@pytest.mark.parametrize("S", [1, 7, 49, 64, 65, 196, 1000])
def test_gn_segment_sums_are_exact_on_integers(S):
    rng = np.random.default_rng(S)
    p = rng.integers(-8, 9, size=(3, 5, S)).astype(np.float32)
    assert np.array_equal(gn_segment_sums(p), p.astype(np.float64).sum(axis=2))


def test_gn_vector_segment_sums_order():
    """The "vector" mode adds each vector's 8 values in element order before the lanes: with 2^24
    at element 0 and ones at elements 1..7, every one is lost against 2^24 (2^24 + 1 rounds back
    to 2^24); one value a lane instead keeps six of them (the tree adds lanes 0 and 1 first, which
    loses one, then the other ones in pairs)."""
    p = np.zeros((1, 1, 16), np.float32)
    p[0, 0, 0] = 2.0**24
    p[0, 0, 1:8] = 1.0
    assert gn_segment_sums(p, 8)[0, 0] == 2.0**24
    assert gn_segment_sums(p)[0, 0] == 2.0**24 + 6


@pytest.mark.parametrize("S", [8, 64, 72, 200, 1000, 8192])
def test_gn_vector_segment_sums_are_exact_on_integers(S):
    rng = np.random.default_rng(S + 1)
    p = rng.integers(-8, 9, size=(2, 3, S)).astype(np.float32)
    assert np.array_equal(gn_segment_sums(p, 8), p.astype(np.float64).sum(axis=2))
    assert np.array_equal(gn_segment_sums(p, 4), p.astype(np.float64).sum(axis=2))


@pytest.mark.parametrize("B,C,S,G,dtype,mode", [
    (2, 8, 8192, 2, "bf16", "vector"), (2, 8, 8192, 2, "f32", None),
    (2, 16, 1024, 1, "bf16", "vector"), (2, 16, 1024, 1, "f32", "vector"),
    (2, 16, 1025, 1, "bf16", None), (3, 8, 1025, 1, "bf16", "element"),
    (2, 32, 1024, 1, "bf16", "vector"), (2, 32, 1024, 1, "f32", None),
    (4, 64, 49, 8, "bf16", "element"), (4, 1280, 16, 32, "f32", "vector"),
    (2, 12, 1111, 1, "f16", "element"), (1, 4096, 4, 1, "bf16", None),
    (2, 64, 10, 4, "bf16", "element"), (2, 64, 10, 4, "f32", "element"),
    (2, 64, 12, 4, "f32", "vector"), (1, 8, 4097, 1, "f32", None)])
def test_gn_kernel_modes(B, C, S, G, dtype, mode):
    """Which kernels serve a shape: rows of up to 32768 (float32 16384) 16-byte elements in channels
    of whole vectors ("vector"), up to 16384 (8192) otherwise ("element"), within one chunk of
    spatial size and 144 KiB of backward LDS; the chunked kernels beyond (None)."""
    assert gn_row_kernel_mode(C, S, G, dtype) == mode


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,C,S,G", [(4, 64, 49, 8), (2, 32, 196, 8), (2, 16, 1000, 2),
                                     (2, 16, 1024, 1), (4, 320, 16, 32)])
def test_gn_model_rates_row_kernels(dtype, B, C, S, G):
    """Rows held by one row group (the row kernels' segment sums, by value or by vector)."""
    wl = GN_BASE[dtype]
    inp = make_gn_inputs(wl, B=B, C=C, S=S, seed=B * 1000 + C + S)
    _, mean, rstd = oracle.groupnorm_fwd(inp["x"], inp["w"], inp["b"], G=G, eps=wl.eps,
                                         dtype=dtype)
    rate = gn_dx_model_bitexact(inp["dy"], inp["x"], inp["w"], mean, rstd, G=G, dtype=dtype,
                                rows=True)
    assert rate >= 0.999, rate


def test_gn_row_model_on_integer_inputs_is_exact():
    """Integer x, dy, w with mean 0 and rstd 1: every float32 sum in the row kernels' order is
    exact, so the model's dx equals the oracle's everywhere."""
    rng = np.random.default_rng(4)
    B, C, S, G = 2, 8, 49, 2
    x = rng.integers(-4, 5, size=(B, C, S)).astype(np.float32)
    dy = rng.integers(-4, 5, size=(B, C, S)).astype(np.float32)
    w = rng.integers(1, 4, size=C).astype(np.float32)
    mean = np.zeros((B, G), np.float32)
    rstd = np.ones((B, G), np.float32)
    assert gn_dx_model_bitexact(dy, x, w, mean, rstd, G=G, dtype="bf16", rows=True) == 1.0
    x64 = rng.integers(-4, 5, size=(B, C, 64)).astype(np.float32)
    dy64 = rng.integers(-4, 5, size=(B, C, 64)).astype(np.float32)
    assert gn_dx_model_bitexact(dy64, x64, w, mean, rstd, G=G, dtype="bf16", rows="vector") == 1.0
