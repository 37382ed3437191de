"""GPU parity of the forward with an OCP 8-bit output (e4m3 / e5m2) against the CPU oracle.

y8 = FP8(fl(xhat * g) * scale) with non-saturating round-to-nearest-even. The cases cover both
formats, all three input dtypes, the Gemma gain, scales that push values into the 8-bit
subnormal range and past the largest finite value (NaN for e4m3, inf for e5m2), every kernel
family, ragged widths, padded and odd output strides (element-wise stores), byte-offset outputs,
and the full 4096 x 4096 bf16 size. rstd must equal the T-output forward's bit for bit.
"""
import numpy as np
import pytest

from parity import check_fwd_fp8, same_bits, to_np
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"
WL = {"f32": WORKLOADS["fp32_64x1024"], "bf16": WORKLOADS["bf16_4096x4096"],
      "f16": WORKLOADS["fp16_8192x8192"]}


def y8_values(y):
    """float32 values of an 8-bit tensor (float8 or raw uint8 of the given format)."""
    return to_np(y)


def run_fp8(dtype, M, N, *, fmt="e4m3", scale=1.0, offset=0.0, eps=1e-6, variant="auto",
            seed=3, ldy=None, y_byte_offset=0):
    wl = WL[dtype].with_(offset=offset, eps=eps)
    inp = make_inputs(wl, M=M, N=N, seed=seed)
    x, w = inp["x"], inp["w"]
    xt, wt = to_device(x, dtype, DEV), to_device(w, dtype, DEV)
    print(f"fp8 case dtype={dtype} M={M} N={N} fmt={fmt} scale={scale} offset={offset} "
          f"variant={variant} ldy={ldy} yoff={y_byte_offset}", flush=True)
    y = None
    if ldy is not None or y_byte_offset:
        ld = ldy or N
        raw = torch.zeros(M * ld + y_byte_offset + 16, dtype=torch.uint8, device=DEV)
        y = raw[y_byte_offset:y_byte_offset + M * ld].view(M, ld)[:, :N]
        y = y.view(rn.fp8_torch_dtype(fmt))
    y8, rstd = rn.fwd_fp8(xt, wt, eps=eps, offset=offset, scale=scale, fmt=fmt,
                          variant=variant, y=y)
    torch.cuda.synchronize()
    yg, rg = y8_values(y8), to_np(rstd)
    st = check_fwd_fp8(yg, rg, x, w, eps=eps, offset=offset, scale=scale, fmt=fmt, dtype=dtype)
    # the statistic is the T-output forward's, bit for bit
    _, r_t = rn.fwd(xt, wt, eps=eps, offset=offset, variant=variant)
    assert same_bits(rg, to_np(r_t)).all()
    return st, yg, rg


SHAPES = [(1, 8), (5, 1), (7, 3), (33, 64), (5000, 128), (3001, 96), (300, 1000), (129, 1027),
          (257, 3072), (64, 4096), (24, 16384), (3, 70000)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("M,N", SHAPES)
def test_fp8_shapes_bf16(M, N, fmt):
    run_fp8("bf16", M, N, fmt=fmt)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("M,N", [(33, 64), (300, 1000), (129, 1027), (40, 8192), (3, 70000)])
def test_fp8_other_dtypes(dtype, M, N):
    run_fp8(dtype, M, N, fmt="e4m3", scale=0.75)
    run_fp8(dtype, M, N, fmt="e5m2", scale=3.0)


@pytest.mark.parametrize("fmt,scale", [
    ("e4m3", 2.0**-9),     # most outputs in the e4m3 subnormal range, many flush to zero
    ("e5m2", 2.0**-15),    # e5m2 subnormals
    ("e4m3", 150.0),       # the tails pass 448: NaN
    ("e5m2", 20000.0),     # the tails pass 57344: inf
    ("e4m3", -1.3),        # negative scale flips every sign
    ("e5m2", 0.0),         # all zeros, sign of xhat * g kept
])
def test_fp8_scale_extremes(fmt, scale):
    st, yg, _ = run_fp8("bf16", 256, 2048, fmt=fmt, scale=scale)
    if scale == 150.0:
        assert np.isnan(yg).any()
    if scale == 20000.0:
        assert np.isinf(yg).any()


def test_fp8_gemma_gain():
    run_fp8("bf16", 512, 3072, fmt="e4m3", offset=1.0, scale=0.5)


@pytest.mark.parametrize("variant", ["registers", "lds", "streaming"])
def test_fp8_families_agree(variant):
    _, y_auto, r_auto = run_fp8("bf16", 200, 4096, fmt="e4m3", scale=1.7)
    _, y_v, r_v = run_fp8("bf16", 200, 4096, fmt="e4m3", scale=1.7, variant=variant)
    assert same_bits(y_auto, y_v).all() and same_bits(r_auto, r_v).all()


@pytest.mark.parametrize("ldy,off", [(4104, 0), (4097, 0), (4096, 3), (4096, 4)])
def test_fp8_output_strides_and_offsets(ldy, off):
    # a stride or base that breaks the 8-byte vector store takes the element-wise path
    run_fp8("bf16", 96, 4096, fmt="e4m3", ldy=ldy, y_byte_offset=off)


def test_fp8_uint8_output_buffer():
    wl = WL["bf16"]
    inp = make_inputs(wl, M=64, N=1024, seed=5)
    xt, wt = to_device(inp["x"], "bf16", DEV), to_device(inp["w"], "bf16", DEV)
    y_u8 = torch.empty((64, 1024), dtype=torch.uint8, device=DEV)
    y_f8, _ = rn.fwd_fp8(xt, wt, fmt="e5m2")
    rn.fwd_fp8(xt, wt, fmt="e5m2", y=y_u8)
    torch.cuda.synchronize()
    assert torch.equal(y_u8, y_f8.view(torch.uint8))


def test_fp8_rows_zero_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y8, rstd = rn.fwd_fp8(x, w)
    assert y8.shape == (0, 64) and rstd.shape == (0,)


def test_fp8_full_size_bf16():
    wl = WORKLOADS["bf16_4096x4096"]
    st, _, _ = run_fp8("bf16", wl.M, wl.N, fmt="e4m3", eps=wl.eps, seed=wl.seed)
    print(st)


def test_fp8_matches_the_float32_forward_scaled():
    """Property at any size: for float32 I/O, y8 = FP8(fl(y * scale)) where y is the T-output
    forward's result (the same rstd, and for float32 the output is fl(xhat * g))."""
    wl = WL["f32"]
    inp = make_inputs(wl, M=2048, N=4096, seed=9)
    xt, wt = to_device(inp["x"], "f32", DEV), to_device(inp["w"], "f32", DEV)
    y, _ = rn.fwd(xt, wt)
    for fmt in ("e4m3", "e5m2"):
        y8, _ = rn.fwd_fp8(xt, wt, fmt=fmt, scale=3.0)
        ref = (y * 3.0).to(rn.fp8_torch_dtype(fmt))
        torch.cuda.synchronize()
        assert torch.equal(y8.view(torch.uint8), ref.view(torch.uint8)), fmt
