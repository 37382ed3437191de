"""GPU parity of LayerNorm (through the C interface) against the CPU oracle.

Shapes span several row groups and persistent blocks, ragged row counts, ragged widths (partial
last vector through a padded row stride; rows that are not 16-byte aligned, which take the
element-wise kernels), single-column rows, rows whose mean is large against their spread, and
widths past the register kernels (streaming kernels). Each case checks y, mean, rstd, dx, dw and db;
families must agree bit for bit, repeated runs must be bit-identical, and a bias-free call must give
the same dx and dw.
"""
import numpy as np
import pytest

from parity import check_ln_bwd, check_ln_fwd, same_bits, to_np
from workloads import LN_WORKLOADS, make_norm_inputs, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"
WL = {"f32": LN_WORKLOADS["ln_fp32_64x1024"], "bf16": LN_WORKLOADS["ln_bf16_4096x4096"],
      "f16": LN_WORKLOADS["ln_fp16_8192x8192"]}


def padded(a, dtype, ld):
    M, N = a.shape
    buf = np.zeros((M, ld), np.float32)
    buf[:, :N] = a
    return to_device(buf, dtype, DEV)[:, :N]


def run_ln(dtype, M, N, *, ld=None, variant="auto", seed=1, bias=True, x_dist=None, eps=None):
    wl = WL[dtype]
    eps = wl.eps if eps is None else eps
    inp = make_norm_inputs(wl, M=M, N=N, seed=seed, x_dist=x_dist)
    x, w, b, dy = inp["x"], inp["w"], (inp["b"] if bias else None), inp["dy"]
    if ld is None:
        xt, dyt = to_device(x, dtype, DEV), to_device(dy, dtype, DEV)
    else:
        xt, dyt = padded(x, dtype, ld), padded(dy, dtype, ld)
    wt = to_device(w, dtype, DEV)
    bt = to_device(b, dtype, DEV) if bias else None
    print(f"ln case dtype={dtype} M={M} N={N} ld={ld} variant={variant} seed={seed} bias={bias} "
          f"x_dist={x_dist}", flush=True)
    # with a padded stride the outputs are padded too, so every operand keeps 16-byte rows
    out = {} if ld is None else {"y": padded(np.zeros((M, N), np.float32), dtype, ld)}
    y, mean, rstd = rn.layernorm_fwd(xt, wt, bt, eps=eps, variant=variant, **out)
    out = {} if ld is None else {"dx": padded(np.zeros((M, N), np.float32), dtype, ld)}
    dx, dw, db = rn.layernorm_bwd(dyt, xt, wt, mean, rstd, bias=bias, variant=variant, **out)
    torch.cuda.synchronize()
    yg, mg, rg, dxg, dwg = (to_np(t) for t in (y, mean, rstd, dx, dw))
    dbg = to_np(db) if bias else None
    st = check_ln_fwd(yg, mg, rg, x, w, b, eps=eps, dtype=dtype)
    st.update(check_ln_bwd(dxg, dwg, dbg, dy, x, w, mg, rg, dtype=dtype, ld=ld))
    return st, (yg, mg, rg, dxg, dwg, dbg)


SHAPES = [
    (1, 8, None), (5, 1, None), (7, 3, None), (33, 64, None), (300, 1000, None),
    (300, 1027, 1032), (129, 1027, None), (257, 3072, None), (64, 4096, None), (40, 8192, None),
    (24, 16384, None), (12, 32768, None), (3, 70000, None),
    (40, 9001, None),   # rows not 16-byte aligned: element-wise, dw and db sums in LDS
    (12, 30001, None),  # the same past the LDS sums' reach: sums in the workspace
]


@pytest.mark.parametrize("M,N,ld", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_ln_parity(dtype, M, N, ld):
    run_ln(dtype, M, N, ld=ld)


@pytest.mark.parametrize("dtype,M,N", [("bf16", 3333, 4096), ("bf16", 6200, 2048),
                                     ("f16", 2049, 8192), ("bf16", 16500, 1024),
                                     ("bf16", 4096, 4097), ("f16", 3000, 1027),
                                     ("bf16", 2100, 8199)])
def test_ln_many_rows_per_block(dtype, M, N):
    """Blocks of 7 to 9 steps of their row loop (the peeled rows 8 to 16), the next step's rows
    loaded during the current one, with a ragged last step."""
    run_ln(dtype, M, N, seed=33)


# Narrow rows (at most 32 vectors): row groups of 4 to 32 lanes, 64 / that rows per wavefront,
# several backward steps per block with a ragged last one.
NARROW = [("bf16", 50152, 128, None), ("bf16", 65869, 64, None), ("bf16", 131077, 32, None),
          ("bf16", 40000, 96, None), ("bf16", 20000, 200, None), ("f16", 20000, 256, None),
          ("f32", 50000, 64, None), ("f32", 30000, 128, None), ("bf16", 30000, 128, 136),
          ("bf16", 30000, 100, 104)]


@pytest.mark.parametrize("dtype,M,N,ld", NARROW)
def test_ln_narrow_rows(dtype, M, N, ld):
    run_ln(dtype, M, N, ld=ld, seed=34)


def test_ln_narrow_rows_bench_shape():
    """The benchmark's narrow-row shape at its full size, bf16 65536 x 128 with a bias."""
    run_ln("bf16", 65536, 128, seed=36)


@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("dtype,M,N", [("bf16", 20000, 128), ("bf16", 33000, 64),
                                       ("f32", 9000, 64), ("f16", 7000, 256), ("bf16", 5000, 40)])
def test_ln_narrow_segments_match_wavefront_rows(dtype, M, N, bias):
    """Rows on segments of lanes (register kernels) against rows on whole wavefronts (streaming):
    y, mean, rstd and dx bit for bit; dw and db within float32 rounding (finer per-block groups)."""
    _, reg = run_ln(dtype, M, N, variant="registers", seed=35, bias=bias)
    _, stream = run_ln(dtype, M, N, variant="streaming", seed=35, bias=bias)
    for k in range(4):
        assert same_bits(reg[k], stream[k]).all(), k
    for k in ((4, 5) if bias else (4,)):
        assert np.linalg.norm(reg[k] - stream[k]) <= 1e-5 * np.linalg.norm(stream[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N", [1000, 4096, 16384])
def test_ln_large_mean_rows(dtype, N):
    """x ~ 16 + N(0, 1): the variance about the mean must survive (no E[x^2] - mean^2)."""
    run_ln(dtype, 96, N, x_dist=("normal", 16.0, 1.0))


@pytest.mark.parametrize("N", [1000, 4096, 8192])
def test_ln_without_bias(N):
    st, res_nb = run_ln("bf16", 130, N, bias=False, seed=5)
    _, res_b = run_ln("bf16", 130, N, bias=True, seed=5)
    # dx and dw do not depend on the bias
    assert same_bits(res_nb[3], res_b[3]).all() and same_bits(res_nb[4], res_b[4]).all()


@pytest.mark.parametrize("dtype,N", [("bf16", 1000), ("bf16", 4096), ("f16", 8192),
                                     ("f32", 1024), ("bf16", 16384)])
def test_ln_families_agree(dtype, N):
    """Register and streaming kernels share the mapping and summation order: y, mean, rstd and dx
    agree bit for bit; dw and db within float32 rounding (another row grouping)."""
    _, reg = run_ln(dtype, 70, N, variant="registers", seed=3)
    _, stream = run_ln(dtype, 70, N, variant="streaming", seed=3)
    for k in range(4):
        assert same_bits(reg[k], stream[k]).all(), k
    for k in (4, 5):
        assert np.allclose(reg[k], stream[k], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype,N", [("bf16", 20000), ("f16", 32768)])
def test_ln_wide_rows_register_sums(dtype, N):
    """Rows past the register kernel take the streaming kernel with dw and db summed in registers
    over each block's rows: 300 rows over 256 blocks give 44 blocks two rows."""
    run_ln(dtype, 300, N, seed=22)


# Contiguous rows of an odd width are not 16-byte aligned: the forward moves whole vectors between
# an element-wise head and tail (w and b funnel-shifted, or element by element when w and b are not
# 16-byte aligned; y stored as vectors when its rows sit at x's offsets).
@pytest.mark.parametrize("layout", ["contiguous", "w_offset", "y_shifted", "no_bias"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_ln_unaligned_rows(dtype, layout):
    M, N = 257, 1027
    wl = WL[dtype]
    inp = make_norm_inputs(wl, M=M, N=N, seed=12)
    bias = layout != "no_bias"
    x, w, b, dy = inp["x"], inp["w"], (inp["b"] if bias else None), inp["dy"]
    xt, dyt = to_device(x, dtype, DEV), to_device(dy, dtype, DEV)
    if layout == "w_offset":
        wt = to_device(np.concatenate([np.zeros(1, np.float32), w]), dtype, DEV)[1:]
        bt = to_device(np.concatenate([np.zeros(1, np.float32), b]), dtype, DEV)[1:]
    else:
        wt = to_device(w, dtype, DEV)
        bt = to_device(b, dtype, DEV) if bias else None
    out = {}
    if layout == "y_shifted":
        out["y"] = torch.empty(M * N + 1, dtype=xt.dtype, device=DEV)[1:].view(M, N)
    print(f"ln unaligned dtype={dtype} layout={layout}", flush=True)
    y, mean, rstd = rn.layernorm_fwd(xt, wt, bt, eps=wl.eps, **out)
    dx, dw, db = rn.layernorm_bwd(dyt, xt, wt, mean, rstd, bias=bias)
    torch.cuda.synchronize()
    mg, rg = to_np(mean), to_np(rstd)
    st = check_ln_fwd(to_np(y), mg, rg, x, w, b, eps=wl.eps, dtype=dtype)
    # w one element off a 16-byte boundary: the element-wise backward
    mapping = "elementwise" if layout == "w_offset" else None
    st.update(check_ln_bwd(to_np(dx), to_np(dw), to_np(db) if bias else None, dy, x, w, mg, rg,
                           dtype=dtype, mapping=mapping))
    print(st, flush=True)


def test_ln_repeatable():
    _, a = run_ln("bf16", 1000, 4096, seed=9)
    _, b = run_ln("bf16", 1000, 4096, seed=9)
    for u, v in zip(a, b):
        assert same_bits(u, v).all()


def test_ln_eps_zero_and_large():
    run_ln("bf16", 200, 2048, eps=0.0)
    run_ln("bf16", 200, 2048, eps=0.25)


def test_ln_lds_family_is_unsupported():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rn.RMSNormError) as e:
        rn.layernorm_fwd(x, w, variant="lds")
    assert e.value.status == 2


def test_ln_zero_rows():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y, m, r = rn.layernorm_fwd(x, w)
    dx, dw, db = rn.layernorm_bwd(x, x, w, m, r)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and dx.shape == (0, 64)
    assert float(dw.abs().sum()) == 0.0 and float(db.abs().sum()) == 0.0


def test_ln_full_size_bf16():
    wl = LN_WORKLOADS["ln_bf16_4096x4096"]
    st, _ = run_ln("bf16", wl.M, wl.N, seed=wl.seed)
    print(st)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ln_two_value_rows(dtype):
    """Rows of two values: xhat = +-1 up to eps, so dx = rstd * ((gdy - c1) - xhat * c2) cancels to
    rounding noise (it vanishes exactly at eps = 0) and no bit-exact rate applies. Each 16-bit dx
    element must lie within the float32 evaluation error of that expression from the oracle's,
    8 * 2^-24 * rstd * (|gdy| + |c1| + |xhat * c2|), plus one ulp of T; y, dw and db as elsewhere."""
    import oracle
    from parity import check_dw
    M, N, ld = 31, 2, 14
    wl = WL[dtype]
    inp = make_norm_inputs(wl, M=M, N=N, seed=236)
    x, w, b, dy = inp["x"], inp["w"], inp["b"], inp["dy"]
    print(f"ln two-value rows dtype={dtype} M={M} ld={ld}", flush=True)
    xt, dyt = padded(x, dtype, ld), padded(dy, dtype, ld)
    wt, bt = to_device(w, dtype, DEV), to_device(b, dtype, DEV)
    y, mean, rstd = rn.layernorm_fwd(xt, wt, bt, eps=wl.eps,
                                     y=padded(np.zeros((M, N), np.float32), dtype, ld))
    dx, dw, db = rn.layernorm_bwd(dyt, xt, wt, mean, rstd,
                                  dx=padded(np.zeros((M, N), np.float32), dtype, ld))
    torch.cuda.synchronize()
    yg, mg, rg, dxg, dwg, dbg = (to_np(t) for t in (y, mean, rstd, dx, dw, db))
    check_ln_fwd(yg, mg, rg, x, w, b, eps=wl.eps, dtype=dtype)
    dx_o, dw_o, db_o = oracle.layernorm_bwd(dy, x, w, mg, rg, dtype=dtype)
    r = rg.astype(np.float64)[:, None]
    xh = (x.astype(np.float64) - mg.astype(np.float64)[:, None]) * r
    gdy = w.astype(np.float64)[None, :] * dy.astype(np.float64)
    c1 = gdy.mean(axis=1, keepdims=True)
    c2 = (gdy * xh).mean(axis=1, keepdims=True)
    bound = 8 * 2.0**-24 * r * (np.abs(gdy) + np.abs(c1) + np.abs(xh * c2))
    err = np.abs(dxg.astype(np.float64) - dx_o)
    ok = err <= bound + oracle.ulp_of(np.abs(dx_o.astype(np.float64)), dtype)
    assert ok.all(), (np.argwhere(~ok)[:5], float((err / np.maximum(bound, 1e-30)).max()))
    check_dw(dwg, dw_o)
    check_dw(dbg, db_o)
