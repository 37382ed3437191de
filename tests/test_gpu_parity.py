"""GPU parity: librmsnorm (through its C interface) against the CPU oracle on seeded inputs.

Shapes span several row groups and blocks, ragged row counts (not multiples of the 256 backward
blocks), ragged widths (a partial last 16-byte vector through a padded row stride; widths whose
rows are not 16-byte aligned, which take the element-wise path), single-column rows, and the
widest rows (streaming kernels). Each case also checks that a forward feeding the backward gives
the documented dw, and that repeated runs are bit-identical.
"""
import numpy as np
import pytest

import oracle
from parity import (check_dw, check_dx, check_fwd, same_bits, to_np)
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"
WL = {"f32": WORKLOADS["fp32_64x1024"], "bf16": WORKLOADS["bf16_4096x4096"],
      "f16": WORKLOADS["fp16_8192x8192"]}


def padded(a: np.ndarray, dtype: str, ld: int):
    """Device [M, N] view with row stride ld >= N."""
    M, N = a.shape
    buf = np.zeros((M, ld), np.float32)
    buf[:, :N] = a
    return to_device(buf, dtype, DEV)[:, :N]


def run_case(dtype, M, N, rounding="twice", offset=0.0, eps=1e-6, ld=None, variant="auto",
             seed=1, casts="float32"):
    wl = WL[dtype].with_(rounding=rounding, offset=offset, eps=eps)
    inp = make_inputs(wl, M=M, N=N, seed=seed)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    if ld is None:
        xt, dyt = to_device(x, dtype, DEV), to_device(dy, dtype, DEV)
    else:
        xt, dyt = padded(x, dtype, ld), padded(dy, dtype, ld)
    wt = to_device(w, dtype, DEV)
    print(f"case dtype={dtype} M={M} N={N} ld={ld} rounding={rounding} offset={offset} "
          f"variant={variant} seed={seed} casts={casts}", flush=True)
    # with a padded stride the outputs are padded too, so every operand keeps 16-byte rows
    out = {} if ld is None else {"y": padded(np.zeros((M, N), np.float32), dtype, ld)}
    y, rstd = rn.fwd(xt, wt, eps=eps, offset=offset, rounding=rounding, variant=variant, **out)
    out = {} if ld is None else {"dx": padded(np.zeros((M, N), np.float32), dtype, ld)}
    dx, dw = rn.bwd(dyt, xt, wt, rstd, eps=eps, offset=offset, rounding=rounding,
                    variant=variant, casts=casts, **out)
    torch.cuda.synchronize()
    yg, rg, dxg, dwg = to_np(y), to_np(rstd), to_np(dx), to_np(dw)
    st = check_fwd(yg, rg, x, w, eps=eps, offset=offset, rounding=rounding, dtype=dtype)
    st.update(check_dx(dxg, dy, x, w, rg, offset=offset, dtype=dtype, rounding=rounding,
                       casts=casts))
    st.update(check_dw(dwg, oracle.rmsnorm_dw(dy, x, rg, dtype=dtype, rounding=rounding,
                                              casts=casts)))
    return st, (yg, rg, dxg, dwg)


SHAPES = [
    # (M, N, ld)
    (1, 8, None),
    (5, 1, None),          # single column: element-wise path
    (7, 3, None),          # tiny ragged width: element-wise path
    (33, 64, None),
    (300, 1000, None),     # 125 vectors per row; 300 rows over 256 backward blocks
    (300, 1027, 1032),     # partial last vector through a padded row stride
    (129, 1027, None),     # rows not 16-byte aligned: vectors between an element-wise head and tail
    (257, 3072, None),
    (64, 4096, None),
    (40, 8192, None),
    (20, 16383, None),     # widest row of the 32-column dw reduction, partial last vector
    (24, 16384, None),
    (12, 32768, None),     # LDS-staged backward
    (6, 40000, None),      # streaming backward (beyond the LDS kernel's width)
    (3, 70000, None),      # streaming forward and backward
    (30, 30001, 30008),    # partial last vector through a padded stride, 4 vectors a thread: LDS-staged
    (40, 30001, None),     # wide rows not 16-byte aligned: head/tail peeled, dw sums in LDS
    (10, 40001, None),     # past the LDS sums' reach: element-wise, dw sums in the workspace
]


@pytest.mark.parametrize("M,N,ld", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_parity_shapes_round_twice(dtype, M, N, ld):
    run_case(dtype, M, N, rounding="twice", ld=ld)


@pytest.mark.parametrize("M,N,ld", [(300, 1000, None), (257, 3072, None), (129, 1027, None),
                                    (12, 32768, None), (3, 70000, None), (300, 1027, 1032)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("offset", [0.0, 1.0])
def test_parity_round_once(dtype, M, N, ld, offset):
    run_case(dtype, M, N, rounding="once", offset=offset, ld=ld)


@pytest.mark.parametrize("M,N,ld", [(300, 1000, None), (257, 3072, None), (129, 1027, None),
                                    (40, 8192, None), (24, 16384, None), (12, 32768, None),
                                    (3, 70000, None), (300, 1027, 1032)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_parity_autograd_casts(dtype, M, N, ld):
    run_case(dtype, M, N, rounding="twice", ld=ld, casts="autograd")


# Many rows per backward block: each of the 256 blocks walks its rows in steps of one row group
# (1024 threads: 8, 4, 2 or 1 rows of 1024, 2048, 4096 or 8192 columns), loading the next step's
# rows while it computes the current one. These shapes give every block 7 to 9 steps, the last one
# ragged (M is not a multiple of 256 row groups).
MANY_STEPS = [(3333, 4096), (6200, 2048), (16500, 1024), (2049, 8192)]


@pytest.mark.parametrize("M,N", MANY_STEPS)
@pytest.mark.parametrize("mode", ["twice", "once", "autograd"])
def test_parity_many_rows_per_block(M, N, mode):
    if mode == "autograd":
        run_case("bf16", M, N, rounding="twice", casts="autograd", seed=31)
    else:
        run_case("bf16", M, N, rounding=mode, offset=1.0 if mode == "once" else 0.0, seed=31)


@pytest.mark.parametrize("M,N", [(3333, 4096), (2049, 8192)])
def test_parity_many_rows_per_block_f16(M, N):
    run_case("f16", M, N, rounding="twice", seed=32)


# Narrow rows (at most 32 vectors): the register kernels give each row a segment of 4 to 32 lanes
# (the next power of two of its vector count), 64 / that rows per wavefront. The row counts give
# every backward block several steps of 1024 / lanes rows with a ragged last step, so a
# wavefront's lanes hold rows of the block's share and rows past it.
NARROW = [("bf16", 50152, 128, None),   # 16 lanes, vectors tile the row exactly
          ("bf16", 65869, 64, None),    # 8 lanes
          ("bf16", 131077, 32, None),   # 4 lanes
          ("bf16", 40000, 96, None),    # 12 vectors on 16 lanes
          ("bf16", 20000, 200, None),   # 25 vectors on 32 lanes
          ("f16", 20000, 256, None),    # 32 lanes
          ("f32", 50000, 64, None),     # 16 lanes of 4 floats
          ("f32", 30000, 128, None),    # 32 lanes
          ("bf16", 30000, 128, 136),    # padded row stride
          ("bf16", 30000, 100, 104)]    # partial last vector: whole-wavefront rows


@pytest.mark.parametrize("dtype,M,N,ld", NARROW)
@pytest.mark.parametrize("mode", ["twice", "once", "autograd"])
def test_parity_narrow_rows(dtype, M, N, ld, mode):
    if mode == "autograd":
        run_case(dtype, M, N, rounding="twice", casts="autograd", ld=ld, seed=41)
    else:
        run_case(dtype, M, N, rounding=mode, offset=1.0 if mode == "once" else 0.0, ld=ld, seed=41)


def test_narrow_rows_bench_shape():
    """The benchmark's narrow-row shape at its full size, bf16 65536 x 128, round twice: every
    element against the oracle."""
    run_case("bf16", 65536, 128, seed=43)


@pytest.mark.parametrize("dtype,M,N", [("bf16", 20000, 128), ("bf16", 33000, 64), ("f32", 9000, 64),
                                       ("f16", 7000, 256), ("bf16", 5000, 40)])
def test_narrow_row_segments_match_wavefront_rows(dtype, M, N):
    """A row on a segment of lanes gets, bit for bit, the rstd, y and dx of the same row on a whole
    wavefront (the streaming kernels keep one wavefront per row); dw within float32 rounding (its
    per-block groups are finer)."""
    _, reg = run_case(dtype, M, N, variant="registers", seed=42)
    _, strm = run_case(dtype, M, N, variant="streaming", seed=42)
    for k in range(3):
        assert same_bits(reg[k], strm[k]).all(), k
    assert np.linalg.norm(reg[3] - strm[3]) <= 1e-5 * np.linalg.norm(strm[3])


@pytest.mark.parametrize("dtype,N", [("bf16", 1000), ("f16", 4096), ("bf16", 16384)])
def test_autograd_casts_kernel_families_agree(dtype, N):
    results = {}
    for variant in ("registers", "lds", "streaming"):
        try:
            _, res = run_case(dtype, 70, N, variant=variant, seed=13, casts="autograd")
        except rn.RMSNormError as e:
            assert e.status == 2, e
            continue
        results[variant] = res
    base = results["streaming"]
    for v, res in results.items():
        assert same_bits(res[2], base[2]).all(), v
        assert np.allclose(res[3], base[3], rtol=1e-5, atol=1e-6)


def test_autograd_flag_is_a_noop_for_round_once_and_f32():
    wl = WL["bf16"]
    inp = make_inputs(wl, M=128, N=2048, seed=14)
    for dtype, rounding in (("bf16", "once"), ("f32", "twice")):
        xt, wt, dyt = (to_device(inp[k], dtype, DEV) for k in ("x", "w", "dy"))
        _, r = rn.fwd(xt, wt, rounding=rounding)
        a = rn.bwd(dyt, xt, wt, r, rounding=rounding, casts="float32")
        b = rn.bwd(dyt, xt, wt, r, rounding=rounding, casts="autograd")
        torch.cuda.synchronize()
        for p, q in zip(a, b):
            assert same_bits(to_np(p), to_np(q)).all(), (dtype, rounding)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.25])
def test_parity_eps(eps):
    run_case("bf16", 200, 2048, eps=eps)


@pytest.mark.parametrize("dtype,N", [("bf16", 1000), ("bf16", 3072), ("f16", 4096),
                                     ("f32", 1024), ("bf16", 8192), ("bf16", 16384),
                                     ("f16", 2040)])
def test_kernel_families_agree_bit_for_bit(dtype, N):
    """Register, LDS-staged and streaming kernels share the thread-to-element mapping and the
    summation order, so rstd, y and dx agree bit for bit; dw is bit-identical between the register
    and LDS kernels and within float32 rounding of the streaming one (another row grouping)."""
    results = {}
    for variant in ("registers", "lds", "streaming"):
        try:
            _, res = run_case(dtype, 70, N, variant=variant, seed=3)
        except rn.RMSNormError as e:
            assert e.status == 2, e  # a family that cannot serve this width says so
            continue
        results[variant] = res
    assert "streaming" in results and len(results) >= 2
    base = results["streaming"]
    for v, res in results.items():
        for k in range(3):
            assert same_bits(res[k], base[k]).all(), (v, k)
        assert np.allclose(res[3], base[3], rtol=1e-5, atol=1e-6)
    if "registers" in results and "lds" in results:
        assert same_bits(results["registers"][3], results["lds"][3]).all()


@pytest.mark.parametrize("dtype,N", [("bf16", 32768), ("bf16", 30000), ("f32", 16384),
                                     ("f16", 20000)])
def test_wide_rows_prefetch_pipeline(dtype, N):
    """Rows past the register kernel's reach (2048 vectors) take the LDS-staged backward, which
    loads a block's next row while it works on the current one. 300 rows over 256 blocks give 44
    blocks two rows, so the prefetched rows are used; exactly tiled (32768, f32 16384) and ragged
    widths. Checked against the oracle, and bit for bit against the streaming kernel (same shape,
    same summation order)."""
    _, lds = run_case(dtype, 300, N, variant="lds", seed=21)
    wl = WL[dtype]
    inp = make_inputs(wl, M=300, N=N, seed=21)
    xt, wt, dyt = (to_device(inp[k], dtype, DEV) for k in ("x", "w", "dy"))
    print(f"case streaming dtype={dtype} M=300 N={N}", flush=True)
    y, r = rn.fwd(xt, wt, variant="streaming")
    dx, dw = rn.bwd(dyt, xt, wt, r, variant="streaming")
    torch.cuda.synchronize()
    for k, t in enumerate((y, r, dx)):
        assert same_bits(lds[k], to_np(t)).all(), k
    assert np.allclose(lds[3], to_np(dw), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype,N,ld", [("bf16", 30001, 30008), ("f16", 24577, 24584),
                                       ("bf16", 32767, 32768)])
def test_ragged_wide_rows_lds_matches_streaming(dtype, N, ld):
    """Rows with a partial last vector through a padded stride at 3-4 vectors a thread: AUTO takes
    the LDS-staged backward (RAGGED layout); its dx and dw are bit-identical to the streaming
    kernel's and match the oracle. 70 rows over 70 blocks."""
    _, auto = run_case(dtype, 70, N, ld=ld, seed=24)
    _, lds = run_case(dtype, 70, N, ld=ld, seed=24, variant="lds")
    _, stream = run_case(dtype, 70, N, ld=ld, seed=24, variant="streaming")
    for k in range(3):
        assert same_bits(auto[k], lds[k]).all(), k
        assert same_bits(lds[k], stream[k]).all(), k
    assert same_bits(auto[3], lds[3]).all()
    assert np.allclose(lds[3], stream[3], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype,N", [("bf16", 40000), ("bf16", 57344), ("f16", 65536)])
def test_wide_rows_streaming_register_sums(dtype, N):
    """Rows past the LDS-staged kernel (more than 4096 vectors) take the streaming kernel with the
    dw sums in registers over each block's rows (7-vector instantiation up to 7 vectors a thread,
    8-vector one at 8): 300 rows give 44 blocks two rows."""
    run_case(dtype, 300, N, seed=23)


def strided(a: np.ndarray, dtype: str, ld: int, off: int):
    """Device [M, N] view at column offset `off` of a [M, ld] buffer (its base `off` elements past
    the buffer's, so its rows start off a 16-byte boundary unless off is a multiple of one)."""
    M, N = a.shape
    buf = np.zeros((M, ld), np.float32)
    buf[:, off:off + N] = a
    return to_device(buf, dtype, DEV)[:, off:off + N]


# Layouts of x, dy and dx (and y) for rows that are not 16-byte aligned: (ld, column offset) per
# operand, None for contiguous. Same phase everywhere: every row's head and tail peeled, vectors
# between; an offset base with an aligned stride: the same head in every row; dx (y) at another
# phase: element stores; dy at another phase than x: the element-wise kernels.
UNALIGNED_LAYOUTS = {
    "contiguous": (None, None, None),
    "w_offset": (None, None, None),  # and w one element past a 16-byte boundary
    "offset_base": ((1040, 3), (1040, 3), (1040, 3)),
    "dx_other_phase": (None, None, (1032, 0)),
    "dy_other_phase": (None, (1032, 0), None),
}


@pytest.mark.parametrize("layout", list(UNALIGNED_LAYOUTS))
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_unaligned_row_layouts(dtype, layout):
    M, N = 257, 1027
    lx, ldy, ldx_ = UNALIGNED_LAYOUTS[layout]
    wl = WL[dtype].with_(rounding="twice")
    inp = make_inputs(wl, M=M, N=N, seed=41)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    place = lambda a, l: to_device(a, dtype, DEV) if l is None else strided(a, dtype, *l)
    xt, dyt = place(x, lx), place(dy, ldy)
    yt = place(np.zeros((M, N), np.float32), ldx_)
    dxt = place(np.zeros((M, N), np.float32), ldx_)
    if layout == "w_offset":
        wbuf = to_device(np.concatenate([np.zeros(1, np.float32), w]), dtype, DEV)
        wt = wbuf[1:]
    else:
        wt = to_device(w, dtype, DEV)
    print(f"case unaligned dtype={dtype} layout={layout}", flush=True)
    y, rstd = rn.fwd(xt, wt, y=yt)
    dx, dw = rn.bwd(dyt, xt, wt, rstd, dx=dxt)
    torch.cuda.synchronize()
    rg = to_np(rstd)
    check_fwd(to_np(y), rg, x, w, eps=1e-6, offset=0.0, rounding="twice", dtype=dtype)
    check_dx(to_np(dx), dy, x, w, rg, offset=0.0, dtype=dtype)
    check_dw(to_np(dw), oracle.rmsnorm_dw(dy, x, rg, dtype=dtype))
    # nothing outside the rows was written
    if ldx_ is not None:
        full = dxt.as_strided((M, ldx_[0]), (ldx_[0], 1), dxt.storage_offset() - ldx_[1])
        rest = to_np(full).copy()
        rest[:, ldx_[1]:ldx_[1] + N] = 0
        assert not rest.any()


# Contiguous rows of an odd width, many per block: the peeled register backward (one whole vector
# per lane, 1 to 16 row groups, its ring wrapping over up to 16 steps), against the oracle, both
# rounding modes and the autograd casts; the streaming peeled kernel on the same inputs.
@pytest.mark.parametrize("dtype,M,N,mode", [
    ("bf16", 4096, 4097, "twice"), ("bf16", 4096, 4097, "autograd"), ("f16", 3000, 1027, "once"),
    ("bf16", 2100, 8199, "twice"), ("f32", 2000, 4097, "twice"), ("bf16", 700, 31, "once")])
def test_unaligned_rows_many_per_block(dtype, M, N, mode):
    rounding = "twice" if mode == "autograd" else mode
    casts = "autograd" if mode == "autograd" else "float32"
    wl = WL[dtype].with_(rounding=rounding)
    inp = make_inputs(wl, M=M, N=N, seed=43)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    xt, wt, dyt = (to_device(a, dtype, DEV) for a in (x, w, dy))
    for variant in ("registers", "streaming"):
        print(f"case unaligned many rows dtype={dtype} M={M} N={N} mode={mode} variant={variant}",
              flush=True)
        y, rstd = rn.fwd(xt, wt, rounding=rounding)
        dx, dw = rn.bwd(dyt, xt, wt, rstd, rounding=rounding, casts=casts, variant=variant)
        torch.cuda.synchronize()
        rg = to_np(rstd)
        st = check_dx(to_np(dx), dy, x, w, rg, offset=0.0, dtype=dtype, rounding=rounding,
                      casts=casts)
        st.update(check_dw(to_np(dw), oracle.rmsnorm_dw(dy, x, rg, dtype=dtype, rounding=rounding,
                                                        casts=casts)))
        print(st, flush=True)


def test_forward_register_and_lds_staging_at_wide_rows():
    for variant in ("registers", "lds", "streaming"):
        wl = WL["bf16"]
        inp = make_inputs(wl, M=9, N=32768, seed=4)
        xt, wt = to_device(inp["x"], "bf16", DEV), to_device(inp["w"], "bf16", DEV)
        print(f"case fwd variant={variant} N=32768", flush=True)
        y, r = rn.fwd(xt, wt, variant=variant)
        torch.cuda.synchronize()
        check_fwd(to_np(y), to_np(r), inp["x"], inp["w"], eps=1e-6, offset=0.0,
                  rounding="twice", dtype="bf16")


def test_repeated_runs_are_bit_identical():
    wl = WL["bf16"]
    inp = make_inputs(wl, M=1024, N=4096, seed=5)
    xt, wt, dyt = (to_device(inp[k], "bf16", DEV) for k in ("x", "w", "dy"))
    outs = []
    for _ in range(3):
        y, r = rn.fwd(xt, wt)
        dx, dw = rn.bwd(dyt, xt, wt, r)
        torch.cuda.synchronize()
        outs.append([to_np(t) for t in (y, r, dx, dw)])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert same_bits(a, b).all()


def test_backward_does_not_depend_on_rounding_or_eps_arguments():
    wl = WL["bf16"]
    inp = make_inputs(wl, M=100, N=2048, seed=6)
    xt, wt, dyt = (to_device(inp[k], "bf16", DEV) for k in ("x", "w", "dy"))
    _, r = rn.fwd(xt, wt)
    a = rn.bwd(dyt, xt, wt, r, rounding="twice", eps=1e-6)
    b = rn.bwd(dyt, xt, wt, r, rounding="once", eps=0.5)
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert same_bits(to_np(p), to_np(q)).all()


def test_noncontiguous_gradient_rows():
    """dy given as a row-strided view (a non-contiguous upstream gradient)."""
    wl = WL["bf16"]
    inp = make_inputs(wl, M=96, N=1024, seed=7)
    xt, wt = to_device(inp["x"], "bf16", DEV), to_device(inp["w"], "bf16", DEV)
    big = np.zeros((96, 3072), np.float32)
    big[:, 1024:2048] = inp["dy"]
    dyt = to_device(big, "bf16", DEV)[:, 1024:2048]
    assert dyt.stride(0) == 3072 and not dyt.is_contiguous()
    _, r = rn.fwd(xt, wt)
    dx, dw = rn.bwd(dyt, xt, wt, r)
    torch.cuda.synchronize()
    rg = to_np(r)
    check_dx(to_np(dx), inp["dy"], inp["x"], inp["w"], rg, offset=0.0, dtype="bf16")
    check_dw(to_np(dw), oracle.rmsnorm_dw(inp["dy"], inp["x"], rg))


def test_no_rows():
    xt = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    wt = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    y, r = rn.fwd(xt, wt)
    dw = torch.full((512,), 7.0, device=DEV)
    dx, dw = rn.bwd(xt, xt, wt, r, dw=dw)
    torch.cuda.synchronize()
    assert y.shape == (0, 512) and dx.shape == (0, 512)
    assert (to_np(dw) == 0).all()


def test_rstd_may_be_omitted():
    wl = WL["bf16"]
    inp = make_inputs(wl, M=64, N=4096, seed=8)
    xt, wt = to_device(inp["x"], "bf16", DEV), to_device(inp["w"], "bf16", DEV)
    y1, r = rn.fwd(xt, wt)
    y2, none = rn.fwd(xt, wt, want_rstd=False)
    torch.cuda.synchronize()
    assert none is None and same_bits(to_np(y1), to_np(y2)).all()


def test_nan_and_zero_rows():
    """A NaN poisons its own row only; a zero row with eps = 0 gives rstd = inf and NaN outputs,
    as IEEE arithmetic does on both sides."""
    x = np.ones((4, 256), np.float32)
    x[1, 17] = np.nan
    x[2] = 0.0
    w = np.ones(256, np.float32)
    xt, wt = to_device(x, "bf16", DEV), to_device(w, "bf16", DEV)
    y, r = rn.fwd(xt, wt, eps=0.0)
    torch.cuda.synchronize()
    yg, rg = to_np(y), to_np(r)
    yo, ro = oracle.rmsnorm_fwd(x, w, eps=0.0, dtype="bf16")
    assert same_bits(rg, ro).all()
    assert same_bits(yg, yo).all()
    assert np.isnan(yg[1]).all() and np.isnan(yg[2]).all() and (yg[[0, 3]] == 1.0).all()


def test_conventions_coincide_on_gpu_for_f32_and_unit_gain():
    wl = WL["bf16"]
    inp = make_inputs(wl, M=64, N=2048, seed=9)
    for dtype, w in (("f32", inp["w"]), ("bf16", np.ones(2048, np.float32))):
        xt, wt = to_device(inp["x"], dtype, DEV), to_device(w, dtype, DEV)
        a, _ = rn.fwd(xt, wt, rounding="once")
        b, _ = rn.fwd(xt, wt, rounding="twice")
        torch.cuda.synchronize()
        assert same_bits(to_np(a), to_np(b)).all()


def test_conventions_differ_on_gpu_as_the_oracle_says():
    """Round once and round twice disagree on about a quarter of bf16 outputs, always by one step,
    and on exactly the elements where the oracle's two conventions disagree (given the same rstd)."""
    wl = WL["bf16"]
    inp = make_inputs(wl, M=256, N=4096, seed=10)
    xt, wt = to_device(inp["x"], "bf16", DEV), to_device(inp["w"], "bf16", DEV)
    a, ra = rn.fwd(xt, wt, rounding="once")
    b, rb = rn.fwd(xt, wt, rounding="twice")
    torch.cuda.synchronize()
    a, b, ra = to_np(a), to_np(b), to_np(ra)
    assert same_bits(ra, to_np(rb)).all()
    differ = a != b
    assert 0.15 < differ.mean() < 0.35
    xh = inp["x"] * ra[:, None]
    g = oracle.gain(inp["w"], 0.0)
    oa = oracle.apply_gain(xh, g, rounding="once", dtype="bf16")
    ob = oracle.apply_gain(xh, g, rounding="twice", dtype="bf16")
    assert np.array_equal(differ, oa != ob)


def test_autograd_function_matches_direct_calls():
    wl = WORKLOADS["bf16_16384x3072_gemma"]
    inp = make_inputs(wl, M=96, N=3072, seed=11)
    x = to_device(inp["x"], "bf16", DEV).reshape(4, 24, 3072).requires_grad_(True)
    w = to_device(inp["w"], "bf16", DEV).requires_grad_(True)
    dy = to_device(inp["dy"], "bf16", DEV).reshape(4, 24, 3072)
    y = rn.rms_norm(x, w, 1e-6, 1.0, "once")
    y.backward(dy)
    y2, r = rn.fwd(x.detach().reshape(96, 3072), w.detach(), offset=1.0, rounding="once")
    dx2, dw2 = rn.bwd(dy.reshape(96, 3072), x.detach().reshape(96, 3072), w.detach(), r,
                      offset=1.0)
    torch.cuda.synchronize()
    assert same_bits(to_np(y.reshape(96, 3072)), to_np(y2)).all()
    assert same_bits(to_np(x.grad.reshape(96, 3072)), to_np(dx2)).all()
    assert w.grad.dtype == torch.bfloat16
    assert same_bits(to_np(w.grad), to_np(dw2.to(torch.bfloat16))).all()


def test_autograd_with_a_broadcast_upstream_gradient():
    """The gradient of (y.sum over the leading dims * c).sum() reaches the backward as c broadcast
    over the rows (row stride 0); the wrapper passes a copy with whole rows, so the result equals
    the direct call with the materialized gradient."""
    wl = WL["bf16"]
    inp = make_inputs(wl, M=64, N=1024, seed=13)
    x = to_device(inp["x"], "bf16", DEV).reshape(4, 16, 1024).requires_grad_(True)
    w = to_device(inp["w"], "bf16", DEV).requires_grad_(True)
    c = to_device(inp["dy"][0], "bf16", DEV)
    print("case autograd broadcast upstream bf16 64x1024", flush=True)
    y = rn.rms_norm(x, w)
    strides = []
    y.register_hook(lambda g: strides.append(g.reshape(-1, 1024).stride()))
    (y.sum(dim=(0, 1)) * c).sum().backward()
    assert strides == [(0, 1)]  # the case under test: a row-broadcast upstream gradient
    x2 = x.detach().reshape(64, 1024)
    _, r = rn.fwd(x2, w.detach())
    dx2, dw2 = rn.bwd(c.expand(64, 1024).contiguous(), x2, w.detach(), r)
    torch.cuda.synchronize()
    assert same_bits(to_np(x.grad.reshape(64, 1024)), to_np(dx2)).all()
    assert same_bits(to_np(w.grad), to_np(dw2.to(torch.bfloat16))).all()


def test_graph_replays_match_eager():
    """The benchmark replays the step from a captured graph: every replay (with eager work and
    synchronizations in between) must reproduce the eager results bit for bit."""
    wl = WL["bf16"]
    inp = make_inputs(wl, M=512, N=4096, seed=12)
    xt, wt, dyt = (to_device(inp[k], "bf16", DEV) for k in ("x", "w", "dy"))
    M, N = 512, 4096
    y = torch.empty_like(xt)
    dx = torch.empty_like(xt)
    r = torch.empty(M, dtype=torch.float32, device=DEV)
    dw = torch.empty(N, dtype=torch.float32, device=DEV)
    ws = torch.empty(rn.workspace_bytes(M, N, "bf16") // 4, dtype=torch.float32, device=DEV)

    def step():
        rn.fwd(xt, wt, y=y, rstd=r)
        rn.bwd_rows(dyt, xt, wt, r, ws, dx=dx)
        rn.dw_reduce(ws, dw, M, N, "bf16")

    step()
    torch.cuda.synchronize()
    ref = [to_np(t) for t in (y, r, dx, dw)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (y, r, dx, dw):
            t.fill_(float("nan"))
        _, _ = rn.fwd(xt[:7], wt)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (y, r, dx, dw)):
            assert same_bits(a, to_np(b)).all(), rep


@pytest.mark.parametrize("dtype,off", [("bf16", 1), ("f16", 3), ("f32", 1)])
def test_fwd_output_alignment_only_changes_the_stores(dtype, off):
    """A y that does not allow 16-byte stores (base off by `off` elements) is written element by
    element by the same kernel: y and rstd equal those of an aligned y, bit for bit."""
    wl = WL[dtype]
    M, N = 130, 2048
    inp = make_inputs(wl, M=M, N=N, seed=21)
    xt, wt = to_device(inp["x"], dtype, DEV), to_device(inp["w"], dtype, DEV)
    print(f"case dtype={dtype} M={M} N={N} y offset={off}", flush=True)
    y_a, r_a = rn.fwd(xt, wt)
    buf = torch.zeros(M * N + off + 8, dtype=xt.dtype, device=DEV)
    y_u = buf[off:off + M * N].view(M, N)
    _, r_u = rn.fwd(xt, wt, y=y_u)
    torch.cuda.synchronize()
    assert same_bits(to_np(y_u), to_np(y_a)).all()
    assert same_bits(to_np(r_u), to_np(r_a)).all()
    st = check_fwd(to_np(y_u), to_np(r_u), inp["x"], inp["w"], eps=wl.eps, offset=0.0,
                   rounding="twice", dtype=dtype)
    print(st)
