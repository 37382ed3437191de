"""GPU parity of softmax over the last dimension and of the float64 RMSNorm (through the C
interface) against the CPU oracle.

Softmax: float32 / float16 / bfloat16 / float64, register and streaming kernels (bit-identical),
ragged and misaligned widths (rows not 16-byte aligned: the peeled kernels when every matrix's rows
sit at one offset from a 16-byte boundary, else the element-wise ones), peaked rows (large logits),
rows of -inf but one element, and the backward from the GPU's own forward output. Float64 RMSNorm: forward and backward to the candle
page's 1e-10 bound against the composed float64 formula.
"""
import numpy as np
import pytest

from parity import check_rms_f64, check_softmax_bwd, check_softmax_fwd, same_bits, to_np
from workloads import F64_WORKLOADS, SM_WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"
WL = {"bf16": SM_WORKLOADS["sm_bf16_4096x4096"], "f16": SM_WORKLOADS["sm_f16_4096x4096"],
      "f32": SM_WORKLOADS["sm_f32_64x1024"], "f64": SM_WORKLOADS["sm_f64_1024x4096"]}


def arr(t):
    return t.detach().cpu().numpy() if t.dtype == torch.float64 else to_np(t)


def run_sm(dtype, M, N, variant="auto", seed=1, x=None, ld=None):
    inp = make_inputs(WL[dtype], M=M, N=N, seed=seed)
    x = inp["x"] if x is None else x
    dy = inp["dy"]
    if ld is None:
        xt, dyt = to_device(x, dtype, DEV), to_device(dy, dtype, DEV)
    else:
        bx = np.zeros((M, ld), x.dtype)
        bx[:, :N] = x
        bd = np.zeros((M, ld), dy.dtype)
        bd[:, :N] = dy
        xt, dyt = to_device(bx, dtype, DEV)[:, :N], to_device(bd, dtype, DEV)[:, :N]
    print(f"softmax case dtype={dtype} M={M} N={N} ld={ld} variant={variant} seed={seed}",
          flush=True)
    y = rn.softmax_fwd(xt, variant=variant)
    dx = rn.softmax_bwd(dyt, y, variant=variant)
    torch.cuda.synchronize()
    yg, dxg = arr(y), arr(dx)
    st = check_softmax_fwd(yg, x, dtype=dtype)
    st.update(check_softmax_bwd(dxg, dy, yg, dtype=dtype))
    return st, (yg, dxg)


SHAPES = [(1, 1), (3, 7), (33, 64), (300, 1000), (129, 1027), (257, 3072), (64, 4096),
          (40, 8192), (12, 16384), (5, 32768), (6, 40000), (4, 50264), (3, 70000)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32", "f64"])
def test_softmax_parity(dtype, M, N):
    run_sm(dtype, M, N)


@pytest.mark.parametrize("dtype,N", [("bf16", 40000), ("f16", 50264), ("bf16", 65000)])
def test_softmax_forward_families_agree_on_wide_rows(dtype, N):
    """Forward rows of 5 to 8 vectors a thread that the vectors do not tile: the register kernel
    (partial vector in the last iteration only) and the streaming kernel give the same bits."""
    wl = WL[dtype]
    x = make_inputs(wl, M=9, N=N, seed=8)["x"]
    xt = to_device(x, dtype, DEV)
    print(f"softmax fwd families dtype={dtype} N={N}", flush=True)
    a = rn.softmax_fwd(xt, variant="registers")
    b = rn.softmax_fwd(xt, variant="streaming")
    torch.cuda.synchronize()
    check_softmax_fwd(arr(a), x, dtype=dtype)
    assert same_bits(arr(a), arr(b)).all()


@pytest.mark.parametrize("dtype,N", [("bf16", 40000), ("bf16", 65000), ("f16", 45000),
                                     ("f64", 12000), ("bf16", 50257)])
def test_softmax_backward_families_agree_on_wide_rows(dtype, N):
    """Backward rows of 5 to 8 vectors a thread (float16: 6) in registers at 1024 threads, against
    the streaming kernel (same bits) and the oracle; 50257 also peeled."""
    _, a = run_sm(dtype, 5, N, variant="registers", seed=9)
    _, b = run_sm(dtype, 5, N, variant="streaming", seed=9)
    assert same_bits(a[0], b[0]).all() and same_bits(a[1], b[1]).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_padded_rows(dtype):
    run_sm(dtype, 100, 1000, ld=1032)


@pytest.mark.parametrize("dtype,N", [("bf16", 1000), ("bf16", 4096), ("f16", 8192),
                                     ("f32", 2048), ("f64", 4096)])
def test_softmax_families_agree(dtype, N):
    _, a = run_sm(dtype, 70, N, variant="registers", seed=3)
    _, b = run_sm(dtype, 70, N, variant="streaming", seed=3)
    assert same_bits(a[0], b[0]).all() and same_bits(a[1], b[1]).all()


def test_softmax_peaked_and_infinite_logits():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 2048)) * 30.0).astype(np.float32)
    x[3, :] = -np.inf
    x[3, 17] = 0.0
    xb = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    st, (yg, _) = run_sm("bf16", 64, 2048, x=xb)
    assert yg[3, 17] == 1.0 and np.count_nonzero(yg[3]) == 1


@pytest.mark.parametrize("dtype,N", [("bf16", 4096), ("f32", 2048), ("bf16", 1000), ("bf16", 128),
                                     ("f32", 64), ("bf16", 96)])
def test_softmax_exp_paths(dtype, N):
    """Rows whose span max - min straddles 87 (the bound below which every exp is a normal float32
    and the forward takes its short exp) and rows with -inf: both exp paths against the oracle, on
    full rows (N = 4096 bf16, 2048 f32: the 8-vector register kernel) and ragged ones, with the
    register and streaming kernels bit-identical; a NaN makes its whole row NaN."""
    spans = [1.0, 20.0, 50.0, 86.5, 86.99, 87.0, 87.01, 88.0, 100.0, 120.0, 200.0]
    rng = np.random.default_rng(11)
    rows = []
    for sp in spans:
        for _ in range(3):
            r = rng.uniform(-sp, 0.0, N).astype(np.float32)
            r[rng.integers(N)] = 0.0
            r[rng.integers(N)] = -sp
            rows.append(r + np.float32(rng.uniform(-5, 5)))
    inf_row = rng.standard_normal(N).astype(np.float32)
    inf_row[::7] = -np.inf
    rows.append(inf_row)
    x = np.stack(rows)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    M = x.shape[0]
    _, a = run_sm(dtype, M, N, variant="registers", x=x)
    _, b = run_sm(dtype, M, N, variant="streaming", x=x)
    assert same_bits(a[0], b[0]).all() and same_bits(a[1], b[1]).all()
    xn = x.copy()
    xn[1, 5] = np.nan
    xt = to_device(xn, dtype, DEV)
    for variant in ("registers", "streaming"):
        y = arr(rn.softmax_fwd(xt, variant=variant)).astype(np.float64)
        assert np.isnan(y[1]).all() and np.isfinite(y[0]).all() and np.isfinite(y[2]).all()


# Narrow rows (at most 32 vectors, float32 compute): the register kernels give each row a segment of
# 4 to 32 lanes, 64 / that rows per wavefront; row counts leave the last block partly empty.
NARROW = [("bf16", 50000, 128, None), ("bf16", 70001, 64, None), ("bf16", 100003, 32, None),
          ("bf16", 30000, 96, None), ("bf16", 20000, 200, None), ("f16", 20000, 256, None),
          ("f32", 40000, 64, None), ("f32", 30000, 128, None), ("bf16", 30000, 128, 136),
          ("f64", 3000, 64, None)]


@pytest.mark.parametrize("dtype,M,N,ld", NARROW)
def test_softmax_narrow_rows(dtype, M, N, ld):
    run_sm(dtype, M, N, ld=ld, seed=12)


def test_softmax_narrow_rows_bench_shape():
    """The benchmark's narrow-row shape at its full size, bf16 65536 x 128."""
    run_sm("bf16", 65536, 128, seed=14)


@pytest.mark.parametrize("dtype,M,N", [("bf16", 20000, 128), ("bf16", 33000, 64),
                                       ("f32", 9000, 64), ("f16", 7000, 256), ("bf16", 5000, 40)])
def test_softmax_narrow_segments_match_wavefront_rows(dtype, M, N):
    """A row on a segment of lanes (register kernels) gets the bits of the same row on a whole
    wavefront (streaming kernels), forward and backward."""
    _, a = run_sm(dtype, M, N, variant="registers", seed=13)
    _, b = run_sm(dtype, M, N, variant="streaming", seed=13)
    assert same_bits(a[0], b[0]).all() and same_bits(a[1], b[1]).all()


# Contiguous rows of an odd width are not 16-byte aligned: whole vectors between a head and a tail
# of single elements (register kernels up to 8 vectors a thread forward, 4 backward; streaming
# beyond: 70001 forward, 50257 and 70001 backward).
UNALIGNED = [("bf16", 129, 1027), ("bf16", 6, 50257), ("f16", 40, 4099), ("f32", 33, 1001),
             ("f64", 17, 1001), ("bf16", 5, 70001), ("f16", 64, 17)]


@pytest.mark.parametrize("dtype,M,N", UNALIGNED)
def test_softmax_unaligned_rows(dtype, M, N):
    run_sm(dtype, M, N, seed=M)


@pytest.mark.parametrize("dtype,N", [("bf16", 1027), ("f16", 30001), ("f32", 1001),
                                     ("f64", 1001)])
def test_softmax_unaligned_families_agree(dtype, N):
    """Peeled rows: the register and streaming kernels give the same bits (head element first in
    a lane's even sum, tail element last in its odd sum, in both)."""
    _, a = run_sm(dtype, 37, N, variant="registers", seed=4)
    _, b = run_sm(dtype, 37, N, variant="streaming", seed=4)
    assert same_bits(a[0], b[0]).all() and same_bits(a[1], b[1]).all()


def test_softmax_unaligned_forward_families_agree_wide():
    """Forward rows of 7 vectors a thread between a head and a tail (50257, the GPT-2 vocabulary)."""
    x = make_inputs(WL["bf16"], M=9, N=50257, seed=8)["x"]
    xt = to_device(x, "bf16", DEV)
    print("softmax fwd families bf16 N=50257 unaligned", flush=True)
    a = rn.softmax_fwd(xt, variant="registers")
    b = rn.softmax_fwd(xt, variant="streaming")
    torch.cuda.synchronize()
    check_softmax_fwd(arr(a), x, dtype="bf16")
    assert same_bits(arr(a), arr(b)).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_unaligned_outputs(dtype):
    """Outputs in padded rows at x's offsets (16 bytes of padding: peeled kernels) must leave the
    padding untouched; outputs one element off x's offsets take the element-wise kernels."""
    M, N = 20, 1027
    inp = make_inputs(WL[dtype], M=M, N=N, seed=6)
    xt, dyt = to_device(inp["x"], dtype, DEV), to_device(inp["dy"], dtype, DEV)
    pad = 16 // xt.element_size()
    for layout in ("padded", "shifted"):
        print(f"softmax unaligned outputs dtype={dtype} layout={layout}", flush=True)
        if layout == "padded":
            ybuf = torch.full((M, N + pad), float("nan"), dtype=xt.dtype, device=DEV)
            dbuf = torch.full((M, N + pad), float("nan"), dtype=xt.dtype, device=DEV)
            y_out, dx_out = ybuf[:, :N], dbuf[:, :N]
        else:
            ybuf = torch.empty(M * N + 1, dtype=xt.dtype, device=DEV)
            dbuf = torch.empty(M * N + 1, dtype=xt.dtype, device=DEV)
            y_out, dx_out = ybuf[1:].view(M, N), dbuf[1:].view(M, N)
        y = rn.softmax_fwd(xt, y=y_out)
        dx = rn.softmax_bwd(dyt, y, dx=dx_out)
        torch.cuda.synchronize()
        yg = arr(y)
        check_softmax_fwd(yg, inp["x"], dtype=dtype)
        check_softmax_bwd(arr(dx), inp["dy"], yg, dtype=dtype)
        if layout == "padded":
            assert torch.isnan(ybuf[:, N:]).all() and torch.isnan(dbuf[:, N:]).all()


def test_softmax_zero_rows():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    assert rn.softmax_fwd(x).shape == (0, 64)
    assert rn.softmax_bwd(x, x).shape == (0, 64)


def test_softmax_full_size_bf16():
    wl = WL["bf16"]
    st, _ = run_sm("bf16", wl.M, wl.N, seed=wl.seed)
    print(st)


def run_f64(M, N, seed=2, eps=1e-6, offset=0.0, ld=None):
    wl = F64_WORKLOADS["f64_4096x4096"]
    inp = make_inputs(wl, M=M, N=N, seed=seed)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    print(f"f64 rmsnorm case M={M} N={N} eps={eps} offset={offset} ld={ld}", flush=True)
    if ld is None:
        xt, dyt = to_device(x, "f64", DEV), to_device(dy, "f64", DEV)
    else:
        bx, bd = np.zeros((M, ld)), np.zeros((M, ld))
        bx[:, :N], bd[:, :N] = x, dy
        xt, dyt = to_device(bx, "f64", DEV)[:, :N], to_device(bd, "f64", DEV)[:, :N]
    wt = to_device(w, "f64", DEV)
    y, rstd = rn.fwd_f64(xt, wt, eps=eps, offset=offset)
    dx, dw = rn.bwd_f64(dyt, xt, wt, rstd, offset=offset)
    torch.cuda.synchronize()
    return check_rms_f64(arr(y), arr(rstd), arr(dx), arr(dw), x, w, dy, eps=eps, offset=offset)


@pytest.mark.parametrize("M,N", [(1, 1), (5, 3), (300, 1000), (129, 1027), (257, 4096),
                                 (24, 16384), (300, 12000), (3, 70000)])  # 12000: register dw sums over two rows per block
def test_rmsnorm_f64_parity(M, N):
    print(run_f64(M, N))


def test_rmsnorm_f64_gemma_offset_and_padding():
    print(run_f64(200, 2048, offset=1.0, eps=1e-5, ld=2056))


def test_rmsnorm_f64_full_size():
    wl = F64_WORKLOADS["f64_4096x4096"]
    print(run_f64(wl.M, wl.N, seed=wl.seed, eps=wl.eps))
