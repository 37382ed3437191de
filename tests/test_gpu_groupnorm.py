"""GPU parity of GroupNorm (through the C interface) against the CPU oracle.

Cases: the group_norm page's shapes that the oracle finishes in seconds ((1, 16, 256, 256) with 4
groups in bf16 and in float16 with an upstream gradient and weight of ones; (2, 64, 32, 32) with 8
groups and an input offset of 16; (2, 8, 16) with 4 groups in float32), segments that split into
several chunks with a ragged last chunk, spatial sizes that break 16-byte alignment (element-wise
kernels), one channel per group and one group, tiny spatial sizes, and no bias.
"""
import numpy as np
import pytest

from parity import check_gn, same_bits, to_np
from workloads import GN_WORKLOADS, make_gn_inputs, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"
BASE = {"bf16": GN_WORKLOADS["gn_bf16_1x16x256x256_g4"],
        "f16": GN_WORKLOADS["gn_bf16_1x16x256x256_g4"].with_(dtype="f16"),
        "f32": GN_WORKLOADS["gn_f32_2x8x16_g4"]}


def run_gn(wl, B=None, C=None, S=None, G=None, seed=None, bias=True):
    inp = make_gn_inputs(wl, B=B, C=C, S=S, seed=seed)
    G = wl.G if G is None else G
    x, w, b, dy = inp["x"], inp["w"], (inp["b"] if bias else None), inp["dy"]
    Bv, Cv, Sv = x.shape
    print(f"gn case {wl.name} dtype={wl.dtype} B={Bv} C={Cv} S={Sv} G={G} seed={seed} "
          f"bias={bias}", flush=True)
    xt, dyt = to_device(x, wl.dtype, DEV), to_device(dy, wl.dtype, DEV)
    wt = to_device(w, wl.dtype, DEV)
    bt = to_device(b, wl.dtype, DEV) if bias else None
    y, mean, rstd = rn.groupnorm_fwd(xt, G, wt, bt, eps=wl.eps)
    dx, dw, db = rn.groupnorm_bwd(dyt, xt, G, wt, mean, rstd, bias=bias)
    torch.cuda.synchronize()
    out = [to_np(t) for t in (y, mean, rstd, dx, dw)] + [to_np(db) if bias else None]
    st = check_gn(out[0], out[1], out[2], out[3], out[4], out[5], x, w, b, dy, G=G, eps=wl.eps,
                  dtype=wl.dtype)
    return st, out


@pytest.mark.parametrize("name", ["gn_bf16_1x16x256x256_g4", "gn_f16_1x16x256x256_g4_ones",
                                  "gn_bf16_2x64x32x32_g8_offset16", "gn_f32_2x8x16_g4"])
def test_gn_page_shapes(name):
    st, out = run_gn(GN_WORKLOADS[name])
    print(st)
    if name == "gn_f16_1x16x256x256_g4_ones":
        dx, db = out[3], out[5]
        assert np.isfinite(dx).all() and float(np.abs(dx).max()) <= 2.0**-24
        assert np.all(db == 65536.0)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B,C,S,G", [
    (2, 8, 8192, 2),      # one full chunk per segment (16-bit; two for float32)
    (2, 8, 4096, 2),      # 16384-element rows: row kernels (16-bit), chunks (float32)
    (3, 6, 9000, 3),      # two chunks, ragged last chunk
    (2, 4, 20000, 2),     # three chunks (16-bit), ragged last chunk
    (2, 4, 1000, 4),      # one channel per group; S * 2 bytes not a multiple of 16 for 16-bit
    (2, 6, 333, 1),       # one group, odd S: element-wise kernels
    (5, 12, 1, 3),        # one element per channel
    (1, 3, 7, 3),         # one channel per group, tiny S
    (4, 64, 64, 16),
    # rows held by one row group: up to 32768 elements (float32 16384) in channels of whole
    # 16-byte vectors, up to 16384 (8192) otherwise
    (32, 256, 49, 32),    # 7 x 7, 8 channels a group: rows not 16-byte aligned (element-wise)
    (16, 128, 196, 32),   # 14 x 14: 16-byte rows, channels of 24.5 vectors (16-bit)
    (8, 64, 256, 32),     # 16 x 16: per-vector segment sums
    (3, 8, 1024, 1),      # rows of 8192 elements: one vector a lane at 1024 lanes
    (3, 8, 1025, 1),      # one element more: two vectors a lane, a partial one
    (2, 16, 1024, 1),     # 16384 elements: two vectors a lane (float32: four)
    (2, 16, 1025, 1),     # channels of 1025 elements: past the by-value rows, chunked kernels
    (2, 32, 1024, 1),     # 32768 elements: four vectors a lane (float32: chunks)
    (2, 320, 4096, 32),   # 10 channels of 64 x 64 a group (40960-element rows): chunks
    (2, 16, 3000, 1),     # chunks of 3000 elements: half a block's lanes hold a partial last vector
    (2, 16, 2000, 1),     # 16-bit: rows held whole; float32: chunks of half a block
    (2, 640, 1024, 32),   # 20 channels of 32 x 32 a group (20480-element rows)
    (4, 1280, 16, 32),    # 40 channels of 16 elements a group (10240-element rows)
    (17, 512, 512, 64),   # 1088 rows: half the threads a row, two vectors a lane (one round)
    (3, 10, 1111, 2),     # 5555-element rows, not 16-byte aligned: 8 elements a lane
    (2, 12, 1111, 1),     # 13332 elements a row: 16 elements a lane (16-bit)
    (1, 4096, 4, 1),      # 16384 elements in 4096 channels: past the LDS cap, chunked kernels
    (1, 4095, 4, 1),      # the same with 4095 chunks: one wavefront a chunk, an idle last one
    (2, 1280, 1024, 32),  # 40 channels of 32 x 32 a group: chunks of one wavefront each
    (2, 64, 10, 4),       # 10-element channels: vectors straddle channel boundaries
    (2, 64, 4, 2),        # channels narrower than a vector (16-bit)
    (5, 6, 500, 3),       # 1000-element rows, 1000 * 2 bytes a multiple of 16
    (1, 2049, 2100, 3),   # 2049 block chunks of 2100 elements, more than the chip holds at once
])
def test_gn_shapes(dtype, B, C, S, G):
    run_gn(BASE[dtype], B=B, C=C, S=S, G=G, seed=B * 1000 + C + S)


def test_gn_without_bias():
    _, a = run_gn(BASE["bf16"], B=2, C=8, S=2048, G=4, seed=5, bias=False)
    _, b = run_gn(BASE["bf16"], B=2, C=8, S=2048, G=4, seed=5, bias=True)
    assert same_bits(a[3], b[3]).all() and same_bits(a[4], b[4]).all()


@pytest.mark.parametrize("S", [4096, 49])
def test_gn_repeatable(S):
    _, a = run_gn(BASE["bf16"], B=4, C=32, S=S, G=8, seed=7)
    _, b = run_gn(BASE["bf16"], B=4, C=32, S=S, G=8, seed=7)
    for u, v in zip(a, b):
        assert same_bits(u, v).all()


def test_gn_row_kernels_without_bias():
    _, a = run_gn(BASE["bf16"], B=8, C=64, S=49, G=16, seed=6, bias=False)
    _, b = run_gn(BASE["bf16"], B=8, C=64, S=49, G=16, seed=6, bias=True)
    assert same_bits(a[3], b[3]).all() and same_bits(a[4], b[4]).all()


def test_gn_four_dim_input():
    """[B, C, H, W] input flattens its spatial dimensions."""
    wl = BASE["bf16"]
    inp = make_gn_inputs(wl, B=2, C=8, S=64 * 32, seed=11)
    x4 = to_device(inp["x"], "bf16", DEV).reshape(2, 8, 64, 32)
    w = to_device(inp["w"], "bf16", DEV)
    y4, m4, r4 = rn.groupnorm_fwd(x4, 4, w)
    y3, m3, r3 = rn.groupnorm_fwd(x4.reshape(2, 8, -1), 4, w)
    torch.cuda.synchronize()
    assert y4.shape == (2, 8, 64, 32)
    assert same_bits(to_np(y4).reshape(2, 8, -1), to_np(y3)).all()


def test_gn_zero_batch():
    x = torch.empty((0, 8, 16), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(8, dtype=torch.bfloat16, device=DEV)
    y, m, r = rn.groupnorm_fwd(x, 4, w)
    dx, dw, db = rn.groupnorm_bwd(x, x, 4, w, m, r)
    torch.cuda.synchronize()
    assert y.shape == (0, 8, 16) and float(dw.abs().sum()) == 0.0 and float(db.abs().sum()) == 0.0


def test_gn_rows_bench_shape():
    """The benchmark's GroupNorm row of many small channels at its full size: bf16 (8, 640, 32, 32),
    32 groups (20480-element rows held by one row group, per-vector segment sums), every element
    against the oracle."""
    run_gn(GN_WORKLOADS["gn_bf16_8x640x32x32_g32"])


def test_gn_full_size_bench_shape():
    """The shape and launch configuration the benchmark times: bf16 (16, 32, 256, 256), 8 groups,
    with bias. mean and rstd of every row, y and dx on sampled batches (the first, a seeded one and
    the last), dW and dB over the whole batch."""
    import oracle
    from parity import check_dw, check_stats
    wl = GN_WORKLOADS["gn_bf16_16x32x256x256_g8"]
    inp = make_gn_inputs(wl)
    x, w, b, dy = inp["x"], inp["w"], inp["b"], inp["dy"]
    B, C, S, G = wl.B, wl.C, wl.S, wl.G
    print(f"gn full size {wl.name}", flush=True)
    xt, dyt = to_device(x, "bf16", DEV), to_device(dy, "bf16", DEV)
    wt, bt = to_device(w, "bf16", DEV), to_device(b, "bf16", DEV)
    y, mean, rstd = rn.groupnorm_fwd(xt, G, wt, bt, eps=wl.eps)
    dx, dw, db = rn.groupnorm_bwd(dyt, xt, G, wt, mean, rstd)
    torch.cuda.synchronize()
    yg, mg, rg, dxg, dwg, dbg = (to_np(t) for t in (y, mean, rstd, dx, dw, db))
    rows = x.reshape(B * G, -1)
    m_o, r_o = oracle.row_stats(rows, wl.eps)
    st = check_stats(mg.reshape(-1), rg.reshape(-1), m_o, r_o, rows)
    pick = sorted({0, int(np.random.default_rng(7).integers(1, B - 1)), B - 1})
    st.update(check_gn(yg[pick], mg[pick], rg[pick], dxg[pick], None, None, x[pick], w, b,
                       dy[pick], G=G, eps=wl.eps, dtype="bf16"))
    _, dw_o, db_o = oracle.groupnorm_bwd(dy, x, w, mg, rg, G=G, dtype="bf16")
    st.update(check_dw(dwg, dw_o))
    st["db_normwise"] = check_dw(dbg, db_o)["dw_normwise"]
    print(pick, st)
