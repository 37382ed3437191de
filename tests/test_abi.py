"""The C interface on the CPU: the library loads, exports every declared symbol, and rejects bad
arguments with the documented status before making any HIP call (no GPU is touched here)."""
import ctypes
import os

import pytest

import bwd_precision_numerics_amd as rn

pytestmark = pytest.mark.skipif(not os.path.exists(rn.LIB_PATH),
                                reason="librmsnorm.so not built (run __graft_entry__.build())")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2
ONCE, TWICE = 0, 1
FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    return rn.library()


def test_exports_every_declared_function(lib):
    declared = rn.header_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(rn.SIGNATURES)


def test_abi_version_and_status_strings(lib):
    assert lib.rmsnorm_abi_version() == 4
    for s in range(6):
        assert lib.rmsnorm_status_string(s)
    assert lib.rmsnorm_status_string(99) == b"unknown status"


def test_workspace_bytes_is_a_pure_function(lib):
    f = lib.rmsnorm_bwd_workspace_bytes
    assert f(4096, 4096, BF16) == 256 * 4096 * 4
    assert f(64, 1024, F32) == 64 * 1024 * 4            # one partial row per row when M < 256
    assert f(300, 1027, F16) == 256 * 1028 * 4           # rows padded to 16 bytes
    assert f(0, 4096, BF16) == 0
    assert f(10, 0, BF16) == 0
    assert f(10, 10, 7) == 0
    assert f(10, (1 << 24) + 1, BF16) == 0


def fwd(lib, x=FAKE, ldx=8, w=FAKE, y=FAKE + 0x1000, ldy=8, rstd=None, M=4, N=8, dtype=BF16,
        eps=1e-6, offset=0.0, rounding=TWICE, variant=0):
    return lib.rmsnorm_fwd_variant(x, ldx, w, y, ldy, rstd, M, N, dtype, eps, offset, rounding,
                                   variant, None)


def bwd(lib, dy=FAKE, lddy=8, x=FAKE + 0x1000, ldx=8, w=FAKE + 0x2000, rstd=FAKE + 0x3000,
        dx=FAKE + 0x4000, lddx=8, dw=FAKE + 0x5000, ws=FAKE + 0x6000, wsb=1 << 20, M=4, N=8,
        dtype=BF16, eps=1e-6, offset=0.0, rounding=TWICE, variant=0):
    return lib.rmsnorm_bwd_variant(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, ws, wsb, M, N, dtype,
                                   eps, offset, rounding, variant, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(M=-1), INVALID), (dict(N=0), INVALID), (dict(ldx=7), INVALID), (dict(ldy=4), INVALID),
    (dict(dtype=3), INVALID), (dict(rounding=2), INVALID), (dict(variant=9), INVALID),
    (dict(eps=-1e-6), INVALID), (dict(eps=float("nan")), INVALID),
    (dict(eps=float("inf")), INVALID), (dict(offset=float("nan")), INVALID),
    (dict(N=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1), UNSUPPORTED),
    (dict(x=FAKE + 1), MISALIGNED), (dict(w=FAKE + 1), MISALIGNED), (dict(y=FAKE + 1), MISALIGNED),
    (dict(rstd=FAKE + 2), MISALIGNED), (dict(dtype=F32, x=FAKE + 2), MISALIGNED),
    (dict(rounding=TWICE | 0x10), INVALID),                  # the autograd flag is backward-only
    (dict(M=2**62, ldx=8), INVALID),                        # row extent overflows int64
    (dict(N=70000, ldx=70000, ldy=70000, variant=1), UNSUPPORTED),  # register kernel too narrow
])
def test_fwd_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status


def fwd8(lib, x=FAKE, ldx=8, w=FAKE, y=FAKE + 0x1000, ldy=8, rstd=None, M=4, N=8, dtype=BF16,
         eps=1e-6, offset=0.0, scale=1.0, fmt=0, variant=0):
    return lib.rmsnorm_fwd_fp8(x, ldx, w, y, ldy, rstd, M, N, dtype, eps, offset, scale, fmt,
                               variant, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(w=None), INVALID),
    (dict(fmt=2), INVALID), (dict(fmt=-1), INVALID), (dict(variant=4), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(eps=-1.0), INVALID), (dict(dtype=5), INVALID), (dict(ldy=7), INVALID),
    (dict(x=FAKE + 1), MISALIGNED), (dict(rstd=FAKE + 2), MISALIGNED),
    (dict(N=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1), UNSUPPORTED),
    # a forced register or LDS kernel needs 16-byte loads of x and w (y's alignment only picks
    # the store width)
    (dict(x=FAKE + 2, variant=1), UNSUPPORTED), (dict(ldx=9, variant=2), UNSUPPORTED),
    (dict(dtype=F32, w=FAKE + 4, variant=1), UNSUPPORTED),
])
def test_fwd_fp8_rejects(lib, kw, status):
    assert fwd8(lib, **kw) == status


def test_fwd_fp8_with_no_rows_is_a_noop(lib):
    assert fwd8(lib, x=None, w=None, y=None, M=0) == OK
    assert fwd8(lib, x=None, w=None, y=None, M=0, fmt=1, scale=-3.0) == OK


def test_bwd_accepts_the_autograd_flag_before_any_hip_call(lib):
    # an otherwise invalid call still fails on the invalid argument, not on the flag
    assert bwd(lib, rounding=TWICE | 0x10, wsb=0) == WORKSPACE
    assert bwd(lib, rounding=ONCE | 0x10, wsb=0) == WORKSPACE


def test_fwd_with_no_rows_is_a_noop(lib):
    # M = 0: nothing to do, no pointers needed, no HIP call made
    assert fwd(lib, x=None, w=None, y=None, M=0) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), INVALID), (dict(x=None), INVALID), (dict(w=None), INVALID),
    (dict(rstd=None), INVALID), (dict(dx=None), INVALID), (dict(dw=None), INVALID),
    (dict(ws=None), INVALID), (dict(lddy=7), INVALID), (dict(ldx=7), INVALID),
    (dict(lddx=7), INVALID), (dict(M=-3), INVALID), (dict(N=0), INVALID),
    (dict(dtype=-1), INVALID), (dict(rounding=5), INVALID), (dict(variant=4), INVALID),
    (dict(rounding=0x12), INVALID), (dict(rounding=0x20 | TWICE), INVALID),
    (dict(eps=float("-inf")), INVALID), (dict(offset=float("inf")), INVALID),
    (dict(wsb=4 * 8 * 4 - 1), WORKSPACE), (dict(wsb=0), WORKSPACE),
    (dict(ws=FAKE + 8), MISALIGNED), (dict(dw=FAKE + 2), MISALIGNED),
    (dict(rstd=FAKE + 1), MISALIGNED), (dict(dx=FAKE + 1), MISALIGNED),
    (dict(N=(1 << 24) + 1, lddy=(1 << 24) + 1, ldx=(1 << 24) + 1, lddx=(1 << 24) + 1),
     UNSUPPORTED),
    (dict(N=40000, lddy=40000, ldx=40000, lddx=40000, wsb=1 << 30, variant=1), UNSUPPORTED),
    (dict(N=70000, lddy=70000, ldx=70000, lddx=70000, wsb=1 << 30, variant=2), UNSUPPORTED),
])
def test_bwd_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_bwd_stages_reject(lib):
    assert lib.rmsnorm_bwd_rows(FAKE, 8, FAKE, 8, FAKE, FAKE, FAKE, 8, FAKE, 16, 4, 8, BF16, 0.0,
                                TWICE, 0, None) == WORKSPACE
    assert lib.rmsnorm_bwd_rows(FAKE, 8, None, 8, FAKE, FAKE, FAKE, 8, FAKE, 1 << 20, 4, 8, BF16,
                                0.0, TWICE, 0, None) == INVALID
    assert lib.rmsnorm_bwd_rows(FAKE, 8, FAKE, 8, FAKE, FAKE, FAKE, 8, FAKE, 1 << 20, 4, 8, BF16,
                                0.0, 0x12, 0, None) == INVALID
    assert lib.rmsnorm_bwd_dw_reduce(FAKE, 1 << 20, None, 4, 8, BF16, None) == INVALID
    assert lib.rmsnorm_bwd_dw_reduce(FAKE + 4, 1 << 20, FAKE, 4, 8, BF16, None) == MISALIGNED
    assert lib.rmsnorm_bwd_dw_reduce(FAKE, 4, FAKE, 4, 8, BF16, None) == WORKSPACE


def test_bwd_noalloc_refuses_before_any_hip_call(lib):
    """The no-allocation backward checks the shape against its scratch array and every argument
    before its first HIP call (the scratch lookup), so these refusals need no GPU."""
    f = lib.rmsnorm_bwd_noalloc
    ok = dict(dy=FAKE, lddy=4096, x=FAKE, ldx=4096, w=FAKE, rstd=FAKE, dx=FAKE, lddx=4096, dw=FAKE,
              M=4096, N=4096, dtype=BF16, eps=1e-6, offset=0.0, rounding=TWICE, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["dy"], a["lddy"], a["x"], a["ldx"], a["w"], a["rstd"], a["dx"], a["lddx"],
                 a["dw"], a["M"], a["N"], a["dtype"], a["eps"], a["offset"], a["rounding"],
                 a["stream"])
    # 256 partial rows of 16384 floats = 16 MiB > the 8 MiB scratch array
    assert call(N=16384, lddy=16384, ldx=16384, lddx=16384) == WORKSPACE
    assert call(M=300, N=8200, lddy=8200, ldx=8200, lddx=8200) == WORKSPACE
    assert call(dw=None) == INVALID
    assert call(rstd=None) == INVALID
    assert call(ldx=100) == INVALID
    assert call(dtype=7) == INVALID
    assert call(N=1 << 25, lddy=1 << 25, ldx=1 << 25, lddx=1 << 25) == UNSUPPORTED
    assert call(dw=FAKE + 2) == MISALIGNED


def test_bandwidth_probe_refuses_before_any_hip_call(lib):
    """The HBM reference kernels' entry point checks kind, pointers, size and alignment first."""
    f = lib.rmsnorm_bandwidth_probe
    assert f(0, FAKE, None, FAKE, 0, None) == OK  # nothing to move: nothing launched
    assert f(9, FAKE, FAKE, FAKE, 4096, None) == INVALID
    assert f(9 | 0x100, FAKE, FAKE, FAKE, 4096, None) == INVALID
    assert f(0, FAKE, None, FAKE, 4100, None) == INVALID
    assert f(0, None, None, FAKE, 4096, None) == INVALID
    assert f(1, FAKE, None, None, 4096, None) == INVALID
    assert f(3, FAKE, None, FAKE, 4096, None) == INVALID
    assert f(2, FAKE + 4, None, FAKE, 4096, None) == MISALIGNED
    assert f(2 | 0x100, FAKE, None, FAKE + 8, 4096, None) == MISALIGNED
    # one word per 512-thread block of two 16-byte vectors per thread
    assert lib.rmsnorm_bandwidth_probe_out_bytes(32 << 20) == ((32 << 20) // 16384) * 4


def test_binding_rejects_host_tensors_before_calling():
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    w = torch.ones(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        rn.fwd(x, w)
    with pytest.raises(TypeError):
        rn.fwd(x.double(), w.double())


def test_binding_refuses_overlapping_rows_and_autograd_copies_them():
    """A broadcast view (row stride 0) or any row stride below N would make the kernels address
    M rows of N elements past the end of the allocation: the binding refuses it before any call,
    and the autograd wrappers, whose upstream gradients are often broadcast views, copy it."""
    import torch
    row = torch.arange(8, dtype=torch.bfloat16).reshape(1, 8)
    for bad in (row.expand(4, 8), torch.zeros(40, dtype=torch.bfloat16).as_strided((4, 8), (4, 1))):
        with pytest.raises(ValueError, match="overlapping rows"):
            rn.fwd(bad, torch.ones(8, dtype=torch.bfloat16))
    g = rn._as_rows(row.expand(2, 3, 8), 8)
    assert g.shape == (6, 8) and g.stride() == (8, 1) and torch.equal(g, row.expand(6, 8))
    ok = torch.zeros(4, 16, dtype=torch.bfloat16)[:, :8]  # padded rows: kept as a view
    assert rn._as_rows(ok, 8).data_ptr() == ok.data_ptr()


def test_binding_checks_caller_outputs_against_the_inputs():
    """Outputs and statistics the caller passes must have the inputs' shape and dtype: a smaller
    buffer would be written or read past its end. Checked on host tensors, before any call."""
    import torch
    bf, f32, f64 = torch.bfloat16, torch.float32, torch.float64
    x = torch.zeros(4, 8, dtype=bf)
    with pytest.raises(ValueError, match="dx must match"):
        rn.softmax_bwd(x, x, dx=torch.zeros(2, 8, dtype=bf))
    xd = torch.zeros(4, 8, dtype=f64)
    wd = torch.ones(8, dtype=f64)
    with pytest.raises(ValueError, match="y must match"):
        rn.fwd_f64(xd, wd, y=torch.zeros(2, 8, dtype=f64))
    with pytest.raises(ValueError, match="dy must have the shape"):
        rn.bwd_f64(torch.zeros(2, 8, dtype=f64), xd, wd, torch.ones(4, dtype=f64))
    with pytest.raises(ValueError, match="dx must match"):
        rn.bwd_f64(xd, xd, wd, torch.ones(4, dtype=f64), dx=torch.zeros(4, 4, dtype=f64))
    xg = torch.zeros(2, 4, 16, dtype=bf)
    wg = torch.ones(4, dtype=bf)
    stats = torch.zeros(2, 2, dtype=f32)
    with pytest.raises(ValueError, match="dx must match"):
        rn.groupnorm_bwd(xg, xg, 2, wg, stats, stats, dx=torch.zeros(2, 4, 8, dtype=bf))
    with pytest.raises(ValueError, match="mean must be float32"):
        rn.groupnorm_bwd(xg, xg, 2, wg, torch.zeros(2, dtype=f32), stats)
    with pytest.raises(ValueError, match="rstd must be float32"):
        rn.groupnorm_bwd(xg, xg, 2, wg, stats, torch.zeros(3, 2, dtype=f32))
    with pytest.raises(TypeError, match="dw must be float32"):
        rn.dw_reduce(torch.zeros(64, dtype=f32), torch.zeros(8, dtype=bf), 4, 8, "bf16")


class _OnDevice:
    """A host tensor presented as a GPU tensor on `device`: the binding's workspace check looks
    only at these attributes, so its refusals can be exercised without a GPU."""

    def __init__(self, t, device="cuda:0"):
        import torch
        self._t, self.is_cuda, self.device = t, True, torch.device(device)

    def __getattr__(self, name):
        return getattr(self._t, name)


def test_binding_checks_caller_workspaces():
    """A workspace the caller passes must be a contiguous GPU tensor on the inputs' device, and the
    size reported to the library is what its storage holds from its first byte: an expanded view
    of 4 bytes must not be reported as 256 KiB (the kernels would write the partial rows past it)."""
    import torch
    dev = torch.device("cuda:0")
    with pytest.raises(ValueError, match="GPU tensor"):
        rn._ws_buffer(torch.zeros(64), dev)
    with pytest.raises(ValueError, match="contiguous"):
        rn._ws_buffer(_OnDevice(torch.zeros(1).expand(65536)), dev)
    with pytest.raises(ValueError, match="contiguous"):
        rn._ws_buffer(_OnDevice(torch.zeros(8, 8).t()), dev)
    with pytest.raises(ValueError, match="is on cuda:1"):
        rn._ws_buffer(_OnDevice(torch.zeros(64), "cuda:1"), dev)
    base = torch.zeros(64)
    ptr, n = rn._ws_buffer(_OnDevice(base), dev)
    assert (ptr, n) == (base.data_ptr(), 256)
    ptr, n = rn._ws_buffer(_OnDevice(base[48:]), dev)  # a view: its own 16 floats, not the rest
    assert (ptr, n) == (base[48:].data_ptr(), 64)


def test_binding_signatures_match_the_header():
    """Each ctypes signature has as many arguments as the header's prototype."""
    import re
    text = rn.header_text()
    for name, (_, args) in rn.SIGNATURES.items():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)", text)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), (name, params)


def lnf(lib, x=FAKE, ldx=8, w=FAKE, b=None, y=FAKE + 0x1000, ldy=8, mean=None, rstd=None, M=4,
        N=8, dtype=BF16, eps=1e-5, variant=0):
    return lib.layernorm_fwd(x, ldx, w, b, y, ldy, mean, rstd, M, N, dtype, eps, variant, None)


def lnb(lib, dy=FAKE, lddy=8, x=FAKE + 0x1000, ldx=8, w=FAKE + 0x2000, mean=FAKE + 0x3000,
        rstd=FAKE + 0x3800, dx=FAKE + 0x4000, lddx=8, dw=FAKE + 0x5000, db=None, ws=FAKE + 0x6000,
        wsb=1 << 20, M=4, N=8, dtype=BF16, variant=0):
    return lib.layernorm_bwd(dy, lddy, x, ldx, w, mean, rstd, dx, lddx, dw, db, ws, wsb, M, N,
                             dtype, variant, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(M=-1), INVALID), (dict(N=0), INVALID), (dict(ldx=7), INVALID), (dict(dtype=3), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(variant=7), INVALID),
    (dict(variant=2), UNSUPPORTED), (dict(b=FAKE + 1), MISALIGNED), (dict(mean=FAKE + 2), MISALIGNED),
    (dict(x=FAKE + 2, variant=1), UNSUPPORTED),
    (dict(N=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1), UNSUPPORTED),
])
def test_layernorm_fwd_rejects(lib, kw, status):
    assert lnf(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), INVALID), (dict(x=None), INVALID), (dict(w=None), INVALID),
    (dict(mean=None), INVALID), (dict(rstd=None), INVALID), (dict(dx=None), INVALID),
    (dict(dw=None), INVALID), (dict(ws=None), INVALID), (dict(lddx=7), INVALID),
    (dict(variant=2), UNSUPPORTED), (dict(wsb=2 * 4 * 8 * 4 - 1), WORKSPACE),
    (dict(db=FAKE + 2), MISALIGNED), (dict(ws=FAKE + 8), MISALIGNED),
    (dict(N=40000, lddy=40000, ldx=40000, lddx=40000, wsb=1 << 30, variant=1), UNSUPPORTED),
])
def test_layernorm_bwd_rejects(lib, kw, status):
    assert lnb(lib, **kw) == status


def test_layernorm_workspace_bytes(lib):
    f = lib.layernorm_bwd_workspace_bytes
    assert f(4096, 4096, BF16) == 2 * 256 * 4096 * 4
    assert f(3, 10, F32) == 2 * 3 * 12 * 4
    assert f(0, 10, F32) == 0 and f(5, 0, F32) == 0 and f(5, 5, 9) == 0


def gnf(lib, x=FAKE, w=FAKE + 0x1000, b=None, y=FAKE + 0x2000, mean=None, rstd=None,
        ws=FAKE + 0x3000, wsb=1 << 20, B=2, C=4, S=8, G=2, dtype=BF16, eps=1e-5):
    return lib.groupnorm_fwd(x, w, b, y, mean, rstd, ws, wsb, B, C, S, G, dtype, eps, None)


def gnb(lib, dy=FAKE, x=FAKE + 0x1000, w=FAKE + 0x2000, mean=FAKE + 0x3000, rstd=FAKE + 0x3800,
        dx=FAKE + 0x4000, dw=FAKE + 0x5000, db=None, ws=FAKE + 0x6000, wsb=1 << 20, B=2, C=4, S=8,
        G=2, dtype=BF16):
    return lib.groupnorm_bwd(dy, x, w, mean, rstd, dx, dw, db, ws, wsb, B, C, S, G, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(ws=None), INVALID), (dict(B=-1), INVALID), (dict(C=0), INVALID), (dict(S=0), INVALID),
    (dict(G=0), INVALID), (dict(G=3), INVALID), (dict(dtype=4), INVALID), (dict(eps=-1.0), INVALID),
    (dict(eps=float("inf")), INVALID), (dict(x=FAKE + 1), MISALIGNED), (dict(b=FAKE + 1), MISALIGNED),
    (dict(mean=FAKE + 2), MISALIGNED), (dict(ws=FAKE + 8), MISALIGNED), (dict(wsb=2 * 4 * 8 - 1), WORKSPACE),
    (dict(C=2, G=1, S=(1 << 23) + 1), UNSUPPORTED),
])
def test_groupnorm_fwd_rejects(lib, kw, status):
    assert gnf(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), INVALID), (dict(x=None), INVALID), (dict(w=None), INVALID),
    (dict(mean=None), INVALID), (dict(rstd=None), INVALID), (dict(dx=None), INVALID),
    (dict(dw=None), INVALID), (dict(G=3), INVALID), (dict(db=FAKE + 2), MISALIGNED),
    (dict(dy=FAKE + 1), MISALIGNED), (dict(wsb=0), WORKSPACE),
])
def test_groupnorm_bwd_rejects(lib, kw, status):
    assert gnb(lib, **kw) == status


def test_groupnorm_workspace_bytes(lib):
    f = lib.groupnorm_workspace_bytes
    assert f(2, 4, 8, 2, BF16) == 2 * 4 * 1 * 8
    assert f(1, 16, 65536, 4, BF16) == 16 * 8 * 8           # 8192-element chunks
    assert f(1, 16, 65536, 4, F32) == 16 * 16 * 8           # 4096-element chunks
    assert f(1, 16, 65537, 4, BF16) == 16 * 9 * 8           # a ragged last chunk
    assert f(0, 4, 8, 2, BF16) == 0
    assert f(2, 4, 8, 3, BF16) == 0 and f(2, 0, 8, 1, BF16) == 0 and f(2, 4, 8, 2, 9) == 0


def test_groupnorm_no_batch_is_a_noop(lib):
    assert gnf(lib, x=None, w=None, y=None, ws=None, B=0) == OK


def smf(lib, x=FAKE, ldx=8, y=FAKE + 0x1000, ldy=8, M=4, N=8, dtype=BF16, variant=0):
    return lib.softmax_fwd(x, ldx, y, ldy, M, N, dtype, variant, None)


def smb(lib, dy=FAKE, lddy=8, y=FAKE + 0x1000, ldy=8, dx=FAKE + 0x2000, lddx=8, M=4, N=8,
        dtype=BF16, variant=0):
    return lib.softmax_bwd(dy, lddy, y, ldy, dx, lddx, M, N, dtype, variant, None)


F64 = 3


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(M=-1), INVALID), (dict(N=0), INVALID),
    (dict(ldx=7), INVALID), (dict(dtype=4), INVALID), (dict(variant=5), INVALID),
    (dict(variant=2), UNSUPPORTED), (dict(x=FAKE + 1), MISALIGNED),
    (dict(dtype=F64, y=FAKE + 4), MISALIGNED), (dict(x=FAKE + 2, variant=1), UNSUPPORTED),
    (dict(N=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1), UNSUPPORTED),
])
def test_softmax_fwd_rejects(lib, kw, status):
    assert smf(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), INVALID), (dict(y=None), INVALID), (dict(dx=None), INVALID),
    (dict(lddy=3), INVALID), (dict(dtype=-2), INVALID), (dict(dy=FAKE + 1), MISALIGNED),
    (dict(variant=2), UNSUPPORTED),
])
def test_softmax_bwd_rejects(lib, kw, status):
    assert smb(lib, **kw) == status


def test_softmax_no_rows_is_a_noop(lib):
    assert smf(lib, x=None, y=None, M=0) == OK
    assert smb(lib, dy=None, y=None, dx=None, M=0, dtype=F64) == OK


def test_f64_dtype_is_rejected_by_the_16_bit_entry_points(lib):
    assert fwd(lib, dtype=F64) == INVALID
    assert lnf(lib, dtype=F64) == INVALID
    assert lib.rmsnorm_bwd_workspace_bytes(4, 8, F64) == 0


def f64f(lib, x=FAKE, ldx=8, w=FAKE + 0x1000, y=FAKE + 0x2000, ldy=8, rstd=None, M=4, N=8,
         eps=1e-6, offset=0.0):
    return lib.rmsnorm_fwd_f64(x, ldx, w, y, ldy, rstd, M, N, eps, offset, None)


def f64b(lib, dy=FAKE, lddy=8, x=FAKE + 0x1000, ldx=8, w=FAKE + 0x2000, rstd=FAKE + 0x3000,
         dx=FAKE + 0x4000, lddx=8, dw=FAKE + 0x5000, ws=FAKE + 0x6000, wsb=1 << 20, M=4, N=8,
         offset=0.0):
    return lib.rmsnorm_bwd_f64(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, ws, wsb, M, N, offset,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID),
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(offset=float("inf")), INVALID),
    (dict(ldy=7), INVALID), (dict(x=FAKE + 4), MISALIGNED), (dict(rstd=FAKE + 4), MISALIGNED),
    (dict(N=(1 << 24) + 1, ldx=(1 << 24) + 1, ldy=(1 << 24) + 1), UNSUPPORTED),
])
def test_rmsnorm_fwd_f64_rejects(lib, kw, status):
    assert f64f(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), INVALID), (dict(rstd=None), INVALID), (dict(dw=None), INVALID),
    (dict(ws=None), INVALID), (dict(wsb=4 * 8 * 8 - 1), WORKSPACE), (dict(ws=FAKE + 8), MISALIGNED),
    (dict(dw=FAKE + 4), MISALIGNED), (dict(offset=float("nan")), INVALID),
])
def test_rmsnorm_bwd_f64_rejects(lib, kw, status):
    assert f64b(lib, **kw) == status


def test_f64_workspace_bytes(lib):
    f = lib.rmsnorm_bwd_f64_workspace_bytes
    assert f(4096, 4096) == 256 * 4096 * 8 and f(3, 5) == 3 * 5 * 8
    assert f(0, 5) == 0 and f(5, 0) == 0
