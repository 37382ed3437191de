"""rmsnorm_bwd_noalloc against rmsnorm_bwd, through the C interface.

The no-allocation entry point runs rmsnorm_bwd's kernels with the dw partial rows in the library's
own device scratch array, so dx and dw must be bit-identical to rmsnorm_bwd with a caller
workspace. Consecutive calls reuse the array: a large call (the largest shape the array holds)
is followed by smaller ones, whose partial rows overwrite only part of what the first left.
"""
import numpy as np
import pytest
import torch

import bwd_precision_numerics_amd as rn
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    a = t.detach().cpu()
    if a.dtype in (torch.bfloat16, torch.float16):
        return a.view(torch.int16).numpy()
    return a.view(torch.int32).numpy()


def _compare(M, N, dtype, rounding, offset, casts, seed):
    print(f"case noalloc M={M} N={N} dtype={dtype} rounding={rounding} offset={offset} "
          f"casts={casts} seed={seed}", flush=True)
    wl = WORKLOADS["bf16_4096x4096"]
    inp = make_inputs(wl, M=max(M, 1), N=N, seed=seed)
    x, w, dy = (to_device(inp[k], dtype, DEV)[:M] if k != "w" else to_device(inp[k], dtype, DEV)
                for k in ("x", "w", "dy"))
    x, dy = x.contiguous(), dy.contiguous()
    _, rstd = rn.fwd(x, w, eps=wl.eps, offset=offset, rounding=rounding)
    lib = rn.library()
    dt = rn.DTYPE_CODES[dtype]
    rc = rn.bwd_rounding_code(rounding, casts)
    stream = torch.cuda.current_stream().cuda_stream
    wsb = rn.workspace_bytes(M, N, dtype)
    ws = torch.empty(max(wsb, 16) // 4, dtype=torch.float32, device=DEV)
    dx_a = torch.empty_like(x)
    dw_a = torch.empty(N, dtype=torch.float32, device=DEV)
    st = lib.rmsnorm_bwd(dy.data_ptr(), N, x.data_ptr(), N, w.data_ptr(), rstd.data_ptr(),
                         dx_a.data_ptr(), N, dw_a.data_ptr(), ws.data_ptr(), wsb, M, N, dt,
                         wl.eps, offset, rc, stream)
    assert st == 0, rn.STATUS_NAMES.get(st, st)
    dx_b = torch.full_like(x, float("nan"))
    dw_b = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    st = lib.rmsnorm_bwd_noalloc(dy.data_ptr(), N, x.data_ptr(), N, w.data_ptr(),
                                 rstd.data_ptr(), dx_b.data_ptr(), N, dw_b.data_ptr(), M, N, dt,
                                 wl.eps, offset, rc, stream)
    assert st == 0, rn.STATUS_NAMES.get(st, st)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(dx_a), _bits(dx_b)), "dx differs from rmsnorm_bwd"
    assert np.array_equal(_bits(dw_a), _bits(dw_b)), "dw differs from rmsnorm_bwd"
    if M == 0:
        assert not dw_b.any()


def test_noalloc_matches_rmsnorm_bwd_on_consecutive_calls():
    # the largest shape the scratch array holds (256 partial rows of 8192 floats = 8 MiB), then
    # smaller ones on the same array
    _compare(4096, 8192, "bf16", "twice", 0.0, "float32", 31)
    _compare(40000, 128, "bf16", "twice", 0.0, "float32", 37)  # narrow rows: 16-lane row groups
    _compare(300, 1000, "bf16", "twice", 0.0, "float32", 32)
    _compare(257, 3072, "bf16", "once", 1.0, "float32", 33)
    _compare(64, 4096, "f16", "twice", 0.0, "autograd", 34)
    _compare(33, 1024, "f32", "twice", 0.0, "float32", 35)
    _compare(0, 512, "bf16", "twice", 0.0, "float32", 36)


def test_noalloc_refuses_shapes_past_its_scratch():
    lib = rn.library()
    N = 16384
    x = torch.zeros((4096, N), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(N, dtype=torch.bfloat16, device=DEV)
    r = torch.ones(4096, dtype=torch.float32, device=DEV)
    dw = torch.empty(N, dtype=torch.float32, device=DEV)
    st = lib.rmsnorm_bwd_noalloc(x.data_ptr(), N, x.data_ptr(), N, w.data_ptr(), r.data_ptr(),
                                 x.data_ptr(), N, dw.data_ptr(), 4096, N, rn.DTYPE_CODES["bf16"],
                                 1e-6, 0.0, rn.ROUNDING_CODES["twice"],
                                 torch.cuda.current_stream().cuda_stream)
    assert rn.STATUS_NAMES[st] == "ERR_WORKSPACE"
