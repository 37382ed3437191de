"""Graph capture of the widened entry points: LayerNorm, GroupNorm (rows held whole, block and
wavefront chunks), softmax, narrow rows of all three row operations, the FP8-output
forward and the float64 RMSNorm, each forward + backward captured once in a HIP graph and replayed
several times, with unrelated eager work and synchronizations between the replays; every replay
must reproduce the eager results bit for bit (the entry points record kernels only: no memsets, no
allocations, no host synchronization)."""
import numpy as np
import pytest

from parity import same_bits
from workloads import (F64_WORKLOADS, GN_WORKLOADS, LN_WORKLOADS, SM_WORKLOADS, make_gn_inputs,
                       make_inputs, make_norm_inputs, to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"


def host(t):
    return t.detach().cpu().numpy() if t.dtype == torch.float64 else t.detach().float().cpu().numpy()


def replay_matches_eager(step, outs, name):
    step()
    torch.cuda.synchronize()
    ref = [host(t) for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    junk = torch.randn(300, 1000, device=DEV, dtype=torch.bfloat16)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        rn.softmax_fwd(junk)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, t in zip(ref, outs):
            assert same_bits(a, host(t)).all(), (name, rep)


def test_layernorm_graph():
    wl = LN_WORKLOADS["ln_bf16_4096x4096"]
    inp = make_norm_inputs(wl, M=600, N=4096, seed=31)
    x, w, b, dy = (to_device(inp[k], "bf16", DEV) for k in ("x", "w", "b", "dy"))
    y, dx = torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty(600, dtype=torch.float32, device=DEV)
    rstd = torch.empty_like(mean)
    dw = torch.empty(4096, dtype=torch.float32, device=DEV)
    db = torch.empty_like(dw)
    ws = torch.empty(rn.layernorm_workspace_bytes(600, 4096, "bf16") // 4, dtype=torch.float32,
                     device=DEV)

    def step():
        rn.layernorm_fwd(x, w, b, y=y, mean=mean, rstd=rstd)
        rn.layernorm_bwd(dy, x, w, mean, rstd, dx=dx, dw=dw, db=db, workspace=ws)

    replay_matches_eager(step, [y, mean, rstd, dx, dw, db], "layernorm")


@pytest.mark.parametrize("B,C,S,G", [
    (2, 16, 5000, 4),     # rows held whole
    (2, 4, 20000, 2),     # chunks of a block each, three a segment
    (2, 1280, 1024, 32),  # chunks of a wavefront each
])
def test_groupnorm_graph(B, C, S, G):
    wl = GN_WORKLOADS["gn_bf16_1x16x256x256_g4"]
    inp = make_gn_inputs(wl, B=B, C=C, S=S, seed=32)
    x, dy = to_device(inp["x"], "bf16", DEV), to_device(inp["dy"], "bf16", DEV)
    w, b = to_device(inp["w"], "bf16", DEV), to_device(inp["b"], "bf16", DEV)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    mean = torch.empty((B, G), dtype=torch.float32, device=DEV)
    rstd = torch.empty_like(mean)
    dw = torch.empty(C, dtype=torch.float32, device=DEV)
    db = torch.empty_like(dw)
    ws = torch.empty(rn.groupnorm_workspace_bytes(B, C, S, G, "bf16") // 4,
                     dtype=torch.float32, device=DEV)

    def step():
        rn.groupnorm_fwd(x, G, w, b, y=y, mean=mean, rstd=rstd, workspace=ws)
        rn.groupnorm_bwd(dy, x, G, w, mean, rstd, dx=dx, dw=dw, db=db, workspace=ws)

    replay_matches_eager(step, [y, mean, rstd, dx, dw, db], "groupnorm")


@pytest.mark.parametrize("dtype", ["bf16", "f64"])
def test_softmax_graph(dtype):
    wl = SM_WORKLOADS["sm_bf16_4096x4096" if dtype == "bf16" else "sm_f64_1024x4096"]
    inp = make_inputs(wl, M=300, N=3000, seed=33)
    x, dy = to_device(inp["x"], dtype, DEV), to_device(inp["dy"], dtype, DEV)
    y, dx = torch.empty_like(x), torch.empty_like(x)

    def step():
        rn.softmax_fwd(x, y=y)
        rn.softmax_bwd(dy, y, dx=dx)

    replay_matches_eager(step, [y, dx], "softmax")


def test_fp8_forward_graph():
    wl = LN_WORKLOADS["ln_bf16_4096x4096"]
    inp = make_inputs(wl, M=512, N=2048, seed=34)
    x, w = to_device(inp["x"], "bf16", DEV), to_device(inp["w"], "bf16", DEV)
    y8 = torch.empty((512, 2048), dtype=torch.uint8, device=DEV)
    rstd = torch.empty(512, dtype=torch.float32, device=DEV)

    def step():
        rn.fwd_fp8(x, w, scale=0.5, y=y8, rstd=rstd)

    replay_matches_eager(step, [y8, rstd], "fp8")


def test_rmsnorm_f64_graph():
    wl = F64_WORKLOADS["f64_4096x4096"]
    inp = make_inputs(wl, M=700, N=4096, seed=35)
    x, w, dy = (to_device(inp[k], "f64", DEV) for k in ("x", "w", "dy"))
    y, dx = torch.empty_like(x), torch.empty_like(x)
    rstd = torch.empty(700, dtype=torch.float64, device=DEV)
    dw = torch.empty(4096, dtype=torch.float64, device=DEV)
    ws = torch.empty(int(rn.library().rmsnorm_bwd_f64_workspace_bytes(700, 4096)) // 8,
                     dtype=torch.float64, device=DEV)

    def step():
        rn.fwd_f64(x, w, y=y, rstd=rstd)
        rn.bwd_f64(dy, x, w, rstd, dx=dx, dw=dw, workspace=ws)

    replay_matches_eager(step, [y, rstd, dx, dw], "rmsnorm_f64")


def test_autograd_wrappers_equal_direct_calls():
    """layer_norm / group_norm / softmax through torch.autograd give exactly the direct calls'
    outputs and gradients (the wrappers only marshal; 3-D inputs flatten to rows)."""
    g = torch.Generator(device="cpu").manual_seed(36)
    x = torch.randn(4, 50, 768, generator=g).to(torch.bfloat16).to(DEV)
    w = (1 + 0.1 * torch.randn(768, generator=g)).to(torch.bfloat16).to(DEV)
    b = (0.1 * torch.randn(768, generator=g)).to(torch.bfloat16).to(DEV)
    gy = torch.randn(4, 50, 768, generator=g).to(torch.bfloat16).to(DEV)

    xa, wa, ba = (t.clone().requires_grad_(True) for t in (x, w, b))
    ya = rn.layer_norm(xa, wa, ba, eps=1e-5)
    ya.backward(gy)
    y, mean, rstd = rn.layernorm_fwd(x.reshape(-1, 768), w, b, eps=1e-5)
    dx, dw, db = rn.layernorm_bwd(gy.reshape(-1, 768), x.reshape(-1, 768), w, mean, rstd)
    torch.cuda.synchronize()
    assert torch.equal(ya.reshape(-1, 768), y) and torch.equal(xa.grad.reshape(-1, 768), dx)
    assert torch.equal(wa.grad, dw.to(torch.bfloat16)) and torch.equal(ba.grad, db.to(torch.bfloat16))

    xs = x.reshape(4, 8, -1)[:, :, :4800].contiguous()  # [B, C, S] with 8 channels
    wg = (1 + 0.1 * torch.randn(8, generator=g)).to(torch.bfloat16).to(DEV)
    xg, wga = xs.clone().requires_grad_(True), wg.clone().requires_grad_(True)
    yg = rn.group_norm(xg, 4, wga, None)
    gyg = torch.randn(yg.shape, generator=g).to(torch.bfloat16).to(DEV)
    yg.backward(gyg)
    y2, m2, r2 = rn.groupnorm_fwd(xs, 4, wg)
    dx2, dw2, _ = rn.groupnorm_bwd(gyg, xs, 4, wg, m2, r2, bias=False)
    torch.cuda.synchronize()
    assert torch.equal(yg, y2) and torch.equal(xg.grad, dx2)
    assert torch.equal(wga.grad, dw2.to(torch.bfloat16))

    xsm = x.clone().requires_grad_(True)
    ysm = rn.softmax(xsm)
    ysm.backward(gy)
    y3 = rn.softmax_fwd(x.reshape(-1, 768))
    dx3 = rn.softmax_bwd(gy.reshape(-1, 768), y3)
    torch.cuda.synchronize()
    assert torch.equal(ysm.reshape(-1, 768), y3) and torch.equal(xsm.grad.reshape(-1, 768), dx3)


def test_narrow_rows_graph():
    """Rows of 128 bf16 values (16-lane segments): RMSNorm, LayerNorm and softmax forward and
    backward in one graph."""
    M, N = 3000, 128
    inp = make_norm_inputs(LN_WORKLOADS["ln_bf16_4096x4096"], M=M, N=N, seed=34)
    x, w, b, dy = (to_device(inp[k], "bf16", DEV) for k in ("x", "w", "b", "dy"))
    outs = {k: torch.empty_like(x) for k in ("y", "dx", "ly", "ldx", "sy", "sdx")}
    rstd = torch.empty(M, dtype=torch.float32, device=DEV)
    mean, lrstd = torch.empty_like(rstd), torch.empty_like(rstd)
    dw, lw, lb = (torch.empty(N, dtype=torch.float32, device=DEV) for _ in range(3))
    ws = torch.empty(rn.workspace_bytes(M, N, "bf16") // 4, dtype=torch.float32, device=DEV)
    lws = torch.empty(rn.layernorm_workspace_bytes(M, N, "bf16") // 4, dtype=torch.float32,
                      device=DEV)

    def step():
        rn.fwd(x, w, y=outs["y"], rstd=rstd)
        rn.bwd(dy, x, w, rstd, dx=outs["dx"], dw=dw, workspace=ws)
        rn.layernorm_fwd(x, w, b, y=outs["ly"], mean=mean, rstd=lrstd)
        rn.layernorm_bwd(dy, x, w, mean, lrstd, dx=outs["ldx"], dw=lw, db=lb, workspace=lws)
        rn.softmax_fwd(x, y=outs["sy"])
        rn.softmax_bwd(dy, outs["sy"], dx=outs["sdx"])

    replay_matches_eager(step, list(outs.values()) + [rstd, mean, lrstd, dw, lw, lb],
                         "narrow rows")
