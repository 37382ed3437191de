"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The bf16 4096 x 4096 and bf16 16384 x 3072 (Gemma-style) workloads are checked on every row. On the
others rows are independent, so the oracle recomputes y, rstd and dx for a sample of rows (the
first, the last and seeded random ones, across several backward blocks). dw is checked in full
against the oracle's column sums over every row, and rstd on every row. The fp16 8192 x 8192
workload (x ~ N(0, 8^2): row sums of squares beyond the binary16 range) also checks that every
output is finite.
"""
import numpy as np
import pytest

import oracle
from parity import check_dw, check_dx, check_fwd, to_np
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bwd_precision_numerics_amd as rn  # noqa: E402

DEV = "cuda:0"
NAMES = [n for n in WORKLOADS]


def sample_rows(M, k=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(min(8, M))) | set(range(max(0, M - 8), M))
    rows |= set(rng.choice(M, size=min(k, M), replace=False).tolist())
    return np.array(sorted(rows))


# Every row of these two is checked (bf16 4096 x 4096 round twice; bf16 16384 x 3072 Gemma-style
# round once with gain 1 + w); the others on sampled rows.
FULL_ROWS = {"bf16_4096x4096", "bf16_16384x3072_gemma"}


def modes(wl):
    """The workload's own rounding first, then the other rounding and the autograd-cast backward
    (round twice) for 16-bit types."""
    if wl.dtype == "f32":
        return [wl.rounding]
    return [wl.rounding] + [r for r in ("once", "twice") if r != wl.rounding] + ["autograd"]


CASES = [(n, m) for n in NAMES for m in modes(WORKLOADS[n])]


@pytest.mark.parametrize("name,mode", CASES)
def test_full_size_workload(name, mode):
    wl = WORKLOADS[name]
    rounding = "twice" if mode == "autograd" else mode
    casts = "autograd" if mode == "autograd" else "float32"
    print(f"workload {name}: generating inputs", flush=True)
    inp = make_inputs(wl)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    xt, wt, dyt = (to_device(a, wl.dtype, DEV) for a in (x, w, dy))
    print(f"workload {name}: mode={mode} M={wl.M} N={wl.N}", flush=True)
    y, rstd = rn.fwd(xt, wt, eps=wl.eps, offset=wl.offset, rounding=rounding)
    dx, dw = rn.bwd(dyt, xt, wt, rstd, eps=wl.eps, offset=wl.offset, rounding=rounding,
                    casts=casts)
    torch.cuda.synchronize()
    rg_all = to_np(rstd)
    if name in FULL_ROWS:
        rows = np.arange(wl.M)
        yg, dxg = to_np(y), to_np(dx)
        xs, dys = x, dy
    else:
        rows = sample_rows(wl.M, seed=modes(wl).index(mode))
        rt = torch.from_numpy(rows).to(DEV)
        yg, dxg = to_np(y.index_select(0, rt)), to_np(dx.index_select(0, rt))
        xs, dys = x[rows], dy[rows]
    rg = rg_all[rows]
    st = check_fwd(yg, rg, xs, w, eps=wl.eps, offset=wl.offset, rounding=rounding, dtype=wl.dtype)
    st.update(check_dx(dxg, dys, xs, w, rg, offset=wl.offset, dtype=wl.dtype, rounding=rounding,
                       casts=casts))
    st.update(check_dw(to_np(dw), oracle.rmsnorm_dw(dy, x, rg_all, dtype=wl.dtype,
                                                    rounding=rounding, casts=casts)))
    # every row's rstd against the oracle's
    ro = oracle.rstd_of(x, wl.eps)
    d = np.abs(rg_all.astype(np.float64) - ro) / oracle.ulp_of(ro, "f32")
    assert np.all(d <= 8), float(d.max())
    if name.startswith("fp16"):
        assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(dx).all())
        assert bool(torch.isfinite(dw).all())
    print(f"workload {name} {mode} ({len(rows)} rows): {st}", flush=True)
