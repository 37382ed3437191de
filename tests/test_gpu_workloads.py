"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Rows are independent, so the oracle recomputes y, rstd and dx for a sample of rows (the first, the
last and seeded random ones, across several backward blocks); dw is checked in full against the
oracle's column sums over every row. The fp16 8192 x 8192 workload (x ~ N(0, 8^2): row sums of
squares beyond the binary16 range) also checks that every output is finite.
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


@pytest.mark.parametrize("name", NAMES)
def test_full_size_workload(name):
    wl = WORKLOADS[name]
    print(f"workload {name}: generating inputs", flush=True)
    inp = make_inputs(wl)
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    xt, wt, dyt = (to_device(a, wl.dtype, DEV) for a in (x, w, dy))
    roundings = [wl.rounding] + ([] if wl.dtype == "f32" else
                                 [r for r in ("once", "twice") if r != wl.rounding])
    for rounding in roundings:
        print(f"workload {name}: rounding={rounding} M={wl.M} N={wl.N}", flush=True)
        y, rstd = rn.fwd(xt, wt, eps=wl.eps, offset=wl.offset, rounding=rounding)
        dx, dw = rn.bwd(dyt, xt, wt, rstd, eps=wl.eps, offset=wl.offset, rounding=rounding)
        torch.cuda.synchronize()
        rows = sample_rows(wl.M)
        rt = torch.from_numpy(rows).to(DEV)
        yg = to_np(y.index_select(0, rt))
        dxg = to_np(dx.index_select(0, rt))
        rg_all = to_np(rstd)
        rg = rg_all[rows]
        st = check_fwd(yg, rg, x[rows], w, eps=wl.eps, offset=wl.offset, rounding=rounding,
                       dtype=wl.dtype)
        st.update(check_dx(dxg, dy[rows], x[rows], w, rg, offset=wl.offset, dtype=wl.dtype))
        st.update(check_dw(to_np(dw), oracle.rmsnorm_dw(dy, x, rg_all)))
        # every row's rstd against the oracle's
        ro = oracle.rstd_of(x, wl.eps)
        d = np.abs(rg_all.astype(np.float64) - ro) / oracle.ulp_of(ro, "f32")
        assert np.all(d <= 8), float(d.max())
        if name.startswith("fp16"):
            assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(dx).all())
            assert bool(torch.isfinite(dw).all())
        print(f"workload {name} {rounding}: {st}", flush=True)
    if wl.dtype != "f32":
        # the autograd-cast backward at full size, round twice
        y, rstd = rn.fwd(xt, wt, eps=wl.eps, offset=wl.offset, rounding="twice")
        dx, dw = rn.bwd(dyt, xt, wt, rstd, eps=wl.eps, offset=wl.offset, rounding="twice",
                        casts="autograd")
        torch.cuda.synchronize()
        rows = sample_rows(wl.M, seed=1)
        rt = torch.from_numpy(rows).to(DEV)
        rg_all = to_np(rstd)
        st = check_dx(to_np(dx.index_select(0, rt)), dy[rows], x[rows], w, rg_all[rows],
                      offset=wl.offset, dtype=wl.dtype, rounding="twice", casts="autograd")
        st.update(check_dw(to_np(dw), oracle.rmsnorm_dw(dy, x, rg_all, dtype=wl.dtype,
                                                        rounding="twice", casts="autograd")))
        print(f"workload {name} autograd casts: {st}", flush=True)
