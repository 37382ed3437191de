#!/usr/bin/env python3
"""RMSNorm forward + backward on one MI355X: achieved HBM bandwidth of the whole step.

A step is one pass of the whole path over one [M, N] batch: the forward (y and the float32 rstd
cache), then the backward (dx and the per-block dw partials, then the fixed-order dw reduction).
Default workload: bf16, M = N = 4096, round twice (Llama convention), eps = 1e-6, seeded synthetic
inputs x ~ N(0,1), w ~ U(0.9,1.1), dy ~ N(0,1).

Measurement:
* Inputs are resident in HBM before timing. The step's buffers rotate over independent buffer
  sets, enough that the x matrices alone span --rotate-mib (default 1 GiB, four times the 256 MiB
  Infinity Cache; 32 sets at 4096 x 4096), and the forward and the backward of one step use sets
  half a rotation apart, so no kernel reads data a recent kernel left in the caches (the outputs are
  written with non-temporal stores and do not displace them either).
* The K timed steps are replayed from a HIP graph captured once (no host launch overhead), with a
  device synchronize before and after; value = K * algorithmic bytes of a step / wall time.
* Algorithmic bytes: forward 2*M*N*s + N*s + 4*M (read x, write y, read w, write rstd); backward
  3*M*N*s + N*s + 4*M + 4*N (read dy and x, write dx, read w and rstd, write dw). The dw partials are
  implementation traffic and are not credited.
* roofline: the dominant kernel is the backward rows kernel. Its per-launch duration comes from HIP
  events recorded on the launch stream around the replays of a graph of K back-to-back launches of
  that kernel alone (over the same rotating sets): the mean over the replays, with median and min
  in kernel_stats_us; achieved = its algorithmic bytes per launch (3*M*N*s + N*s + 4*M) / that
  duration. traffic is the HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
  WRITE_SIZE, scaled by the same counters' reading for the library's copy kernel of known size),
  read from the committed summary under profiles/, and null when the kernel sources have changed
  since that summary was taken.
* ceilings: the library's own HBM reference kernels (rmsnorm_bandwidth_probe: read only, write
  only, copy, two reads + one write; 16-byte non-temporal accesses) over the same rotating
  buffers, timed the same way; the forward is reported as a fraction of the copy (its traffic)
  and the backward rows kernel as a fraction of the two-read-one-write kernel (its traffic).
* cpu_baseline: the CPU oracle (NumPy, one thread) on a bounded sample of the same rows.
* rows: LayerNorm, softmax, GroupNorm and the float64 RMSNorm, forward and backward, timed the same
  way (graph of back-to-back launches over rotating buffers), each with its own CPU oracle sample;
  RMSNorm, LayerNorm and softmax on many narrow rows (bf16 65536 x 128); GroupNorm with many
  channels of a small spatial size (bf16 (8, 640, 32, 32), 32 groups: rows held whole).
* configs: every RMSNorm configuration (fp32 64 x 1024; bf16 4096 x 4096 in the other rounding
  mode; fp16 8192 x 8192; bf16 16384 x 3072 Gemma round once; bf16 M = 4096 hidden-size sweep up to
  N = 32768): step, forward and backward times, GB/s and fraction of peak per phase, on inputs
  drawn on the device with the same distributions.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload NAME] [--rounding once]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD published peak
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_bwd_rows_bf16_4096x4096.md")
KERNEL_SOURCES = [os.path.join(ROOT, "bwd_precision_numerics_amd", "csrc", f) for f in
                  ("librmsnorm.hip", "host_common.hpp", "rmsnorm_common.hpp", "rmsnorm_fwd.hpp",
                   "rmsnorm_bwd.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """Measured HBM bytes per backward-rows launch, if the committed counters match the sources."""
    if workload != "bf16_4096x4096" or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    with open(TRAFFIC_SUMMARY, encoding="utf-8") as f:
        for line in f:
            if line.startswith("traffic:"):
                for kv in line[len("traffic:"):].split():
                    k, _, v = kv.partition("=")
                    vals[k] = v
    if vals.get("sources") != kernel_source_hash() or "bytes_per_launch" not in vals:
        return None
    return float(vals["bytes_per_launch"])


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description="RMSNorm fwd+bwd HBM bandwidth on one MI355X")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: bf16_4096x4096)")
    ap.add_argument("--rounding", choices=["once", "twice"], default=None)
    ap.add_argument("--bwd-casts", choices=["float32", "autograd"], default="float32",
                    help="backward reading: float32 (default) or the autograd casts")
    ap.add_argument("--rotate-mib", type=int, default=1024,
                    help="rotate over enough buffer sets that the x matrices span this many MiB")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch everything eagerly (steps, per-kernel timings, rows) instead "
                         "of replaying graphs, so per-dispatch profiler counters see each launch")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget for the CPU oracle baseline (0 disables it)")
    ap.add_argument("--kernel-only", choices=["fwd", "bwd_rows", "dw_reduce", "fwd_fp8"],
                    default=None,
                    help="launch only this kernel --steps times (for counter collection)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the LayerNorm / GroupNorm measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration RMSNorm sweep")
    ap.add_argument("--ceilings", action="store_true",
                    help="time the library's HBM reference kernels (read, write, copy, two "
                         "reads + one write) at 32 MiB to 1 GiB per stream and exit")
    ap.add_argument("--summarize-trace", metavar="CSV", default=None,
                    help="print per-kernel dispatch statistics (count, mean, median, min, max "
                         "in ns) of a rocprofv3 kernel-trace CSV and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run a reference kernel (--probe-kind, default "
                         "copy) over streams of this many MiB --steps times (the copy calibrates "
                         "the HBM byte counters)")
    ap.add_argument("--probe-kind", choices=["read", "write", "copy", "sum2"], default="copy")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="print per-run, per-kernel means of the rocprofv3 --pmc CSVs under DIR "
                         "(and HBM traffic scaled by the run named copy, whose buffer size "
                         "--copy-probe-mib gives) and exit")
    return ap.parse_args(argv)


class Sets:
    """Rotating device buffer sets and the raw C-interface calls on them."""

    def __init__(self, rn, torch, wl, rounding, inp, nsets, device, casts="float32"):
        from workloads import to_device
        self.rn, self.torch, self.wl, self.rounding = rn, torch, wl, rounding
        self.lib = rn.library()
        M, N = wl.M, wl.N

        def dev(a):  # host arrays of T values, or tensors already on the device
            return a.contiguous() if isinstance(a, torch.Tensor) else to_device(a, wl.dtype,
                                                                                  device)
        x0, dy0, self.w = dev(inp["x"]), dev(inp["dy"]), dev(inp["w"])
        self.sets = []
        for _ in range(nsets):
            s = {"x": x0.clone(), "dy": dy0.clone(),
                 "y": torch.empty_like(x0), "dx": torch.empty_like(x0),
                 "rstd": torch.empty(M, dtype=torch.float32, device=device),
                 "y8": torch.empty((M, N), dtype=torch.uint8, device=device),
                 "dw": torch.empty(N, dtype=torch.float32, device=device)}
            self.sets.append(s)
        del x0, dy0
        self.wsb = rn.workspace_bytes(M, N, wl.dtype)
        self.ws = torch.empty(max(self.wsb, 16) // 4, dtype=torch.float32, device=device)
        self.dt = rn.DTYPE_CODES[wl.dtype]
        self.rc = rn.ROUNDING_CODES[rounding]
        self.bwd_rc = rn.bwd_rounding_code(rounding, casts)

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def fwd(self, i):
        s, wl = self.sets[i], self.wl
        st = self.lib.rmsnorm_fwd(s["x"].data_ptr(), wl.N, self.w.data_ptr(), s["y"].data_ptr(),
                                  wl.N, s["rstd"].data_ptr(), wl.M, wl.N, self.dt, wl.eps,
                                  wl.offset, self.rc, self.stream())
        if st:
            raise RuntimeError(f"rmsnorm_fwd status {st}")

    def fwd_fp8(self, i):
        """The forward with an e4m3 output (scale 1), same input and rstd cache."""
        s, wl = self.sets[i], self.wl
        st = self.lib.rmsnorm_fwd_fp8(s["x"].data_ptr(), wl.N, self.w.data_ptr(),
                                      s["y8"].data_ptr(), wl.N, s["rstd"].data_ptr(), wl.M, wl.N,
                                      self.dt, wl.eps, wl.offset, 1.0,
                                      self.rn.FP8_CODES["e4m3"], 0, self.stream())
        if st:
            raise RuntimeError(f"rmsnorm_fwd_fp8 status {st}")

    def bwd_rows(self, i):
        s, wl = self.sets[i], self.wl
        st = self.lib.rmsnorm_bwd_rows(s["dy"].data_ptr(), wl.N, s["x"].data_ptr(), wl.N,
                                       self.w.data_ptr(), s["rstd"].data_ptr(), s["dx"].data_ptr(),
                                       wl.N, self.ws.data_ptr(), self.wsb, wl.M, wl.N, self.dt,
                                       wl.offset, self.bwd_rc, 0, self.stream())
        if st:
            raise RuntimeError(f"rmsnorm_bwd_rows status {st}")

    def dw_reduce(self, i):
        s, wl = self.sets[i], self.wl
        st = self.lib.rmsnorm_bwd_dw_reduce(self.ws.data_ptr(), self.wsb, s["dw"].data_ptr(), wl.M,
                                            wl.N, self.dt, self.stream())
        if st:
            raise RuntimeError(f"rmsnorm_bwd_dw_reduce status {st}")

    def step(self, k):
        """Forward on one set, backward on the set half a rotation away."""
        n = len(self.sets)
        a, b = k % n, (k + n // 2) % n
        self.fwd(a)
        self.bwd_rows(b)
        self.dw_reduce(b)


def copy_probe(torch, rn, mib, steps, kind="copy"):
    """One of the library's reference kernels (default: copy) over streams of `mib` MiB, `steps`
    times: the known-size reference that calibrates the HBM byte counters, and the ceiling kernels
    for issue and occupancy counters."""
    nbytes = mib * 2**20
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.ones_like(a) if kind == "sum2" else None
    c = torch.empty_like(a) if kind != "read" else torch.empty(
        rn.library().rmsnorm_bandwidth_probe_out_bytes(nbytes) // 4 + 1, dtype=torch.float32,
        device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    moved = {"read": 1, "write": 1, "copy": 2, "sum2": 3}[kind] * nbytes
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        probe_call(rn, kind, None if kind == "write" else a.data_ptr(),
                   None if b is None else b.data_ptr(), c.data_ptr(), nbytes, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t
    print(json.dumps({"probe": kind, "bytes_per_launch": moved, "launches": steps,
                      "GBps": moved * steps / dt / 1e9}), flush=True)


def summarize_counters(folder, copy_mib):
    """Per (run, kernel, grid size) means of every counter in the rocprofv3 --pmc CSVs under
    `folder` (one run per `<run>_counter_collection.csv`). With FETCH_SIZE and WRITE_SIZE present and a run
    named `copy` (the library's copy kernel over one buffer of `copy_mib` MiB, --copy-probe-mib),
    also the traffic in bytes: each counter scaled by the factor that maps its copy reading to the
    copy's true bytes (one buffer read, one written)."""
    import csv
    import glob
    vals = {}
    for path in sorted(glob.glob(os.path.join(folder, "**", "*_counter_collection.csv"),
                                 recursive=True)):
        run = os.path.basename(path)[:-len("_counter_collection.csv")]
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                # one kernel launched at several sizes is told apart by its grid size
                kern = f'{r["Kernel_Name"]} [grid {r.get("Grid_Size", "?")}]'
                key = (run, kern, r["Counter_Name"])
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    means = {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}
    for (run, kern, ctr), (m, n) in sorted(means.items()):
        print(json.dumps({"run": run, "kernel": kern, "counter": ctr, "dispatches": n,
                          "mean": round(m, 3)}))
    copies = {ctr: m for (run, kern, ctr), (m, n) in means.items()
              if run == "copy" and "copy_kernel" in kern}
    if "FETCH_SIZE" in copies and "WRITE_SIZE" in copies and copy_mib:
        true = copy_mib * 2.0**20
        fs = true / (copies["FETCH_SIZE"] * 1024.0)
        ws = true / (copies["WRITE_SIZE"] * 1024.0)
        print(json.dumps({"calibration": {"FETCH_SIZE_KiB": round(copies["FETCH_SIZE"], 1),
                                          "WRITE_SIZE_KiB": round(copies["WRITE_SIZE"], 1),
                                          "true_bytes": int(true), "fetch_scale": round(fs, 4),
                                          "write_scale": round(ws, 4)}}))
        for (run, kern, ctr), (m, n) in sorted(means.items()):
            if ctr != "FETCH_SIZE" or run == "copy":
                continue
            w = means.get((run, kern, "WRITE_SIZE"))
            if w is None:
                continue
            rb, wb = m * 1024.0 * fs, w[0] * 1024.0 * ws
            print(json.dumps({"run": run, "kernel": kern, "read_bytes": round(rb),
                              "write_bytes": round(wb), "traffic_bytes": round(rb + wb)}))


def summarize_trace(path):
    """Per-kernel dispatch statistics of a rocprofv3 kernel-trace CSV (durations in ns)."""
    import csv
    by = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name")
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            by.setdefault(name, []).append(d)
    rows = []
    for name, v in by.items():
        v.sort()
        n = len(v)
        med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
        rows.append({"kernel": name, "count": n, "mean_ns": round(sum(v) / n, 1),
                     "median_ns": med, "min_ns": v[0], "max_ns": v[-1]})
    rows.sort(key=lambda r: -r["mean_ns"] * r["count"])
    for r in rows:
        print(json.dumps(r))


class Eager:
    """Stands in for a captured graph under --no-graph: replay() makes the calls directly on the
    current stream, so a profiler that counts per dispatch sees every launch."""

    def __init__(self, fn, count):
        self.fn, self.count = fn, count

    def replay(self):
        for k in range(self.count):
            self.fn(k)


EAGER = False  # set by --no-graph


def capture(torch, fn, count):
    """A graph of `count` back-to-back calls fn(0), fn(1), ... on the capture stream (direct calls
    under --no-graph)."""
    if EAGER:
        fn(0)
        torch.cuda.synchronize()
        return Eager(fn, count)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(count):
            fn(k)
    g.replay()  # first replay is untimed
    torch.cuda.synchronize()
    return g


def kernel_durations(torch, sets, launches):
    """Per-launch duration of each kernel: events on the launch stream around the replays of a
    graph of `launches` back-to-back launches of that kernel alone over the rotating sets.
    Returns ({kernel: mean seconds per launch over all replays}, {kernel: mean/median/min in
    us over the replays})."""
    mean, stats = {}, {}
    n = len(sets.sets)
    for name, fn in (("fwd", sets.fwd), ("bwd_rows", sets.bwd_rows),
                     ("dw_reduce", sets.dw_reduce), ("fwd_fp8", sets.fwd_fp8)):
        t = graph_stats(torch, lambda k: fn(k % n), launches)
        stats[name] = summary(t)
        mean[name] = sum(t) / len(t)
    return mean, stats


PROBE_BYTES = {"read": 1, "write": 1, "copy": 2, "sum2": 3}  # streams moved per probe launch


def probe_call(rn, kind, a, b, c, nbytes, stream, cached=False):
    code = rn.PROBE_CODES[kind] | (rn.PROBE_CACHED_STORES if cached else 0)
    st = rn.library().rmsnorm_bandwidth_probe(code, a, b, c, nbytes, stream)
    if st:
        raise RuntimeError(f"rmsnorm_bandwidth_probe status {st}")


def probe_ceilings(torch, rn, streams, nbytes, launches, cached_too=False):
    """The library's HBM reference kernels (read, write, copy, two reads + one write; with
    `cached_too` also with plain stores) over the rotating buffers `streams` = [(a, b, c), ...] of
    `nbytes` each, timed like the RMSNorm kernels (graph of back-to-back launches rotating through
    the buffers), and an empty launch. GB/s counts every stream."""
    n = len(streams)
    out_words = torch.empty(max(rn.library().rmsnorm_bandwidth_probe_out_bytes(nbytes), 16) // 4,
                            dtype=torch.int32, device="cuda:0")
    res = {}
    kinds = [("read", False), ("write", False), ("copy", False), ("sum2", False)]
    if cached_too:
        kinds += [("write", True), ("copy", True), ("sum2", True)]
    for kind, cached in kinds:
        def fn(k, kind=kind, cached=cached):
            a, b, c = streams[k % n]
            stream = torch.cuda.current_stream().cuda_stream
            if kind == "read":
                probe_call(rn, kind, a.data_ptr(), None, out_words.data_ptr(), nbytes, stream)
            else:
                probe_call(rn, kind, a.data_ptr(), b.data_ptr(), c.data_ptr(), nbytes, stream,
                           cached)
        t = graph_stats(torch, fn, launches)
        med = sorted(t)[len(t) // 2]
        moved = PROBE_BYTES[kind] * nbytes
        res[kind + ("_cached_stores" if cached else "")] = {
            "GBps": round(moved / med / 1e9, 1), **summary(t), "bytes_per_launch": moved}

    def empty(k):
        probe_call(rn, "launch", None, None, None, 0, torch.cuda.current_stream().cuda_stream)
    res["empty_launch"] = summary(graph_stats(torch, empty, launches))
    return res


def large_ceilings(torch, rn, mib, launches, total_mib=2048):
    """probe_ceilings over fresh buffers of `mib` MiB per stream, rotating through at least
    `total_mib` MiB per stream role (past the 256 MiB Infinity Cache)."""
    nbytes = mib * 2**20
    nsets = max(2, -(-total_mib // mib))
    streams = [tuple(torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda:0")
                     for _ in range(3)) for _ in range(nsets)]
    res = probe_ceilings(torch, rn, streams, nbytes, launches, cached_too=True)
    del streams
    torch.cuda.empty_cache()
    return {"stream_MiB": mib, "buffer_sets": nsets, **res}


def ceilings(torch, rn, launches):
    """The reference kernels at several buffer sizes (--ceilings)."""
    out = []
    for mib in (32, 64, 256, 1024):
        row = large_ceilings(torch, rn, mib, launches if mib < 1024 else max(8, launches // 8))
        out.append(row)
        print(json.dumps(row), flush=True)
    return out


REPLAYS = 5  # replays of each timing graph: per-launch mean, min and median over them


def graph_stats(torch, fn, launches, replays=REPLAYS):
    """Seconds per call of fn(k): a graph of `launches` back-to-back calls fn(0), fn(1), ...,
    replayed `replays` times with events on the launch stream around each replay. Returns the
    per-launch time of every replay (seconds)."""
    g = capture(torch, fn, launches)
    out = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / 1e3 / launches)
    del g
    return out


def summary(times):
    """mean / median / min of per-launch times (seconds) in microseconds."""
    v = sorted(times)
    mid = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    return {"mean_us": round(sum(v) / len(v) * 1e6, 3), "median_us": round(mid * 1e6, 3),
            "min_us": round(v[0] * 1e6, 3)}


def graph_time(torch, fn, launches):
    """Median seconds per call of fn(k) over the replays of graph_stats."""
    v = sorted(graph_stats(torch, fn, launches))
    return v[len(v) // 2]


def layernorm_row(torch, rn, sets, launches):
    """LayerNorm forward and backward at the headline shape, on the same rotating x / dy buffers
    (their values are the LayerNorm workload's: x, w and dy are drawn first, then the bias)."""
    from workloads import LN_WORKLOADS, make_norm_inputs, to_device
    wl = LN_WORKLOADS["ln_bf16_4096x4096"]
    assert (wl.M, wl.N, wl.dtype) == (sets.wl.M, sets.wl.N, sets.wl.dtype)
    lib, M, N = sets.lib, wl.M, wl.N
    dt = rn.DTYPE_CODES[wl.dtype]
    b = to_device(make_norm_inputs(wl)["b"], wl.dtype, "cuda:0")
    n = len(sets.sets)
    mean = [torch.empty(M, dtype=torch.float32, device="cuda:0") for _ in range(n)]
    db = torch.empty(N, dtype=torch.float32, device="cuda:0")
    wsb = rn.layernorm_workspace_bytes(M, N, wl.dtype)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda:0")

    def fwd(k):
        s = sets.sets[k % n]
        st = lib.layernorm_fwd(s["x"].data_ptr(), N, sets.w.data_ptr(), b.data_ptr(),
                               s["y"].data_ptr(), N, mean[k % n].data_ptr(), s["rstd"].data_ptr(),
                               M, N, dt, wl.eps, 0, sets.stream())
        if st:
            raise RuntimeError(f"layernorm_fwd status {st}")

    def bwd(k):
        s = sets.sets[(k + n // 2) % n]
        st = lib.layernorm_bwd(s["dy"].data_ptr(), N, s["x"].data_ptr(), N, sets.w.data_ptr(),
                               mean[(k + n // 2) % n].data_ptr(), s["rstd"].data_ptr(),
                               s["dx"].data_ptr(), N, s["dw"].data_ptr(), db.data_ptr(),
                               ws.data_ptr(), wsb, M, N, dt, 0, sets.stream())
        if st:
            raise RuntimeError(f"layernorm_bwd status {st}")

    for k in range(n):
        fwd(k)
    torch.cuda.synchronize()
    tf, tb = graph_time(torch, fwd, launches), graph_time(torch, bwd, launches)
    s = wl.itemsize
    fb = 2 * M * N * s + 2 * N * s + 8 * M
    bb = 3 * M * N * s + N * s + 8 * M + 8 * N
    return {"workload": wl.name, "fwd_us": round(tf * 1e6, 3), "bwd_us": round(tb * 1e6, 3),
            "fwd_GBps": round(fb / tf / 1e9, 1), "bwd_GBps": round(bb / tb / 1e9, 1),
            "fwd_bytes": fb, "bwd_bytes": bb,
            "bwd_includes": "rows kernel + dw and db reductions"}


def softmax_row(torch, rn, sets, launches):
    """Softmax over the last dimension, forward and backward, at the headline shape and dtype, on
    the rotating buffers (x as logits, y the output, then dy, y -> dx)."""
    lib, wl = sets.lib, sets.wl
    M, N, dt, n = wl.M, wl.N, rn.DTYPE_CODES[wl.dtype], len(sets.sets)

    def fwd(k):
        s = sets.sets[k % n]
        st = lib.softmax_fwd(s["x"].data_ptr(), N, s["y"].data_ptr(), N, M, N, dt, 0,
                             sets.stream())
        if st:
            raise RuntimeError(f"softmax_fwd status {st}")

    def bwd(k):
        s = sets.sets[(k + n // 2) % n]
        st = lib.softmax_bwd(s["dy"].data_ptr(), N, s["y"].data_ptr(), N, s["dx"].data_ptr(), N,
                             M, N, dt, 0, sets.stream())
        if st:
            raise RuntimeError(f"softmax_bwd status {st}")

    for k in range(n):
        fwd(k)
    torch.cuda.synchronize()
    tf, tb = graph_time(torch, fwd, launches), graph_time(torch, bwd, launches)
    s = wl.itemsize
    fb, bb = 2 * M * N * s, 3 * M * N * s
    return {"workload": f"softmax_{wl.dtype}_{M}x{N}", "fwd_us": round(tf * 1e6, 3),
            "bwd_us": round(tb * 1e6, 3), "fwd_GBps": round(fb / tf / 1e9, 1),
            "bwd_GBps": round(bb / tb / 1e9, 1), "fwd_bytes": fb, "bwd_bytes": bb}


NARROW_SHAPE = (65536, 128)  # many narrow rows (per-head widths): 16 vectors of 16 bits a row


def narrow_rows(torch, rn, launches, rotate_mib):
    """RMSNorm (round twice), LayerNorm and softmax, forward and backward, on bf16 65536 x 128: rows
    of 16 vectors, which the register kernels give 16 lanes each (4 rows a wavefront). Inputs drawn
    on the device (x, dy ~ N(0, 1), w ~ U(0.9, 1.1), LayerNorm bias ~ U(-0.1, 0.1)), timed like the
    other rows over rotating buffer sets."""
    from workloads import WORKLOADS, make_device_inputs
    M, N = NARROW_SHAPE
    dev = "cuda:0"
    wl = WORKLOADS["bf16_4096x4096"].with_(name=f"bf16_{M}x{N}", M=M, N=N)
    inp = make_device_inputs(wl, dev)
    n = max(4, -(-rotate_mib * 2**20 // (M * N * wl.itemsize)))
    sets = Sets(rn, torch, wl, "twice", inp, n, dev)
    del inp
    lib, dt, s, ss = sets.lib, sets.dt, wl.itemsize, sets.sets
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    b = (torch.rand(N, generator=g, device=dev) * 0.2 - 0.1).to(torch.bfloat16)
    mean = [torch.empty(M, dtype=torch.float32, device=dev) for _ in range(n)]
    db = torch.empty(N, dtype=torch.float32, device=dev)
    lwsb = rn.layernorm_workspace_bytes(M, N, wl.dtype)
    lws = torch.empty(lwsb // 4, dtype=torch.float32, device=dev)

    def half(k):
        return (k + n // 2) % n

    def check(st, what):
        if st:
            raise RuntimeError(f"{what} status {st}")

    def rms_fwd(k):
        sets.fwd(k % n)

    def rms_bwd(k):
        sets.bwd_rows(half(k))
        sets.dw_reduce(half(k))

    def ln_fwd(k):
        t = ss[k % n]
        check(lib.layernorm_fwd(t["x"].data_ptr(), N, sets.w.data_ptr(), b.data_ptr(),
                                t["y"].data_ptr(), N, mean[k % n].data_ptr(),
                                t["rstd"].data_ptr(), M, N, dt, 1e-5, 0, sets.stream()),
              "layernorm_fwd")

    def ln_bwd(k):
        t = ss[half(k)]
        check(lib.layernorm_bwd(t["dy"].data_ptr(), N, t["x"].data_ptr(), N, sets.w.data_ptr(),
                                mean[half(k)].data_ptr(), t["rstd"].data_ptr(),
                                t["dx"].data_ptr(), N, t["dw"].data_ptr(), db.data_ptr(),
                                lws.data_ptr(), lwsb, M, N, dt, 0, sets.stream()),
              "layernorm_bwd")

    def sm_fwd(k):
        t = ss[k % n]
        check(lib.softmax_fwd(t["x"].data_ptr(), N, t["y"].data_ptr(), N, M, N, dt, 0,
                              sets.stream()), "softmax_fwd")

    def sm_bwd(k):
        t = ss[half(k)]
        check(lib.softmax_bwd(t["dy"].data_ptr(), N, t["y"].data_ptr(), N, t["dx"].data_ptr(), N,
                              M, N, dt, 0, sets.stream()), "softmax_bwd")

    mn = M * N * s
    families = (
        ("rmsnorm_narrow", rms_fwd, rms_bwd, wl.fwd_bytes(), wl.bwd_bytes(),
         "rows kernel + dw reduction"),
        ("layernorm_narrow", ln_fwd, ln_bwd, 2 * mn + 2 * N * s + 8 * M,
         3 * mn + N * s + 8 * M + 8 * N, "rows kernel + dw and db reductions"),
        ("softmax_narrow", sm_fwd, sm_bwd, 2 * mn, 3 * mn, None))
    out = {}
    for name, fwd, bwd, fb, bb, inc in families:
        for k in range(n):
            fwd(k)
        torch.cuda.synchronize()
        tf, tb = graph_time(torch, fwd, launches), graph_time(torch, bwd, launches)
        out[name] = {"workload": wl.name, "fwd_us": round(tf * 1e6, 3),
                     "bwd_us": round(tb * 1e6, 3), "fwd_GBps": round(fb / tf / 1e9, 1),
                     "bwd_GBps": round(bb / tb / 1e9, 1), "fwd_bytes": fb, "bwd_bytes": bb,
                     "buffer_sets": n}
        if inc:
            out[name]["bwd_includes"] = inc
    return out


def f64_row(torch, rn, launches, rotate_mib):
    """The float64 RMSNorm, forward and backward, at 4096 x 4096."""
    from workloads import F64_WORKLOADS, make_inputs, to_device
    wl = F64_WORKLOADS["f64_4096x4096"]
    lib, dev, M, N = rn.library(), "cuda:0", wl.M, wl.N
    inp = make_inputs(wl)
    x0, dy0 = to_device(inp["x"], "f64", dev), to_device(inp["dy"], "f64", dev)
    w = to_device(inp["w"], "f64", dev)
    del inp
    n = max(4, -(-rotate_mib * 2**20 // (M * N * 8)))
    sets = [{"x": x0.clone(), "dy": dy0.clone(), "y": torch.empty_like(x0),
             "dx": torch.empty_like(x0),
             "rstd": torch.empty(M, dtype=torch.float64, device=dev)} for _ in range(n)]
    del x0, dy0
    dw = torch.empty(N, dtype=torch.float64, device=dev)
    wsb = int(lib.rmsnorm_bwd_f64_workspace_bytes(M, N))
    ws = torch.empty(wsb // 8, dtype=torch.float64, device=dev)
    stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731

    def fwd(k):
        s = sets[k % n]
        st = lib.rmsnorm_fwd_f64(s["x"].data_ptr(), N, w.data_ptr(), s["y"].data_ptr(), N,
                                 s["rstd"].data_ptr(), M, N, wl.eps, wl.offset, stream())
        if st:
            raise RuntimeError(f"rmsnorm_fwd_f64 status {st}")

    def bwd(k):
        s = sets[(k + n // 2) % n]
        st = lib.rmsnorm_bwd_f64(s["dy"].data_ptr(), N, s["x"].data_ptr(), N, w.data_ptr(),
                                 s["rstd"].data_ptr(), s["dx"].data_ptr(), N, dw.data_ptr(),
                                 ws.data_ptr(), wsb, M, N, wl.offset, stream())
        if st:
            raise RuntimeError(f"rmsnorm_bwd_f64 status {st}")

    for k in range(n):
        fwd(k)
    torch.cuda.synchronize()
    tf, tb = graph_time(torch, fwd, launches), graph_time(torch, bwd, launches)
    fb = 2 * M * N * 8 + N * 8 + 8 * M
    bb = 3 * M * N * 8 + N * 8 + 8 * M + 8 * N
    return {"workload": wl.name, "fwd_us": round(tf * 1e6, 3), "bwd_us": round(tb * 1e6, 3),
            "fwd_GBps": round(fb / tf / 1e9, 1), "bwd_GBps": round(bb / tb / 1e9, 1),
            "fwd_bytes": fb, "bwd_bytes": bb, "buffer_sets": n,
            "bwd_includes": "rows kernel + float64 dw reduction"}


GN_PASSES = "fwd reads x twice (statistics, then normalize); bwd reads x and dy twice"


def groupnorm_row(torch, rn, launches, rotate_mib, name=None, passes=GN_PASSES):
    """GroupNorm forward and backward at the group_norm page's (16, 32, 256, 256), 8 groups, or
    the GroupNorm workload `name`."""
    from workloads import GN_HEADLINE, GN_WORKLOADS, make_gn_inputs, to_device
    wl = GN_WORKLOADS[name or GN_HEADLINE]
    lib, dev = rn.library(), "cuda:0"
    dt = rn.DTYPE_CODES[wl.dtype]
    inp = make_gn_inputs(wl)
    x0, dy0 = to_device(inp["x"], wl.dtype, dev), to_device(inp["dy"], wl.dtype, dev)
    w, b = to_device(inp["w"], wl.dtype, dev), to_device(inp["b"], wl.dtype, dev)
    del inp
    n = max(4, -(-rotate_mib * 2**20 // (wl.numel * wl.itemsize)))
    sets = [{"x": x0.clone(), "dy": dy0.clone(), "y": torch.empty_like(x0),
             "dx": torch.empty_like(x0),
             "mean": torch.empty(wl.B * wl.G, dtype=torch.float32, device=dev),
             "rstd": torch.empty(wl.B * wl.G, dtype=torch.float32, device=dev)} for _ in range(n)]
    del x0, dy0
    dw = torch.empty(wl.C, dtype=torch.float32, device=dev)
    db = torch.empty(wl.C, dtype=torch.float32, device=dev)
    wsb = rn.groupnorm_workspace_bytes(wl.B, wl.C, wl.S, wl.G, wl.dtype)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731

    def fwd(k):
        s = sets[k % n]
        st = lib.groupnorm_fwd(s["x"].data_ptr(), w.data_ptr(), b.data_ptr(), s["y"].data_ptr(),
                               s["mean"].data_ptr(), s["rstd"].data_ptr(), ws.data_ptr(), wsb,
                               wl.B, wl.C, wl.S, wl.G, dt, wl.eps, stream())
        if st:
            raise RuntimeError(f"groupnorm_fwd status {st}")

    def bwd(k):
        s = sets[(k + n // 2) % n]
        st = lib.groupnorm_bwd(s["dy"].data_ptr(), s["x"].data_ptr(), w.data_ptr(),
                               s["mean"].data_ptr(), s["rstd"].data_ptr(), s["dx"].data_ptr(),
                               dw.data_ptr(), db.data_ptr(), ws.data_ptr(), wsb, wl.B, wl.C,
                               wl.S, wl.G, dt, stream())
        if st:
            raise RuntimeError(f"groupnorm_bwd status {st}")

    for k in range(n):
        fwd(k)
    torch.cuda.synchronize()
    tf, tb = graph_time(torch, fwd, launches), graph_time(torch, bwd, launches)
    return {"workload": wl.name, "fwd_us": round(tf * 1e6, 3), "bwd_us": round(tb * 1e6, 3),
            "fwd_GBps": round(wl.fwd_bytes() / tf / 1e9, 1),
            "bwd_GBps": round(wl.bwd_bytes() / tb / 1e9, 1),
            "fwd_bytes": wl.fwd_bytes(), "bwd_bytes": wl.bwd_bytes(), "buffer_sets": n,
            "passes": passes}


# Every RMSNorm configuration the library is specified for, timed like the headline: the
# correctness case (fp32 64 x 1024, launch-bound), the headline shape in the other rounding mode,
# the fp16 8192 x 8192 overflow case, the Gemma round-once shape, and the hidden-size sweep at
# M = 4096 (N = 32768 takes the LDS-staged backward).
CONFIG_SWEEP = [("fp32_64x1024", None), ("bf16_4096x4096", "once"), ("fp16_8192x8192", None),
                ("bf16_16384x3072_gemma", None)] + [
    (f"bf16_sweep_4096x{n}", None) for n in (1024, 2048, 4096, 8192, 16384, 32768)]
MAX_SETS = 1024  # only the launch-bound float32 64 x 1024 correctness case reaches it


def config_sweep(torch, rn, launches, rotate_mib):
    """Per configuration and rounding mode: step time (graph of `launches` steps), each kernel's
    per-launch time (median, with mean and min, over the replays of its timing graph), algorithmic
    GB/s and fraction of the HBM peak per phase. Inputs are drawn on the device with each
    workload's distributions (make_device_inputs). Every configuration rotates over enough buffer
    sets that its x matrices span `rotate_mib` MiB, except the float32 64 x 1024 case (capped at
    MAX_SETS sets: cache-resident and launch-bound, not a bandwidth figure)."""
    from workloads import WORKLOADS, make_device_inputs
    out = []
    for name, rounding in CONFIG_SWEEP:
        wl = WORKLOADS[name]
        rounding = rounding or wl.rounding
        inp = make_device_inputs(wl, "cuda:0")
        nsets = min(MAX_SETS, max(4, -(-rotate_mib * 2**20 // (wl.M * wl.N * wl.itemsize))))
        sets = Sets(rn, torch, wl, rounding, inp, nsets, "cuda:0")
        del inp
        for i in range(nsets):
            sets.fwd(i)
        torch.cuda.synchronize()
        step_t = graph_stats(torch, sets.step, launches)
        step = sorted(step_t)[len(step_t) // 2]
        dur, stats = kernel_durations(torch, sets, launches)
        stats["step"] = summary(step_t)
        bwd = dur["bwd_rows"] + dur["dw_reduce"]
        fb, bb = wl.fwd_bytes(), wl.bwd_bytes()
        cached = nsets * wl.M * wl.N * wl.itemsize < 2**30
        out.append({
            "workload": name, "dtype": wl.dtype, "M": wl.M, "N": wl.N, "rounding": rounding,
            "offset": wl.offset, "buffer_sets": nsets, "cache_resident": cached,
            "step_us": round(step * 1e6, 3), "fwd_us": round(dur["fwd"] * 1e6, 3),
            "bwd_us": round(bwd * 1e6, 3), "bwd_rows_us": round(dur["bwd_rows"] * 1e6, 3),
            "dw_reduce_us": round(dur["dw_reduce"] * 1e6, 3),
            "step_GBps": round((fb + bb) / step / 1e9, 1),
            "fwd_GBps": round(fb / dur["fwd"] / 1e9, 1), "bwd_GBps": round(bb / bwd / 1e9, 1),
            "step_frac_of_peak": round((fb + bb) / step / 1e9 / PEAK_HBM_GBPS, 4),
            "fwd_frac_of_peak": round(fb / dur["fwd"] / 1e9 / PEAK_HBM_GBPS, 4),
            "bwd_frac_of_peak": round(bb / bwd / 1e9 / PEAK_HBM_GBPS, 4),
            "stats": {k: v for k, v in stats.items() if k != "fwd_fp8"}})
        print(json.dumps({"config_done": name, "rounding": rounding}), file=sys.stderr,
              flush=True)
        del sets
        torch.cuda.empty_cache()
    return out


def row_cpu_baselines(budget_s):
    """The oracle of each widened row, one NumPy thread, on a bounded sample of the same workload
    (whole rows; GroupNorm on batch 0), forward + backward: algorithmic GB/s of the sample."""
    import oracle
    from workloads import (F64_WORKLOADS, GN_HEADLINE, GN_WORKLOADS, LN_WORKLOADS, SM_WORKLOADS,
                           make_gn_inputs, make_inputs, make_norm_inputs)
    out = {}

    def timed(fn, nbytes_per_call, what):
        calls, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s or calls == 0:
            fn()
            calls += 1
        dt = time.perf_counter() - t0
        return {"value": round(nbytes_per_call * calls / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                "kind": "oracle", "sample": f"{what}, {calls} passes in {dt:.1f} s"}

    wl = LN_WORKLOADS["ln_bf16_4096x4096"]
    rows = 64
    inp = make_norm_inputs(wl, M=rows)

    def ln():
        y, m, r = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], eps=wl.eps, dtype="bf16")
        oracle.layernorm_bwd(inp["dy"], inp["x"], inp["w"], m, r, dtype="bf16")
    s, N = 2, wl.N
    out["layernorm"] = timed(ln, rows * (2 * N * s + 8) + rows * (3 * N * s + 8) + 4 * N * s,
                             f"{rows} rows of {wl.name}")

    wl = SM_WORKLOADS["sm_bf16_4096x4096"]
    inp = make_inputs(wl, M=rows)

    def sm():
        y = oracle.softmax_fwd(inp["x"], dtype="bf16")
        oracle.softmax_bwd(inp["dy"], y, dtype="bf16")
    out["softmax"] = timed(sm, rows * 5 * wl.N * 2, f"{rows} rows of {wl.name}")

    wl = GN_WORKLOADS[GN_HEADLINE]
    inp = make_gn_inputs(wl, B=1)

    def gn():
        y, m, r = oracle.groupnorm_fwd(inp["x"], inp["w"], inp["b"], G=wl.G, eps=wl.eps,
                                       dtype="bf16")
        oracle.groupnorm_bwd(inp["dy"], inp["x"], inp["w"], m, r, G=wl.G, dtype="bf16")
    out["groupnorm"] = timed(gn, 5 * wl.C * wl.S * 2, f"batch 0 of {wl.name}")

    wl = F64_WORKLOADS["f64_4096x4096"]
    inp = make_inputs(wl, M=rows)

    def f64():
        y, r = oracle.rmsnorm_fwd_f64(inp["x"], inp["w"], eps=wl.eps)
        oracle.rmsnorm_bwd_f64(inp["dy"], inp["x"], inp["w"], r)
    out["rmsnorm_f64"] = timed(f64, rows * 5 * wl.N * 8, f"{rows} rows of {wl.name}")
    return out


def cpu_baseline(wl, rounding, inp, budget_s):
    """The CPU oracle, single-threaded, over row chunks of the same inputs (cycling through the
    rows again if one pass takes less than the budget) until the time budget is used."""
    import oracle
    x, w, dy = inp["x"], inp["w"], inp["dy"]
    rows, start, chunk, t0 = 0, 0, 64, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        sl = slice(start, min(start + chunk, wl.M))
        y, r = oracle.rmsnorm_fwd(x[sl], w, eps=wl.eps, offset=wl.offset, rounding=rounding,
                                  dtype=wl.dtype)
        oracle.rmsnorm_bwd(dy[sl], x[sl], w, r, offset=wl.offset, dtype=wl.dtype)
        rows += sl.stop - sl.start
        start = 0 if sl.stop >= wl.M else sl.stop
    dt = time.perf_counter() - t0
    sub = wl.with_(M=rows)
    nbytes = sub.fwd_bytes() + sub.bwd_bytes()
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} rows ({rows / wl.M:.2f} passes over the {wl.M} x {wl.N} inputs in "
                      f"chunks of {chunk} rows), forward + backward, {dt:.1f} s, NumPy single "
                      f"thread (host has {cores} usable cores)"}


def main(argv=None) -> int:
    args = parse_args(argv)
    global EAGER
    EAGER = args.no_graph
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: librmsnorm has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.copy_probe_mib)
        return 0

    import torch

    import bwd_precision_numerics_amd as rn
    from workloads import HEADLINE, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    rn.library()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        copy_probe(torch, rn, args.copy_probe_mib, args.steps, args.probe_kind)
        return 0
    if args.ceilings:
        ceilings(torch, rn, max(min(args.steps, 100), 20))
        return 0

    name = args.workload or HEADLINE
    wl = WORKLOADS[name]
    rounding = args.rounding or wl.rounding
    inp = make_inputs(wl)
    nsets = max(4, -(-args.rotate_mib * 2**20 // (wl.M * wl.N * wl.itemsize)))
    sets = Sets(rn, torch, wl, rounding, inp, nsets, "cuda:0", casts=args.bwd_casts)
    for i in range(len(sets.sets)):  # every set gets a valid rstd cache
        sets.fwd(i)
    torch.cuda.synchronize()

    if args.kernel_only:
        fn = {"fwd": sets.fwd, "bwd_rows": sets.bwd_rows, "dw_reduce": sets.dw_reduce,
              "fwd_fp8": sets.fwd_fp8}[args.kernel_only]
        for k in range(args.warmup + args.steps):
            fn(k % len(sets.sets))
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": args.kernel_only, "launches": args.warmup + args.steps,
                          "workload": name}), flush=True)
        return 0

    for k in range(args.warmup):
        sets.step(k)
    torch.cuda.synchronize()

    graph = None if args.no_graph else capture(torch, sets.step, args.steps)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for k in range(args.steps):
            sets.step(k)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    step_bytes = wl.fwd_bytes() + wl.bwd_bytes()
    value = step_bytes * args.steps / elapsed / 1e9

    dur, kstats = kernel_durations(torch, sets, max(args.steps, 20))
    # The library's reference kernels over the same rotating buffers (x, dy read; y, dx written),
    # and at 1 GiB per stream (steady state).
    streams = [(st["x"], st["dy"], st["dx"]) for st in sets.sets]
    ceil32 = probe_ceilings(torch, rn, streams, wl.M * wl.N * wl.itemsize, max(args.steps, 20))
    del graph
    s = wl.itemsize
    rows_bytes = 3 * wl.M * wl.N * s + wl.N * s + 4 * wl.M
    fp8_bytes = wl.M * wl.N * (s + 1) + wl.N * s + 4 * wl.M  # x, w in; y8, rstd out
    achieved = rows_bytes / dur["bwd_rows"] / 1e9
    traffic = read_traffic(name)

    line = {
        "metric": f"RMSNorm fwd+bwd achieved HBM GB/s and % of peak, {wl.dtype} M={wl.M} N={wl.N}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": name, "M": wl.M, "N": wl.N, "rounding": rounding,
                   "bwd_casts": args.bwd_casts,
                   "offset": wl.offset, "eps": wl.eps, "buffer_sets": len(sets.sets),
                   "graph": not args.no_graph},
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
        "step_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "kernel": "bwd_rows_kernel",
                     "bytes_per_launch": rows_bytes,
                     "avg_us": round(dur["bwd_rows"] * 1e6, 3)},
        "kernels_us": {k: round(v * 1e6, 3) for k, v in dur.items()},
        "phase_GBps": {"fwd": round(wl.fwd_bytes() / dur["fwd"] / 1e9, 1),
                       "fwd_fp8": round(fp8_bytes / dur["fwd_fp8"] / 1e9, 1),
                       "bwd": round(wl.bwd_bytes() / (dur["bwd_rows"] + dur["dw_reduce"]) / 1e9,
                                    1)},
        "kernel_stats_us": kstats,
        "ceilings": {"stream_bytes": wl.M * wl.N * s, "rotating_sets": len(sets.sets),
                     "what": "rmsnorm_bandwidth_probe: read / write / copy (1 read + 1 write) / "
                             "sum2 (2 reads + 1 write), 16-byte non-temporal accesses, same "
                             "rotation and graph timing", **ceil32},
        "fwd_frac_of_copy_ceiling": round(wl.fwd_bytes() / dur["fwd"] / 1e9
                                          / ceil32["copy"]["GBps"], 4),
        "bwd_rows_frac_of_sum2_ceiling": round(achieved / ceil32["sum2"]["GBps"], 4),
    }
    if not args.no_rows and name == HEADLINE:
        launches = max(min(args.steps, 100), 20)
        line["rows"] = {"layernorm": layernorm_row(torch, rn, sets, launches),
                        "softmax": softmax_row(torch, rn, sets, launches)}
        sets = None
        torch.cuda.empty_cache()
        line["rows"]["groupnorm"] = groupnorm_row(torch, rn, launches, args.rotate_mib)
        torch.cuda.empty_cache()
        line["rows"]["groupnorm_rows"] = groupnorm_row(
            torch, rn, launches, args.rotate_mib, "gn_bf16_8x640x32x32_g32",
            "a (batch, group) row held by one row group: x (and dy) read once")
        torch.cuda.empty_cache()
        line["rows"]["rmsnorm_f64"] = f64_row(torch, rn, launches, args.rotate_mib)
        torch.cuda.empty_cache()
        line["rows"].update(narrow_rows(torch, rn, launches, args.rotate_mib))
    if "rows" in line:
        for r in line["rows"].values():
            r["fwd_frac_of_peak"] = round(r["fwd_GBps"] / PEAK_HBM_GBPS, 4)
            r["bwd_frac_of_peak"] = round(r["bwd_GBps"] / PEAK_HBM_GBPS, 4)
    if not args.no_configs and name == HEADLINE:
        sets = None
        torch.cuda.empty_cache()
        line["configs"] = config_sweep(torch, rn, max(min(args.steps, 100), 20), args.rotate_mib)
    if not args.no_rows and name == HEADLINE:
        sets = None
        torch.cuda.empty_cache()
        line["ceilings_1GiB"] = large_ceilings(torch, rn, 1024, 8)
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(wl, rounding, inp, args.cpu_seconds)
        if "rows" in line:
            for k, v in row_cpu_baselines(min(1.5, args.cpu_seconds)).items():
                line["rows"][k]["cpu_baseline"] = v
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
