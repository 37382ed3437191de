"""Compile the HIP library ``librmsnorm.so`` for gfx950, in place next to this file.

The library is built from four translation units: ``librmsnorm.hip`` (the RMSNorm entry points of
``include/librmsnorm.h``), ``libnorms.hip`` (LayerNorm and GroupNorm, ``include/libnorms.h``),
``libsoftmax.hip`` (softmax, ``include/libsoftmax.h``, and the float64 RMSNorm) and
``libceiling.hip`` (the HBM bandwidth reference kernels of the measurement section of
``include/librmsnorm.h``).

Usage: ``python -m bwd_precision_numerics_amd.build [--resource-usage FILE [--summary]]``: with
``--resource-usage`` the compiler's per-kernel resource remarks go to FILE, and ``--summary`` prints
them as a table (one row per kernel instantiation: VGPRs, AGPRs, spilled VGPRs, scratch bytes per
lane, occupancy in waves per SIMD, static LDS bytes).

Flags:
* ``--offload-arch=gfx950``: MI355X only.
* ``-ffp-contract=off``: no implicit multiply-add fusion, so every product and difference in the
  elementwise formulas is one IEEE float32 operation as the contract states; the kernels request
  fused multiply-adds explicitly where a reduction may use them.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed float32 VALU instructions.
* ``-fvisibility=hidden``: only the ``extern "C"`` entry points are exported.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("librmsnorm.hip", "libnorms.hip", "libsoftmax.hip",
                                                 "libceiling.hip")]
OUT = os.path.join(HERE, "librmsnorm.so")
HEADERS = [os.path.join(HERE, "csrc", f) for f in
           ("host_common.hpp", "rmsnorm_common.hpp", "rmsnorm_fwd.hpp", "rmsnorm_bwd.hpp",
            "layernorm.hpp", "groupnorm.hpp", "softmax.hpp")]
HEADERS += [os.path.join(ROOT, "include", f) for f in ("librmsnorm.h", "libnorms.h", "libsoftmax.h")]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def flags() -> list:
    """Compile flags of every translation unit."""
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    return proc.returncode, proc.stdout + proc.stderr


def build(resource_usage: str | None = None, verbose: bool = False) -> str:
    """Compile librmsnorm.so (always recompiles; the translation units in parallel, into objects
    under ``_build/``, then one link). Returns the path of the library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    objs = [os.path.join(objdir, os.path.splitext(os.path.basename(s))[0] + ".o") for s in SRCS]
    cmds = [[hipcc()] + flags() + extra + ["-c", src, "-o", obj] for src, obj in zip(SRCS, objs)]
    with concurrent.futures.ThreadPoolExecutor(len(cmds)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    diag = "".join(d for _, d in results)
    if resource_usage:
        with open(resource_usage, "w") as f:
            f.write(diag)
    if any(rc for rc, _ in results):
        sys.stderr.write(diag)
        raise RuntimeError("hipcc failed compiling " +
                           ", ".join(os.path.basename(s) for s, (rc, _) in zip(SRCS, results) if rc))
    tmp = OUT + ".tmp"
    rc, d = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                 verbose)
    if rc:
        sys.stderr.write(d)
        raise RuntimeError(f"hipcc link failed with exit code {rc}")
    os.replace(tmp, OUT)
    return OUT


def resource_table(diag: str) -> str:
    """Markdown table of the kernel-resource-usage remarks in `diag` (names demangled with c++filt
    when it is installed)."""
    import re
    rows, order = {}, []
    cur = None
    for line in diag.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            if cur not in rows:
                order.append(cur)
            rows[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\w+)", line)
        if m and cur:
            rows[cur][m.group(1).strip()] = m.group(2)
    names = order
    if shutil.which("c++filt"):
        out = subprocess.run(["c++filt"], input="\n".join(order), capture_output=True, text=True)
        if out.returncode == 0:
            names = out.stdout.splitlines()
    lines = ["| kernel | VGPRs | AGPRs | VGPRs spilled | scratch B/lane | waves/SIMD | LDS B |",
             "|---|---|---|---|---|---|---|"]
    for mangled, name in sorted(zip(order, names), key=lambda p: p[1]):
        r = rows[mangled]
        lines.append(f"| `{name}` | {r.get('VGPRs', '?')} | {r.get('AGPRs', '?')} | "
                     f"{r.get('VGPRs Spill', '?')} | {r.get('ScratchSize', '?')} | "
                     f"{r.get('Occupancy', '?')} | {r.get('LDS Size', '?')} |")
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--resource-usage", help="write the compiler's per-kernel resource report here")
    ap.add_argument("--summary", action="store_true",
                    help="with --resource-usage: print the remarks as a table")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    out = build(args.resource_usage, args.verbose)
    if args.summary and args.resource_usage:
        with open(args.resource_usage) as f:
            print(resource_table(f.read()))
    else:
        print(out)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
