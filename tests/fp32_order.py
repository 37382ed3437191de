"""Models of the float32 summation order of the LayerNorm and GroupNorm backward kernels.

The oracle sums a row's c1 = sum(w * dy) / N and c2 = sum(w * dy * xhat) / N in float64 and rounds
once; the GPU sums in float32, in the order its thread-to-element mapping fixes. Where w * dy is
nearly constant along a row (an upstream gradient of ones), dx = rstd * ((w * dy - c1) - xhat * c2)
cancels, and the last bits of c1 reach the rounding to T for more elements than elsewhere. These
models reproduce the kernels' float32 order on the CPU, so a test can measure how many dx
elements that order alone moves off the oracle on its own inputs, and bound the bit-exact rate
from that instead of from the GPU's output.

LayerNorm (one row group per row, the mapping of the register and streaming kernels): a row of
nv 16-byte vectors of V elements goes to TPR = clamp(next power of two >= nv, 64, 1024) threads,
thread t owning vectors t, t + TPR, ...; each thread keeps two accumulators (even and odd elements
of its vectors, in order; compensated (Kahan) sums once a thread holds more than 8 vectors, plain
sums with fused multiply-adds for c2 otherwise), adds them, and the 64 lanes of a wavefront are
summed by a pairwise tree in lane order (the DPP reduction), then the wavefronts in order.

Rows that are not 16-byte aligned (x and dy rows at one offset from a 16-byte boundary, at most
1024 whole vectors a row): the peeled register kernel. Row r's whole vectors start h_r < V elements
in (h_r from the row's address); TPR = clamp(next power of two >= N // V, 64, 1024) lanes, lane l
holding whole vector l, lanes below h_r the head elements (first in the even accumulators) and
lanes below t_r the tail elements (last in the odd accumulators); plain sums, fused multiply-adds
for c2; then as above.

GroupNorm (a row is a (batch, group) slice of Cg channels of S elements), rows of more than 8192
elements (float32: 4096): each channel's elements are cut into chunks of at most 8192 (16-bit
types) elements; a chunk's 256 threads own 4 vectors of 8 elements each (vector it * 256 + t), keep
even/odd accumulators, and the block sums them (the pairwise lane tree, then 4 wavefronts in
order). The row constants then add w_c * chunk sum over
the row's chunks, lane-strided over 64 lanes (chunk e to lane e % 64, in order) and a halving
shuffle tree (lane i adds lane i + 32, then + 16, ...). Shorter rows (the row kernels): each
(batch, channel) segment is one chunk whose sums are taken by one wavefront, lane l adding the
segment's p1 = dy and p2 = fl(dy * xhat) at l, l + 64, ... in order (plain float32 additions), then
the lane tree; the row constants as above.
"""
from __future__ import annotations

import numpy as np

from oracle.layernorm import normalize
from oracle.rounding import rne_to

import oracle


def _fma(a, b, c):
    """float32 fused multiply-add (the float64 product of two float32 values is exact)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def _kahan(s, c, v):
    y = (v - c).astype(np.float32)
    t = (s + y).astype(np.float32)
    c = ((t - s).astype(np.float32) - y).astype(np.float32)
    return t, c


def _lane_tree(t):
    """Pairwise sum over the last axis (64 lanes) in lane order."""
    while t.shape[-1] > 1:
        t = (t[..., 0::2] + t[..., 1::2]).astype(np.float32)
    return t[..., 0]


def ln_row_sums(gd, xh, V: int = 8):
    """float32 sums(gd) and sums(gd * xhat) of each row [M, N], in the LayerNorm backward's order."""
    M, N = gd.shape
    nv = -(-N // V)
    tpr = int(min(max(1 << max(nv - 1, 0).bit_length(), 64), 1024))
    iters = -(-nv // tpr)
    pad = iters * tpr * V - N
    G = np.pad(gd, ((0, 0), (0, pad))).reshape(M, iters, tpr, V)
    X = np.pad(xh, ((0, 0), (0, pad))).reshape(M, iters, tpr, V)
    comp = iters > 8
    acc = {k: np.zeros((M, tpr), np.float32) for k in ("a1", "b1", "a2", "b2",
                                                     "ca1", "cb1", "ca2", "cb2")}
    for it in range(iters):
        for e in range(V):
            g, x = G[:, it, :, e], X[:, it, :, e]
            p = "a" if e % 2 == 0 else "b"
            if comp:
                acc[p + "1"], acc["c" + p + "1"] = _kahan(acc[p + "1"], acc["c" + p + "1"], g)
                acc[p + "2"], acc["c" + p + "2"] = _kahan(acc[p + "2"], acc["c" + p + "2"],
                                                          (g * x).astype(np.float32))
            else:
                acc[p + "1"] = (acc[p + "1"] + g).astype(np.float32)
                acc[p + "2"] = _fma(g, x, acc[p + "2"])
    out = []
    for k in ("1", "2"):
        t = ((acc["a" + k] + acc["b" + k]).astype(np.float32)
             - (acc["ca" + k] + acc["cb" + k]).astype(np.float32)).astype(np.float32)
        waves = _lane_tree(t.reshape(M, tpr // 64, 64))
        s = waves[:, 0]
        for w in range(1, waves.shape[1]):
            s = (s + waves[:, w]).astype(np.float32)
        out.append(s)
    return out[0], out[1]


def row_heads(M: int, N: int, itemsize: int, ld: int | None = None, base: int = 0):
    """Elements before the first 16-byte boundary of each row (at most N) for rows starting at byte
    base + r * ld * itemsize (the kernels' peel_head)."""
    ld = N if ld is None else ld
    addr = base + np.arange(M, dtype=np.int64) * ld * itemsize
    return np.minimum(((16 - addr % 16) % 16) // itemsize, N)


def ln_row_sums_peel(gd, xh, V: int, heads):
    """float32 sums(gd) and sums(gd * xhat) of each row in the peeled register kernel's order."""
    M, N = gd.shape
    tpr = int(min(max(1 << max(N // V - 1, 0).bit_length(), 64), 1024))
    out1 = np.zeros(M, np.float32)
    out2 = np.zeros(M, np.float32)
    heads = np.asarray(heads)
    for h in np.unique(heads):
        rows = np.nonzero(heads == h)[0]
        g, x = gd[rows], xh[rows]
        R = len(rows)
        nb = (N - h) // V
        t0 = h + nb * V
        t = N - t0
        a1, b1, a2, b2 = (np.zeros((R, tpr), np.float32) for _ in range(4))
        a1[:, :h] = g[:, :h]
        a2[:, :h] = _fma(g[:, :h], x[:, :h], a2[:, :h])
        G = g[:, h:t0].reshape(R, nb, V)
        X = x[:, h:t0].reshape(R, nb, V)
        for e in range(0, V, 2):
            a1[:, :nb] = (a1[:, :nb] + G[:, :, e]).astype(np.float32)
            b1[:, :nb] = (b1[:, :nb] + G[:, :, e + 1]).astype(np.float32)
            a2[:, :nb] = _fma(G[:, :, e], X[:, :, e], a2[:, :nb])
            b2[:, :nb] = _fma(G[:, :, e + 1], X[:, :, e + 1], b2[:, :nb])
        b1[:, :t] = (b1[:, :t] + g[:, t0:]).astype(np.float32)
        b2[:, :t] = _fma(g[:, t0:], x[:, t0:], b2[:, :t])
        for out, (p, q) in ((out1, (a1, b1)), (out2, (a2, b2))):
            waves = _lane_tree((p + q).astype(np.float32).reshape(R, tpr // 64, 64))
            acc = waves[:, 0]
            for k in range(1, waves.shape[1]):
                acc = (acc + waves[:, k]).astype(np.float32)
            out[rows] = acc
    return out1, out2


def ln_dx_model_bitexact(dy, x, w, mean, rstd, *, dtype: str, wide: bool = True,
                         mapping: str | None = None, heads=None) -> float:
    """Fraction of dx elements that the LayerNorm kernels' float32 order of c1, c2 leaves
    bit-identical to the oracle's dx (same mean and rstd, same elementwise steps). ``mapping``:
    "wide" (rows 16-byte aligned, vectors of 16 bytes), "elementwise" (threads hold single elements,
    vectors of one, all in the even accumulator) or "peel" (rows not 16-byte aligned; ``heads`` the
    rows' h, by default contiguous rows from a 16-byte aligned base); by default ``wide`` picks
    between the first two."""
    x = np.asarray(x, np.float32)
    xh = normalize(x, mean, rstd, False).astype(np.float32)
    gd = (np.asarray(w, np.float32) * np.asarray(dy, np.float32)).astype(np.float32)
    V = 4 if dtype == "f32" else 8
    mapping = mapping or ("wide" if wide else "elementwise")
    if mapping == "peel":
        if heads is None:
            heads = row_heads(x.shape[0], x.shape[1], 4 if dtype == "f32" else 2)
        s1, s2 = ln_row_sums_peel(gd, xh, V, heads)
    else:
        s1, s2 = ln_row_sums(gd, xh, V if mapping == "wide" else 1)
    n = np.float32(x.shape[-1])
    c1 = (s1 / n).astype(np.float32)[:, None]
    c2 = (s2 / n).astype(np.float32)[:, None]
    r = np.asarray(rstd, np.float32)[:, None]
    with np.errstate(invalid="ignore", over="ignore"):
        dx = rne_to((r * ((gd - c1).astype(np.float32) - (xh * c2).astype(np.float32))
                     ).astype(np.float32), dtype)
    dx_o, _, _ = oracle.layernorm_bwd(dy, x, w, mean, rstd, dtype=dtype)
    return _same_frac(dx, dx_o)


def gn_row_kernel_mode(C: int, S: int, G: int, dtype: str):
    """Which kernels serve a GroupNorm shape (16-byte aligned contiguous tensors): "vector" (row
    kernels whose segment sums add per-vector sums: 16-byte rows, S a multiple of the vector, rows
    of up to 32768 elements, float32 16384), "element" (row kernels adding single values: rows of up
    to 16384, float32 8192), or None (the chunked kernels). Both row modes need S within one chunk
    (8192 elements, float32 4096) and the backward's LDS, 2 * (m + Cg) + 128 floats for m staged
    values a row, within 36864."""
    f32 = dtype == "f32"
    V = 4 if f32 else 8
    Cg = C // G
    n = Cg * S
    rmax = 8192 if f32 else 16384
    if S > (4096 if f32 else 8192):
        return None
    wide = (n * (4 if f32 else 2)) % 16 == 0
    if wide and S % V == 0 and n <= 2 * rmax and 2 * (n // V + Cg) + 128 <= 36864:
        return "vector"
    if n <= rmax and 2 * (n + Cg) + 128 <= 36864:
        return "element"
    return None


def gn_uses_row_kernels(C: int, S: int, G: int, dtype: str) -> bool:
    """Whether the row kernels serve the shape (gn_row_kernel_mode)."""
    return gn_row_kernel_mode(C, S, G, dtype) is not None


def gn_segment_sums(p, V: int = 1):
    """float32 sums over the last axis of p [B, C, S] in the row kernels' segment order: lane l
    adds values l, l + 64, ... in order, then the 64-lane tree. V > 1 (the "vector" mode): the
    values are first the per-vector sums, each vector's V elements added in element order."""
    p = np.asarray(p, np.float32)
    if V > 1:
        B, C, S = p.shape
        q = p.reshape(B, C, S // V, V)
        acc = q[..., 0]
        for e in range(1, V):
            acc = (acc + q[..., e]).astype(np.float32)
        p = acc
    B, C, S = p.shape
    L = -(-S // 64)
    P = np.pad(p, ((0, 0), (0, 0), (0, L * 64 - S))).reshape(B, C, L, 64)
    lanes = np.zeros((B, C, 64), np.float32)
    for i in range(L):
        lanes = (lanes + P[:, :, i, :]).astype(np.float32)
    return _lane_tree(lanes)


def gn_dx_model_bitexact(dy, x, w, mean, rstd, *, G: int, dtype: str,
                         rows: bool | str | None = None) -> float:
    """As ln_dx_model_bitexact for GroupNorm ([B, C, S] inputs, mean and rstd [B, G]). ``rows``:
    None takes the kernels that serve the shape (gn_row_kernel_mode); False the chunked kernels'
    sums; True the row kernels' ("vector" when S is a multiple of the vector, else "element");
    or the mode itself."""
    x = np.asarray(x, np.float32)
    dy = np.asarray(dy, np.float32)
    B, C, S = x.shape
    Cg = C // G
    ch = 8192 if dtype != "f32" else 4096
    V = 8 if dtype != "f32" else 4
    if rows is None:
        rows = gn_row_kernel_mode(C, S, G, dtype)
    elif rows is True:
        rows = "vector" if S % V == 0 else "element"
    elif rows is False:
        rows = None
    K = 1 if rows else -(-S // ch)
    m = np.asarray(mean, np.float32).reshape(B, G)
    r = np.asarray(rstd, np.float32).reshape(B, G)
    mc = np.repeat(m, Cg, axis=1)[..., None]
    rc = np.repeat(r, Cg, axis=1)[..., None]
    xh = ((x - mc).astype(np.float32) * rc).astype(np.float32)  # [B, C, S]
    if rows:
        vs = V if rows == "vector" else 1
        sums = [gn_segment_sums(p, vs)[..., None] for p in (dy, (dy * xh).astype(np.float32))]
    else:
        # per-chunk sums: T threads x 4 vectors of V (thread t holds vectors t, t + T, ...), even /
        # odd accumulators, lane tree, the 4 waves in order (T = 256); segments of at most a
        # quarter chunk take one wavefront each (T = 64: the lane tree is the sum)
        T = 64 if S <= ch // 4 else 256
        pad = K * (4 * T * V) - S
        D = np.pad(dy, ((0, 0), (0, 0), (0, pad))).reshape(B, C, K, 4, T, V)
        X = np.pad(xh, ((0, 0), (0, 0), (0, pad))).reshape(B, C, K, 4, T, V)
        a1 = b1 = a2 = b2 = np.zeros((B, C, K, T), np.float32)
        for it in range(4):
            for e in range(V):
                d, xx = D[..., it, :, e], X[..., it, :, e]
                if e % 2:
                    b1, b2 = (b1 + d).astype(np.float32), _fma(d, xx, b2)
                else:
                    a1, a2 = (a1 + d).astype(np.float32), _fma(d, xx, a2)
        sums = []
        for p, q in ((a1, b1), (a2, b2)):
            waves = _lane_tree((p + q).astype(np.float32).reshape(B, C, K, T // 64, 64))
            s = waves[..., 0]
            for k in range(1, T // 64):
                s = (s + waves[..., k]).astype(np.float32)
            sums.append(s)  # [B, C, K]
    wv = np.asarray(w, np.float32)
    consts = []
    for s in sums:
        ent = (wv[None, :, None] * s).astype(np.float32).reshape(B, G, Cg * K)  # row entries
        nent = Cg * K
        lanes = np.zeros((B, G, 64), np.float32)
        for e in range(nent):
            lanes[..., e % 64] = (lanes[..., e % 64] + ent[..., e]).astype(np.float32)
        off = 32
        while off >= 1:
            lanes[..., :off] = (lanes[..., :off] + lanes[..., off:2 * off]).astype(np.float32)
            off //= 2
        consts.append((lanes[..., 0] / np.float32(Cg * S)).astype(np.float32))
    c1 = np.repeat(consts[0], Cg, axis=1)[..., None]
    c2 = np.repeat(consts[1], Cg, axis=1)[..., None]
    gd = (wv[None, :, None] * dy).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        dx = rne_to((rc * ((gd - c1).astype(np.float32) - (xh * c2).astype(np.float32))
                     ).astype(np.float32), dtype)
    dx_o, _, _ = oracle.groupnorm_bwd(dy, x, w, m, r, G=G, dtype=dtype)
    return _same_frac(dx, dx_o)


def _same_frac(a, b) -> float:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    eq = (np.isnan(a) & np.isnan(b)) | (a.view(np.uint32) == b.view(np.uint32))
    return float(eq.mean()) if eq.size else 1.0
