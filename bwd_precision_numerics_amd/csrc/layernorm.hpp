// LayerNorm forward and backward kernels (row-wise over the last dimension).
//
// Forward, per row (candle pull request 4059, "Add backward passes to the fused rms_norm,
// layer_norm and softmax_last_dim ops": float32 statistics for the 16-bit types, one cast at the
// store; Liger-Kernel pull request 1608, "fix(group_norm): keep the backward statistics and
// reductions in fp32": mean and rstd kept in float32 for the backward):
//   mean = (sum_j x_j) / N,   var = (sum_j (x_j - mean)^2) / N,   rstd = 1 / sqrt(var + eps)
//   y    = T( (x - mean) * rstd * w + b )          each step one float32 operation, left to right
// The row stays in registers, so the variance is taken about the mean in a second pass over the
// registers rather than as E[x^2] - mean^2 (which cancels when the mean is large against the
// spread).
//
// Backward, from the float32 mean and rstd caches, inputs upcast on load:
//   xhat = (x - mean) * rstd,  gdy = w * dy,  c1 = (sum_j gdy_j) / N,  c2 = (sum_j gdy_j xhat_j) / N
//   dx   = T( rstd * ((gdy - c1) - xhat * c2) )
//   dw_j = sum over rows of dy_j * xhat_j,  db_j = sum over rows of dy_j      (float32)
// dw and db come from the same persistent-grid partials as the RMSNorm backward (no atomics): the
// workspace holds [2][P][ldp] floats, the dw partial rows then the db partial rows, each reduced in
// a fixed order by dw_reduce_kernel.
#pragma once

#include "rmsnorm_bwd.hpp"
#include "rmsnorm_fwd.hpp"

namespace rmsn {

struct LnFwdArgs {
  const void* x;
  const void* w;
  const void* b;  // may be null (no bias)
  void* y;
  float* mean;    // may be null
  float* rstd;    // may be null
  int64_t ldx, ldy, M;
  int N;
  int tpr;     // threads per row, multiple of 64
  int groups;  // rows per block
  int yvec;    // y and ldy allow 16-byte stores
  int comp;    // streaming kernel: compensated row sums (long per-thread chains)
  float eps;
};

// y for V elements of one vector: ((x - mean) * rstd) * w (+ b), one float32 operation each.
template <int V, bool HAS_B>
__device__ __forceinline__ void ln_affine(const float (&xf)[V], const float (&wf)[V],
                                          const float (&bf)[V], float mean, float rs,
                                          float (&yf)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const float xh = (xf[e] - mean) * rs;
    yf[e] = HAS_B ? xh * wf[e] + bf[e] : xh * wf[e];
  }
}

// Centred squares of the valid elements of one vector (elements at or past N excluded).
template <int V>
__device__ __forceinline__ void add_centred_squares(const float (&f)[V], float mean, int n,
                                                    RowAcc& q, bool comp) {
  if (n >= V) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float d = f[e] - mean;
      q.fma(e, d, d, comp);
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float d = e < n ? f[e] - mean : 0.f;
      q.fma(e, d, d, comp);
    }
  }
}

// Register kernel: the row stays in registers through the two reductions and the store. With
// LATE_WB, w and b (cache-resident, shared by every row) are loaded in the store loop instead of
// with x, so wider rows fit one wavefront without holding three row slices in registers.
// LDS: two reduction slots of wpr floats per row group. FULL: the host has checked
// N = ITERS * TPR * V (the threads' vectors tile the row), and there is no partial-vector code.
// SUB > 0: rows of at most SUB vectors on row groups of SUB lanes (segment_sum, bit for bit the
// one-wavefront sums), as the RMSNorm forward; no LDS.
template <DT D, int ITERS, bool HAS_B, bool LATE_WB = false, bool FULL = false, int SUB = 0>
__global__ void __launch_bounds__(1024) ln_fwd_rows_kernel(LnFwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  static_assert(SUB == 0 || (ITERS == 1 && !LATE_WB), "narrow rows: one vector per lane");
  extern __shared__ uint4 smem[];

  const int TPR = SUB ? SUB : a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  float* red = reinterpret_cast<float*>(smem) + grp * 2 * wpr;

  const S* xr = static_cast<const S*>(a.x) + (valid ? row : 0) * a.ldx;
  const S* wr = static_cast<const S*>(a.w);
  const S* br = static_cast<const S*>(a.b);
  constexpr int WB = LATE_WB ? 1 : ITERS;
  Raw raw[ITERS], wraw[WB], braw[HAS_B ? WB : 1];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    Raw r = IO::zero(), rw = IO::zero(), rb = IO::zero();
    if (valid) {
      if (FULL || col + V <= N) {
        r = IO::load_nt(xr + col);
        if constexpr (!LATE_WB) {
          rw = IO::load(wr + col);
          if constexpr (HAS_B) rb = IO::load(br + col);
        }
      } else if (col < N) {
        r = IO::load_part(xr + col, N - col);
        if constexpr (!LATE_WB) {
          rw = IO::load_part(wr + col, N - col);
          if constexpr (HAS_B) rb = IO::load_part(br + col, N - col);
        }
      }
    }
    raw[it] = r;
    if constexpr (!LATE_WB) {
      wraw[it] = rw;
      if constexpr (HAS_B) braw[it] = rb;
    }
  }
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    float f[V];
    IO::unpack(raw[it], f);
#pragma unroll
    for (int e = 0; e < V; e += 2) {
      s0 += f[e];
      s1 += f[e + 1];
    }
  }
  float sum_x;
  if constexpr (SUB > 0) sum_x = segment_sum<SUB>(s0 + s1);
  else sum_x = group_sum(s0 + s1, red, wpr, tl);
  const float mean = sum_x / (float)N;
  RowAcc q;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    float f[V];
    IO::unpack(raw[it], f);
    add_centred_squares<V>(f, mean, FULL ? V : N - col, q, false);
  }
  float sum_q;
  if constexpr (SUB > 0) sum_q = segment_sum<SUB>(q.total());
  else sum_q = group_sum(q.total(), red + wpr, wpr, tl);
  const float var = sum_q / (float)N;
  const float rs = 1.0f / __builtin_sqrtf(var + a.eps);
  if (!valid) return;
  if (tl == 0) {
    if (a.mean) a.mean[row] = mean;
    if (a.rstd) a.rstd[row] = rs;
  }
  void* yr = out_row<D, Out::ONCE>(a.y, row, a.ldy);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (!FULL && col >= N) continue;
    float xf[V], wf[V], bf[V], yf[V];
    IO::unpack(raw[it], xf);
    if constexpr (LATE_WB) {
      const bool full = FULL || col + V <= N;
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
      if constexpr (HAS_B)
        IO::unpack(full ? IO::load(br + col) : IO::load_part(br + col, N - col), bf);
    } else {
      IO::unpack(wraw[it], wf);
      if constexpr (HAS_B) IO::unpack(braw[it], bf);
    }
    ln_affine<V, HAS_B>(xf, wf, bf, mean, rs, yf);
    store_out<D, Out::ONCE, true, V>(yr, col, FULL ? V : N - col, a.yvec != 0, yf);
  }
}

// Any N and any alignment: three passes over the row (sum, centred squares, store), reading x again
// from the caches. Same thread-to-element mapping and summation order as the register kernel.
// PEEL (16-byte vectors on rows that are not 16-byte aligned, as the RMSNorm forward's peeled
// kernel): per row the whole vectors start h < V elements in (h from the row's address), lanes
// 0 .. h-1 hold the head elements (first in their even sums) and lanes 0 .. t-1 the tail elements
// (last in their odd sums); w and b for a vector come aligned and funnel-shifted by h (peel_w), and
// y takes vector stores when its rows sit at x's offsets (yvec).
template <DT D, bool WIDE, bool HAS_B, bool PEEL = false>
__global__ void __launch_bounds__(1024) ln_fwd_stream_kernel(LnFwdArgs a) {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  static_assert(!PEEL || WIDE, "PEEL takes 16-byte vectors");
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  float* red = reinterpret_cast<float*>(smem) + grp * 2 * wpr;
  const S* xr = static_cast<const S*>(a.x) + (valid ? row : 0) * a.ldx;
  // The vector part of the row: NV elements from xv (the whole row unless PEEL).
  int h = 0, t = 0;
  if constexpr (PEEL) {
    h = peel_head(xr, N);
    t = (N - h) % V;
  }
  const S* xv = xr + h;
  const int NV = N - h - t;
  const int nv = (NV + V - 1) / V;

  const bool comp = a.comp != 0;
  RowAcc sx;
  if (valid) {
    if constexpr (PEEL) {
      if (tl < h) sx.add(0, to_f32<D>(xr[tl]), comp);
    }
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      float f[V];
      IO::unpack(col + V <= NV ? IO::load(xv + col) : IO::load_part(xv + col, NV - col), f);
#pragma unroll
      for (int e = 0; e < V; ++e) sx.add(e, f[e], comp);
    }
    if constexpr (PEEL) {
      if (tl < t) sx.add(1, to_f32<D>(xv[NV + tl]), comp);
    }
  }
  const float mean = group_sum(sx.total(), red, wpr, tl) / (float)N;
  RowAcc q;
  if (valid) {
    if constexpr (PEEL) {
      if (tl < h) {
        const float d = to_f32<D>(xr[tl]) - mean;
        q.fma(0, d, d, comp);
      }
    }
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      float f[V];
      IO::unpack(col + V <= NV ? IO::load(xv + col) : IO::load_part(xv + col, NV - col), f);
      add_centred_squares<V>(f, mean, NV - col, q, comp);
    }
    if constexpr (PEEL) {
      if (tl < t) {
        const float d = to_f32<D>(xv[NV + tl]) - mean;
        q.fma(1, d, d, comp);
      }
    }
  }
  const float var = group_sum(q.total(), red + wpr, wpr, tl) / (float)N;
  const float rs = 1.0f / __builtin_sqrtf(var + a.eps);
  if (!valid) return;
  if (tl == 0) {
    if (a.mean) a.mean[row] = mean;
    if (a.rstd) a.rstd[row] = rs;
  }
  const S* wr = static_cast<const S*>(a.w);
  const S* br = static_cast<const S*>(a.b);
  void* yr = out_row<D, Out::ONCE>(a.y, row, a.ldy);
  if constexpr (PEEL) {
    auto one = [&](int col) {
      const float xf[1] = {to_f32<D>(xr[col])}, wf[1] = {to_f32<D>(wr[col])};
      const float bf[1] = {HAS_B ? to_f32<D>(br[col]) : 0.f};
      float yf[1];
      ln_affine<1, HAS_B>(xf, wf, bf, mean, rs, yf);
      store_out<D, Out::ONCE, false, 1>(yr, col, 1, false, yf);
    };
    if (tl < h) one(tl);
    if (tl < t) one(h + NV + tl);
  }
  const bool walign = ((uintptr_t)wr & 15u) == 0, balign = ((uintptr_t)br & 15u) == 0;
  for (int v = tl; v < nv; v += TPR) {
    const int col = v * V;
    const bool full = col + V <= NV;
    float xf[V], wf[V], bf[V], yf[V];
    // the row's last read of x: non-temporal
    IO::unpack(full ? IO::load_nt(xv + col) : IO::load_part(xv + col, NV - col), xf);
    if constexpr (PEEL) {
      peel_w<D, V>(wr, walign, N, h, h + col, wf);
      if constexpr (HAS_B) peel_w<D, V>(br, balign, N, h, h + col, bf);
    } else {
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
      if constexpr (HAS_B)
        IO::unpack(full ? IO::load(br + col) : IO::load_part(br + col, N - col), bf);
    }
    ln_affine<V, HAS_B>(xf, wf, bf, mean, rs, yf);
    store_out<D, Out::ONCE, WIDE, V>(yr, h + col, NV - col, a.yvec != 0, yf);
  }
}

struct LnBwdArgs {
  const void* dy;
  const void* x;
  const void* w;
  const float* mean;
  const float* rstd;
  void* dx;
  float* part;  // [2][P][ldp]: dw partial rows, then db partial rows
  int64_t lddy, ldx, lddx, M;
  int N, ldp, P;
  int tpr;     // threads per row, multiple of 64
  int groups;  // rows processed concurrently per block
  int comp;    // streaming kernel: compensated row sums (long per-thread chains)
  int dxvec = 0;  // peeled rows: dx rows sit at x's offsets from a 16-byte boundary
};

// combine_groups' first level split in two around a barrier the caller already has (the one of
// the last row's sums), so that the block's column sums leave before the last row's dx is
// written: combine_give (before that barrier) has the upper floor(groups / 2) groups hand their
// sums over, combine_take (after it) adds them into the groups below, and combine_groups with
// groups - floor(groups / 2) completes the same tree. `buf` as for combine_groups, apart from the
// values of the barrier's own round.
template <int K>
__device__ __forceinline__ void combine_give(const float (&acc)[K], float* buf, int groups,
                                             int grp, int tl, int slice_threads) {
  const int h = groups >> 1;
  if (grp >= groups - h) {
    float* dst = buf + ((size_t)(grp - (groups - h)) * slice_threads + tl) * K;
#pragma unroll
    for (int k = 0; k < K; ++k) dst[k] = acc[k];
  }
}
template <int K>
__device__ __forceinline__ void combine_take(float (&acc)[K], const float* buf, int groups,
                                             int grp, int tl, int slice_threads) {
  const int h = groups >> 1;
  if (grp >= groups - 2 * h && grp < groups - h) {
    const float* src = buf + ((size_t)(grp - (groups - 2 * h)) * slice_threads + tl) * K;
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] += src[k];
  }
}

// Register kernel on the persistent grid of the RMSNorm backward (block b owns rows b, b + P, ...).
// A ring of DEPTH + 1 rows of raw (x, dy) and their (mean, rstd) per row group keeps DEPTH rows in
// flight while one is reduced and written. HAS_DB adds the bias-gradient accumulators. KEEP holds
// xhat and w * dy from the first pass for the second (fewer vector ALU operations, more registers)
// instead of recomputing them from the raw row. TAIL and WPR as for the RMSNorm bwd_rows_kernel,
// whose load discipline this kernel follows: every step issues its row's loads as straight-line
// buffer loads (rows past the block's share read w), only the arithmetic and stores are guarded.
// SUB > 0: narrow rows of whole vectors on row groups of SUB lanes, as the RMSNorm bwd_rows_kernel
// (a wavefront's rows addressed from its first row's descriptor, segment_sum for the row sums,
// combine_columns for the dw and db sums: its LDS is the only LDS such an instantiation uses).
template <DT D, int ITERS, int DEPTH, bool HAS_DB, bool KEEP, Tail TAIL, int WPR, int SUB = 0>
__global__ void __launch_bounds__(1024) ln_bwd_rows_kernel(LnBwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  constexpr int RING = DEPTH + 1;
  constexpr int K = ITERS * V;
  // partial rows written in the last step (row groups of whole wavefronts)
  constexpr bool EARLY = ITERS == 1 && SUB == 0;
  static_assert(SUB == 0 || (ITERS == 1 && TAIL != Tail::RAGGED && WPR == 0),
                "narrow rows: at most one whole vector per lane");
  extern __shared__ uint4 smem[];

  const int TPR = SUB ? SUB : WPR ? 64 * WPR : a.tpr, wpr = SUB ? 1 : WPR ? WPR : TPR >> 6;
  const int G = SUB ? 1024 / SUB : WPR ? 1024 / (64 * WPR) : a.groups, N = a.N;
  const int tid = threadIdx.x;
  const int grp = SUB ? tid / TPR : wave_group(tid, TPR);
  const int g0 = SUB ? wave_group(tid & ~63, TPR) : grp;  // group of the wavefront's first lane
  const int dg = grp - g0;
  const int tl = tid - grp * TPR;
  // Byte distance between a wavefront's consecutive rows in x, dy and dx.
  const uint32_t dx_step = SUB ? (uint32_t)((int64_t)a.P * a.ldx * (int64_t)sizeof(S)) : 0u;
  const uint32_t dd_step = SUB ? (uint32_t)((int64_t)a.P * a.lddy * (int64_t)sizeof(S)) : 0u;
  const uint32_t do_step = SUB ? (uint32_t)((int64_t)a.P * a.lddx * (int64_t)sizeof(S)) : 0u;
  const int b = blockIdx.x, P = a.P;
  const int64_t nloc = block_rows(a.M, P, b);
  const int nsteps = (int)((nloc + G - 1) / G);
  float* red = reinterpret_cast<float*>(smem);  // [2][G][wpr][2]
  // The cross-group combine's slices past the row sums (dw sums, then db sums): the last step
  // hands its column sums over in the barrier of its own row sums.
  float* cbw = red + ((4 * G * wpr + 3) & ~3);
  float* cbb = cbw + (size_t)(G >> 1) * TPR * K;

  const S* wr = static_cast<const S*>(a.w);
  bool whole[ITERS], live[ITERS];
  uint32_t voff[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    live[it] = TAIL == Tail::FULL || col < N;
    whole[it] = TAIL == Tail::RAGGED ? col + V <= N : live[it];
    voff[it] = whole[it] ? (uint32_t)col * (uint32_t)sizeof(S) : 0u;
  }

  float g[ITERS][V];
  {
    const BufRsrc wb = buf_rsrc(wr);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      Raw r = IO::load_b(wb, voff[it], 0);
      if (!whole[it]) r = live[it] ? IO::load_part(at(wr, col), N - col) : IO::zero();
      IO::unpack(r, g[it]);
    }
  }
  float accw[K], accb[HAS_DB ? K : 1];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    accw[k] = 0.f;
    if constexpr (HAS_DB) accb[k] = 0.f;
  }

  Raw rx[RING][ITERS], rd[RING][ITERS];
  float rm[RING], rr[RING];
  auto load_row = [&](int slot, int s) {
    const int64_t l0 = (int64_t)s * G + g0, li = l0 + dg;
    const bool ok0 = s < nsteps && l0 < nloc, ok = s < nsteps && li < nloc;
    const int64_t row0 = b + (ok0 ? l0 : 0) * P;
    const S* xr = ok0 ? static_cast<const S*>(a.x) + row0 * a.ldx : wr;
    const S* dr = ok0 ? static_cast<const S*>(a.dy) + row0 * a.lddy : wr;
    const BufRsrc xb = buf_rsrc(xr), db = buf_rsrc(dr);
    // A lane whose own row lies past the block's share reads the wavefront's first row (or w).
    const uint32_t ex = SUB && ok ? (uint32_t)dg * dx_step : 0u;
    const uint32_t ed = SUB && ok ? (uint32_t)dg * dd_step : 0u;
    const int64_t row = SUB ? b + (ok ? li : 0) * P : row0;
    rm[slot] = a.mean[row];
    rr[slot] = a.rstd[row];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      rx[slot][it] = IO::load_b_nt(xb, voff[it] + ex, 0);
      rd[slot][it] = IO::load_b_nt(db, voff[it] + ed, 0);
      if constexpr (TAIL == Tail::RAGGED) {
        const int col = (it * TPR + tl) * V;
        if (!whole[it] && live[it]) {
          rx[slot][it] = IO::load_part(at(xr, col), N - col);
          rd[slot][it] = IO::load_part(at(dr, col), N - col);
        }
      }
    }
  };
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) load_row(j, j);

  // c1, c2 = sums / N: a multiply for exactly tiled rows (a power of two wide), else a division.
  const float inv_n = 1.0f / (float)N;

  for (int s0 = 0; s0 < nsteps; s0 += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      const int s = s0 + j;
      load_row((j + DEPTH) % RING, s + DEPTH);
      if (s < nsteps) {  // block-uniform
        const int64_t l0 = (int64_t)s * G + g0, li = l0 + dg;
        const bool valid = li < nloc;  // wave-uniform unless SUB
        const float mu = rm[j], rs = rr[j];
        float d1a = 0.f, d1b = 0.f, d2a = 0.f, d2b = 0.f;
        float kx[KEEP ? K : 1], kg[KEEP ? K : 1];
        if (valid) {
#pragma unroll
          for (int it = 0; it < ITERS; ++it) {
            if (!live[it]) continue;
            float xf[V], df[V];
            IO::unpack(rx[j][it], xf);
            IO::unpack(rd[j][it], df);
#pragma unroll
            for (int e = 0; e < V; e += 2) {
              const float xh0 = (xf[e] - mu) * rs, xh1 = (xf[e + 1] - mu) * rs;
              const float gd0 = g[it][e] * df[e], gd1 = g[it][e + 1] * df[e + 1];
              if constexpr (KEEP) {
                kx[it * V + e] = xh0;
                kx[it * V + e + 1] = xh1;
                kg[it * V + e] = gd0;
                kg[it * V + e + 1] = gd1;
              }
              accw[it * V + e] = __builtin_fmaf(df[e], xh0, accw[it * V + e]);
              accw[it * V + e + 1] = __builtin_fmaf(df[e + 1], xh1, accw[it * V + e + 1]);
              if constexpr (HAS_DB) {
                accb[it * V + e] += df[e];
                accb[it * V + e + 1] += df[e + 1];
              }
              d1a += gd0;
              d1b += gd1;
              d2a = __builtin_fmaf(gd0, xh0, d2a);
              d2b = __builtin_fmaf(gd1, xh1, d2b);
            }
            // Done here, not after the row's reduction where the compiler would otherwise sink
            // them (which keeps every vector's operands live across the reduction).
#pragma unroll
            for (int e = 0; e < V; ++e) {
              asm volatile("" : "+v"(accw[it * V + e]));
              if constexpr (HAS_DB) asm volatile("" : "+v"(accb[it * V + e]));
            }
          }
        }
        float dots[2] = {d1a + d1b, d2a + d2b};
        // After the last step's first pass the column sums are final: the first level of the
        // cross-group combine rides on this step's barrier and, with two groups or fewer, the
        // partial rows are written before the last row's dx. With two groups and a bias, group 1
        // hands over its dw sums and group 0 its db sums, so each group adds one pair (in either
        // order the same float32 sum) and writes one partial row.
        // (One vector a thread only: at two the extra live sums would spill registers.)
        const bool last = EARLY && G <= 2 && s == nsteps - 1;  // block-uniform
        const bool swap = HAS_DB && G == 2;
        if (last) {
          if (swap) {
            if (grp == 1) {
#pragma unroll
              for (int k = 0; k < K; ++k) cbw[tl * K + k] = accw[k];
            } else if constexpr (HAS_DB) {
#pragma unroll
              for (int k = 0; k < K; ++k) cbb[tl * K + k] = accb[k];
            }
          } else {
            combine_give<K>(accw, cbw, G, grp, tl, TPR);
            if constexpr (HAS_DB) combine_give<K>(accb, cbb, G, grp, tl, TPR);
          }
        }
        if constexpr (SUB > 0) {
          dots[0] = segment_sum<SUB>(dots[0]);
          dots[1] = segment_sum<SUB>(dots[1]);
        } else {
          group_sum_batch<2, WPR>(dots, red + ((s & 1) * G + grp) * wpr * 2, wpr, tl);
        }
        if (last) {
          if (!(WPR > 1 || (WPR == 0 && wpr > 1))) lds_barrier();  // one-wave rows: no barrier yet
          if (swap) {
            if (grp == 0) {
#pragma unroll
              for (int k = 0; k < K; ++k) accw[k] += cbw[tl * K + k];
              store_partial<ITERS, V>(accw, a.part + (int64_t)b * a.ldp, TPR, tl, N);
            } else if constexpr (HAS_DB) {
#pragma unroll
              for (int k = 0; k < K; ++k) accb[k] += cbb[tl * K + k];
              store_partial<ITERS, V>(accb, a.part + (int64_t)(P + b) * a.ldp, TPR, tl, N);
            }
          } else {
            combine_take<K>(accw, cbw, G, grp, tl, TPR);
            if constexpr (HAS_DB) combine_take<K>(accb, cbb, G, grp, tl, TPR);
            if (G - (G >> 1) == 1 && grp == 0) {
              store_partial<ITERS, V>(accw, a.part + (int64_t)b * a.ldp, TPR, tl, N);
              if constexpr (HAS_DB)
                store_partial<ITERS, V>(accb, a.part + (int64_t)(P + b) * a.ldp, TPR, tl, N);
            }
          }
        }
        if (valid) {
          const int64_t row0 = b + l0 * P;  // l0 <= li: the wavefront's first row is valid too
          const float c1 = TAIL == Tail::FULL ? dots[0] * inv_n : dots[0] / (float)N;
          const float c2 = TAIL == Tail::FULL ? dots[1] * inv_n : dots[1] / (float)N;
          S* dxr = static_cast<S*>(a.dx) + row0 * a.lddx;
          const BufRsrc ob = buf_rsrc(dxr);
          const uint32_t eo = SUB ? (uint32_t)dg * do_step : 0u;
#pragma unroll
          for (int it = 0; it < ITERS; ++it) {
            if (!live[it]) continue;
            float o[V];
            if constexpr (KEEP) {
#pragma unroll
              for (int e = 0; e < V; ++e)
                o[e] = rs * ((kg[it * V + e] - c1) - kx[it * V + e] * c2);
            } else {
              float xf[V], df[V];
              IO::unpack(rx[j][it], xf);
              IO::unpack(rd[j][it], df);
#pragma unroll
              for (int e = 0; e < V; ++e) {
                const float xh = (xf[e] - mu) * rs;
                const float gd = g[it][e] * df[e];
                o[e] = rs * ((gd - c1) - xh * c2);
              }
            }
            const Raw out = IO::pack(o);
            if (whole[it]) IO::store_b(ob, voff[it] + eo, 0, out);
            else IO::store_part(at(dxr, (it * TPR + tl) * V), out, N - (it * TPR + tl) * V);
          }
        }
      }
    }
  }

  if constexpr (ITERS == 1) {
    if (SUB > 0 || G >= 4) {  // four or more row groups: the column combine, dw then db
      float* buf = reinterpret_cast<float*>(smem);
      combine_columns<V>(accw, buf, grp, tl, TPR, a.part + (int64_t)b * a.ldp, N);
      if constexpr (HAS_DB)
        combine_columns<V>(accb, buf, grp, tl, TPR, a.part + (int64_t)(P + b) * a.ldp, N);
      return;
    }
  }
  // Without the early first level (no rows, or two vectors a thread) the whole tree runs here;
  // with it and two groups, nothing is left.
  const bool early = EARLY && G <= 2 && nsteps > 0;
  const int rest = early ? G - (G >> 1) : G;
  if (rest > 1 || !early) {
    combine_groups<K>(accw, cbw, rest, grp, tl, TPR);
    if (grp == 0) store_partial<ITERS, V>(accw, a.part + (int64_t)b * a.ldp, TPR, tl, N);
    if constexpr (HAS_DB) {
      combine_groups<K>(accb, cbb, rest, grp, tl, TPR);
      if (grp == 0) store_partial<ITERS, V>(accb, a.part + (int64_t)(P + b) * a.ldp, TPR, tl, N);
    }
  }
}

// Rows that are not 16-byte aligned, x and dy rows at one offset from a 16-byte boundary, at most one
// whole vector per lane: the RMSNorm backward's peeled register kernel (bwd_peel_rows_kernel) with
// the two row sums c1, c2 and the mean: G row groups on the persistent grid, the next row's x, dy,
// mean, rstd and gain loaded one step ahead (all unconditionally), a lane's head element first in
// its even sums and its tail element last in its odd sums, dw and db sums of each group in LDS
// (columns at peel_col; the dw arrays of the G groups, then the db arrays), added in group order
// into the block's two partial rows at the end. w must be 16-byte aligned.
template <DT D, bool HAS_DB>
__global__ void __launch_bounds__(1024) ln_bwd_peel_rows_kernel(LnBwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, G = a.groups, N = a.N;
  const int tid = threadIdx.x;
  const int grp = wave_group(tid, TPR);
  const int tl = tid - grp * TPR;
  const int b = blockIdx.x, P = a.P;
  const int64_t nloc = block_rows(a.M, P, b);
  const int nsteps = (int)((nloc + G - 1) / G);
  const int stride = (int)peel_sum_floats(a.ldp);
  float* red = reinterpret_cast<float*>(smem);            // [2][G][wpr][2]
  float* const sw0 = red + ((4 * G * wpr + 3) & ~3);      // [G][stride] dw sums
  float* const sb0 = sw0 + (size_t)G * stride;            // [G][stride] db sums
  float* const sw = sw0 + (size_t)grp * stride;
  float* const sb = sb0 + (size_t)grp * stride;
  for (int c = tl; c < N; c += TPR) {
    sw[peel_col(c)] = 0.f;
    if constexpr (HAS_DB) sb[peel_col(c)] = 0.f;
  }

  const S* wr = static_cast<const S*>(a.w);
  const BufRsrc wb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<S*>(wr), 0, (N * (int)sizeof(S) + 15) & ~15, kBufDword3);

  Raw rx[2], rd[2], wa[2], wv[2];
  S hx[2], hd[2], hw[2], tx[2], td[2], tw[2];
  float rm[2], rr[2];
  int hh[2];
  auto load_row = [&](int slot, int s) {
    const int64_t li = (int64_t)s * G + grp;
    const bool ok = s < nsteps && li < nloc;
    const int64_t row = b + (ok ? li : 0) * P;
    const S* xr = static_cast<const S*>(a.x) + row * a.ldx;
    const S* dr = static_cast<const S*>(a.dy) + row * a.lddy;
    const int h = peel_head(xr, N);
    const int nb = (N - h) / V;
    const int t = N - h - nb * V;
    hh[slot] = h;
    const uint32_t vo = (uint32_t)((tl < nb ? tl : 0) * V) * (uint32_t)sizeof(S);
    rx[slot] = IO::load_b_nt(buf_rsrc(xr), vo + (uint32_t)h * (uint32_t)sizeof(S), 0);
    rd[slot] = IO::load_b_nt(buf_rsrc(dr), vo + (uint32_t)h * (uint32_t)sizeof(S), 0);
    wa[slot] = IO::load_b(wb, vo, 0);
    wv[slot] = IO::load_b(wb, vo + 16u, 0);
    const int hi = tl < h ? tl : 0;
    const int ti = t > 0 ? h + nb * V + (tl < t ? tl : 0) : 0;
    hx[slot] = xr[hi];
    hd[slot] = dr[hi];
    hw[slot] = wr[hi];
    tx[slot] = xr[ti];
    td[slot] = dr[ti];
    tw[slot] = wr[ti];
    rm[slot] = a.mean[row];
    rr[slot] = a.rstd[row];
  };
  load_row(0, 0);

  for (int s0 = 0; s0 < nsteps; s0 += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int s = s0 + j;
      load_row(j ^ 1, s + 1);
      if (s >= nsteps) continue;  // block-uniform
      const int64_t li = (int64_t)s * G + grp;
      const bool valid = li < nloc;  // wave-uniform
      const int h = hh[j];
      const int nb = (N - h) / V;
      const int t = N - h - nb * V;
      const int t0 = h + nb * V;
      const float mu = rm[j], rs = rr[j];
      float xh[V], gd[V], df[V];
      float hxh = 0.f, hgd = 0.f, hdy = 0.f, txh = 0.f, tgd = 0.f, tdy = 0.f;
      float d1a = 0.f, d1b = 0.f, d2a = 0.f, d2b = 0.f;
      {
        float xf[V], wf[V];
        IO::unpack(rx[j], xf);
        IO::unpack(rd[j], df);
        IO::unpack(peel_vec<D>(h, wa[j], wv[j]), wf);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xh[e] = (xf[e] - mu) * rs;
          gd[e] = wf[e] * df[e];
        }
      }
      if (valid) {
        if (tl < h) {
          hxh = (to_f32<D>(hx[j]) - mu) * rs;
          hdy = to_f32<D>(hd[j]);
          hgd = to_f32<D>(hw[j]) * hdy;
          d1a += hgd;
          d2a = __builtin_fmaf(hgd, hxh, d2a);
        }
        if (tl < nb) {
#pragma unroll
          for (int e = 0; e < V; e += 2) {
            d1a += gd[e];
            d1b += gd[e + 1];
            d2a = __builtin_fmaf(gd[e], xh[e], d2a);
            d2b = __builtin_fmaf(gd[e + 1], xh[e + 1], d2b);
          }
        }
        if (tl < t) {
          txh = (to_f32<D>(tx[j]) - mu) * rs;
          tdy = to_f32<D>(td[j]);
          tgd = to_f32<D>(tw[j]) * tdy;
          d1b += tgd;
          d2b = __builtin_fmaf(tgd, txh, d2b);
        }
      }
      float dots[2] = {d1a + d1b, d2a + d2b};
      group_sum_batch<2>(dots, red + ((s & 1) * G + grp) * wpr * 2, wpr, tl);
      if (wpr == 1) lds_barrier();  // orders the LDS sums of consecutive rows (no barrier above)
      if (!valid) continue;
      const float c1 = dots[0] / (float)N, c2 = dots[1] / (float)N;
      S* dxr = static_cast<S*>(a.dx) + (b + li * P) * a.lddx;
      auto sums = [&](int c, float dyv, float xhv) {
        const int k = peel_col(c);
        sw[k] = __builtin_fmaf(dyv, xhv, sw[k]);
        if constexpr (HAS_DB) sb[k] += dyv;
      };
      if (tl < h) {
        dxr[tl] = from_f32<D>(rs * ((hgd - c1) - hxh * c2));
        sums(tl, hdy, hxh);
      }
      if (tl < nb) {
        const int col = h + tl * V;
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          o[e] = rs * ((gd[e] - c1) - xh[e] * c2);
          sums(col + e, df[e], xh[e]);
        }
        const Raw out = IO::pack(o);
        if (a.dxvec) IO::store(at(dxr, col), out);
        else IO::store_part(at(dxr, col), out, V);
      }
      if (tl < t) {
        dxr[t0 + tl] = from_f32<D>(rs * ((tgd - c1) - txh * c2));
        sums(t0 + tl, tdy, txh);
      }
    }
  }
  lds_barrier();  // every group's last sums are in LDS
  float* const pw = a.part + (int64_t)b * a.ldp;
  float* const pb = a.part + (int64_t)(P + b) * a.ldp;
  for (int c = tid; c < N; c += G * TPR) {
    float v = sw0[peel_col(c)];
    for (int g = 1; g < G; ++g) v += sw0[(size_t)g * stride + peel_col(c)];
    pw[c] = v;
    if constexpr (HAS_DB) {
      float u = sb0[peel_col(c)];
      for (int g = 1; g < G; ++g) u += sb0[(size_t)g * stride + peel_col(c)];
      pb[c] = u;
    }
  }
}

// Any N and any alignment. One row at a time per block; the elementwise pass reads x and dy again.
// KREG = 0: the block's dw (and db) partial rows accumulate in the workspace itself (each column
// owned by one thread, rows added in order). KREG > 0 (16-byte vectors, at most KREG per thread):
// the same sums in registers, written once at the end; bit-identical to KREG = 0.
template <DT D, bool WIDE, bool HAS_DB, int KREG = 0, bool LACC = false>
__global__ void __launch_bounds__(1024) ln_bwd_stream_kernel(LnBwdArgs a) {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  static_assert(KREG == 0 || WIDE, "register sums take 16-byte vectors");
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int nv = (N + V - 1) / V;
  const int tl = threadIdx.x;
  const int b = blockIdx.x, P = a.P;
  float* red = reinterpret_cast<float*>(smem);  // [2][wpr][2]
  const S* wr = static_cast<const S*>(a.w);
  float* const gw = a.part + (int64_t)b * a.ldp;
  float* const gb = a.part + (int64_t)(P + b) * a.ldp;
  static_assert(!LACC || KREG == 0, "LDS sums replace the workspace sums");
  // The row's dw and db sums: LDS (after the 64-float reduction area, ldp floats each) or the
  // workspace rows themselves.
  float* const pw = LACC ? reinterpret_cast<float*>(smem) + 64 : gw;
  float* const pb = LACC ? reinterpret_cast<float*>(smem) + 64 + a.ldp : gb;
  constexpr int K = KREG > 0 ? KREG * V : 1;
  float accw[K], accb[HAS_DB ? K : 1];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    accw[k] = 0.f;
    if constexpr (HAS_DB) accb[k] = 0.f;
  }

  if constexpr (KREG == 0) {
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (col + e < N) {
          pw[col + e] = 0.f;
          if constexpr (HAS_DB) pb[col + e] = 0.f;
        }
      }
    }
  }

  int s = 0;
  for (int64_t row = b; row < a.M; row += P, ++s) {
    const S* xr = static_cast<const S*>(a.x) + row * a.ldx;
    const S* dr = static_cast<const S*>(a.dy) + row * a.lddy;
    const float mu = a.mean[row], rs = a.rstd[row];
    const bool comp = a.comp != 0;
    RowAcc d1, d2;
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      const bool full = col + V <= N;
      float xf[V], df[V], wf[V];
      IO::unpack(full ? IO::load(xr + col) : IO::load_part(xr + col, N - col), xf);
      IO::unpack(full ? IO::load(dr + col) : IO::load_part(dr + col, N - col), df);
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (xf[e] - mu) * rs;
        const float gd = wf[e] * df[e];
        d1.add(e, gd, comp);
        d2.fma(e, gd, xh, comp);
      }
    }
    float dots[2] = {d1.total(), d2.total()};
    group_sum_batch<2>(dots, red + (s & 1) * wpr * 2, wpr, tl);
    const float c1 = dots[0] / (float)N, c2 = dots[1] / (float)N;
    S* dxr = static_cast<S*>(a.dx) + row * a.lddx;
    auto elementwise = [&](int v, float* aw, float* ab) {
      const int col = v * V;
      const bool full = col + V <= N;
      float xf[V], df[V], wf[V], o[V];
      // the row's last read of x and dy: non-temporal
      IO::unpack(full ? IO::load_nt(xr + col) : IO::load_part(xr + col, N - col), xf);
      IO::unpack(full ? IO::load_nt(dr + col) : IO::load_part(dr + col, N - col), df);
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = (xf[e] - mu) * rs;
        const float gd = wf[e] * df[e];
        o[e] = rs * ((gd - c1) - xh * c2);
        if constexpr (KREG > 0) {
          aw[e] = __builtin_fmaf(df[e], xh, aw[e]);
          if constexpr (HAS_DB) ab[e] += df[e];
        } else if (col + e < N) {
          pw[col + e] = __builtin_fmaf(df[e], xh, pw[col + e]);
          if constexpr (HAS_DB) pb[col + e] += df[e];
        }
      }
      const auto out = IO::pack(o);
      if (full) IO::store(dxr + col, out);
      else IO::store_part(dxr + col, out, N - col);
    };
    if constexpr (KREG > 0) {
#pragma unroll
      for (int k = 0; k < KREG; ++k) {
        const int v = tl + k * TPR;
        if (v < nv) elementwise(v, accw + k * V, HAS_DB ? accb + k * V : nullptr);
        // One vector at a time, its sums done here (see the RMSNorm streaming kernel).
#pragma unroll
        for (int e = 0; e < V; ++e) {
          asm volatile("" : "+v"(accw[k * V + e]));
          if constexpr (HAS_DB) asm volatile("" : "+v"(accb[k * V + e]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int v = tl; v < nv; v += TPR) elementwise(v, nullptr, nullptr);
    }
  }

  if constexpr (KREG > 0) {
#pragma unroll
    for (int k = 0; k < KREG; ++k) {
      const int col = (tl + k * TPR) * V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (col + e < N) {
          gw[col + e] = accw[k * V + e];
          if constexpr (HAS_DB) gb[col + e] = accb[k * V + e];
        }
      }
    }
  } else if constexpr (LACC) {
    // each thread copies the columns it summed: no barrier needed
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (col + e < N) {
          gw[col + e] = pw[col + e];
          if constexpr (HAS_DB) gb[col + e] = pb[col + e];
        }
      }
    }
  }
}

}  // namespace rmsn
