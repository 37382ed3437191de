// RMSNorm backward kernels.
//
// Per row, with rstd read from the forward's float32 cache, every operation one float32 operation
// and inputs upcast on load (candle pull request 4059, "Add backward passes to the fused rms_norm,
// layer_norm and softmax_last_dim ops"; Liger-Kernel pull request 1608, "fix(group_norm): keep the
// backward statistics and reductions in fp32", Summary):
//   xhat = x * rstd,  gdy = g * dy  (g = offset + w),  c = (sum_j gdy_j * xhat_j) / N
//   dx   = T(rstd * (gdy - xhat * c))
//   dw_j = sum over rows of dy_j * xhat_j         (float32; Liger-Kernel pull request 92 keeps the
//                                                   weight gradient in float32)
//
// dw without atomics: the rows are split into P contiguous, balanced chunks, one per block of a
// persistent grid (P depends only on M, so the result does not depend on the device). A block's
// threads keep float32 column accumulators in registers while they walk the chunk, combine them
// across the block's row groups in a fixed tree order, and write one partial row of a
// [P, ldp] float32 workspace. A second kernel adds the P partial rows in a fixed order.
#pragma once

#include "rmsnorm_common.hpp"

namespace rmsn {

// Partial rows of the dw workspace: one per block; a function of M only.
constexpr int kMaxPartials = 256;
inline int64_t num_partials(int64_t M) { return M < kMaxPartials ? M : kMaxPartials; }
// Row stride of the workspace in floats (16-byte aligned rows).
inline int64_t partial_ld(int64_t N) { return (N + 3) & ~int64_t(3); }

struct BwdArgs {
  const void* dy;
  const void* x;
  const void* w;
  const float* rstd;
  void* dx;
  float* part;  // [P, ldp]
  int64_t lddy, ldx, lddx, M;
  int N, ldp, P;
  int tpr;     // threads per row, multiple of 64
  int groups;  // rows processed concurrently per block
  float offset;
};

// Fixed-order tree combine of per-group column accumulators into group 0. `buf` holds
// floor(groups / 2) slices of slice_floats floats. Every thread of the block must call it.
template <int K>
__device__ __forceinline__ void combine_groups(float (&acc)[K], float* buf, int groups, int grp,
                                               int tl, int slice_threads) {
  int n = groups;
  while (n > 1) {
    const int h = n >> 1;
    lds_barrier();  // previous readers of buf are done
    if (grp >= n - h && grp < n) {
      float* dst = buf + ((size_t)(grp - (n - h)) * slice_threads + tl) * K;
#pragma unroll
      for (int k = 0; k < K; ++k) dst[k] = acc[k];
    }
    lds_barrier();
    if (grp >= n - 2 * h && grp < n - h) {
      const float* src = buf + ((size_t)(grp - (n - 2 * h)) * slice_threads + tl) * K;
#pragma unroll
      for (int k = 0; k < K; ++k) acc[k] += src[k];
    }
    n -= h;
  }
}

// Write a block's combined column accumulators as partial row b of the workspace (group 0 only).
template <int ITERS, int V>
__device__ __forceinline__ void store_partial(const float (&acc)[ITERS * V], float* pr, int TPR,
                                              int tl, int N) {
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (col + V <= N) {
#pragma unroll
      for (int q = 0; q < V; q += 4)
        *reinterpret_cast<float4*>(pr + col + q) =
            make_float4(acc[it * V + q], acc[it * V + q + 1], acc[it * V + q + 2],
                        acc[it * V + q + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (col + e < N) pr[col + e] = acc[it * V + e];
    }
  }
}

// Register kernel: a row group keeps its row's xhat and g*dy in registers between the reduction
// and the elementwise pass, and prefetches the next row of its chunk into registers while the
// current one is reduced. The gain g = offset + w stays in registers for the whole chunk.
template <DT D, int ITERS>
__global__ void __launch_bounds__(1024) bwd_rows_kernel(BwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, G = a.groups, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int b = blockIdx.x;
  const int64_t r0 = (int64_t)b * a.M / a.P;
  const int64_t r1 = (int64_t)(b + 1) * a.M / a.P;
  const int nsteps = (int)((r1 - r0 + G - 1) / G);
  float* red = reinterpret_cast<float*>(smem);  // [2][G * wpr]

  const S* dyb = static_cast<const S*>(a.dy);
  const S* xb = static_cast<const S*>(a.x);
  S* dxb = static_cast<S*>(a.dx);

  float g[ITERS][V];
  {
    const S* wr = static_cast<const S*>(a.w);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      Raw r = IO::zero();
      if (col + V <= N) r = IO::load(wr + col);
      else if (col < N) r = IO::load_part(wr + col, N - col);
      float wf[V];
      IO::unpack(r, wf);
#pragma unroll
      for (int e = 0; e < V; ++e) g[it][e] = a.offset + wf[e];
    }
  }
  float acc[ITERS * V];
#pragma unroll
  for (int k = 0; k < ITERS * V; ++k) acc[k] = 0.f;

  Raw nx[ITERS], nd[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) nx[it] = nd[it] = IO::zero();
  auto load_row = [&](int64_t row) {
    const S* xr = xb + row * a.ldx;
    const S* dr = dyb + row * a.lddy;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      if (col + V <= N) {
        nx[it] = IO::load(xr + col);
        nd[it] = IO::load(dr + col);
      } else if (col < N) {
        nx[it] = IO::load_part(xr + col, N - col);
        nd[it] = IO::load_part(dr + col, N - col);
      }
    }
  };
  if (r0 + grp < r1) load_row(r0 + grp);

  for (int s = 0; s < nsteps; ++s) {
    const int64_t row = r0 + (int64_t)s * G + grp;
    const bool valid = row < r1;
    Raw cx[ITERS], cd[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      cx[it] = nx[it];
      cd[it] = nd[it];
    }
    if (row + G < r1) load_row(row + G);  // prefetch; consumed next step
    const float rs = valid ? a.rstd[row] : 0.f;

    float xh[ITERS][V], gdy[ITERS][V];
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      float xf[V], df[V];
      IO::unpack(cx[it], xf);
      IO::unpack(cd[it], df);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xh[it][e] = xf[e] * rs;
        gdy[it][e] = g[it][e] * df[e];
        acc[it * V + e] = __builtin_fmaf(df[e], xh[it][e], acc[it * V + e]);
      }
#pragma unroll
      for (int e = 0; e < V; e += 2) {
        d0 = __builtin_fmaf(gdy[it][e], xh[it][e], d0);
        d1 = __builtin_fmaf(gdy[it][e + 1], xh[it][e + 1], d1);
      }
    }
    const float dot = group_sum(d0 + d1, red + (s & 1) * G * wpr + grp * wpr, wpr, tl);
    const float c = dot / (float)N;
    if (valid) {
      S* dxr = dxb + row * a.lddx;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int col = (it * TPR + tl) * V;
        if (col >= N) continue;
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = rs * (gdy[it][e] - xh[it][e] * c);
        const Raw out = IO::pack(o);
        if (col + V <= N) IO::store(dxr + col, out);
        else IO::store_part(dxr + col, out, N - col);
      }
    }
  }

  combine_groups<ITERS * V>(acc, reinterpret_cast<float*>(smem), G, grp, tl, TPR);
  if (grp == 0) store_partial<ITERS, V>(acc, a.part + (int64_t)b * a.ldp, TPR, tl, N);
}

// LDS-staged kernel for rows too wide to keep in registers (e.g. N = 32768 in 16-bit types): the
// raw x and dy of the current row are written to LDS as they arrive and read back for the
// elementwise pass, so registers hold only the column accumulators and one row's loads in flight.
// The gain is re-read from w (cache-resident) in each pass. Same thread-to-element mapping and
// summation order as the register kernel, so dx is bit-identical to it for the same shape.
template <DT D, int ITERS>
__global__ void __launch_bounds__(1024) bwd_lds_kernel(BwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, G = a.groups, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int b = blockIdx.x;
  const int64_t r0 = (int64_t)b * a.M / a.P;
  const int64_t r1 = (int64_t)(b + 1) * a.M / a.P;
  const int nsteps = (int)((r1 - r0 + G - 1) / G);
  float* red = reinterpret_cast<float*>(smem);                                    // [2][G * wpr]
  Raw* stage = smem + ((2 * G * wpr + 3) >> 2) + (size_t)grp * 2 * ITERS * TPR;  // [G][2][ITERS*TPR]

  const S* wr = static_cast<const S*>(a.w);
  float acc[ITERS * V];
#pragma unroll
  for (int k = 0; k < ITERS * V; ++k) acc[k] = 0.f;

  for (int s = 0; s < nsteps; ++s) {
    const int64_t row = r0 + (int64_t)s * G + grp;
    const bool valid = row < r1;
    const int64_t lrow = valid ? row : r0;
    const S* xr = static_cast<const S*>(a.x) + lrow * a.ldx;
    const S* dr = static_cast<const S*>(a.dy) + lrow * a.lddy;
    Raw rx[ITERS], rd[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      rx[it] = rd[it] = IO::zero();
      if (valid) {
        if (col + V <= N) {
          rx[it] = IO::load(xr + col);
          rd[it] = IO::load(dr + col);
        } else if (col < N) {
          rx[it] = IO::load_part(xr + col, N - col);
          rd[it] = IO::load_part(dr + col, N - col);
        }
      }
    }
    const float rs = valid ? a.rstd[row] : 0.f;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      stage[it * TPR + tl] = rx[it];
      stage[(ITERS + it) * TPR + tl] = rd[it];
      Raw rw = IO::zero();
      if (col + V <= N) rw = IO::load(wr + col);
      else if (col < N) rw = IO::load_part(wr + col, N - col);
      float xf[V], df[V], wf[V];
      IO::unpack(rx[it], xf);
      IO::unpack(rd[it], df);
      IO::unpack(rw, wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = xf[e] * rs;
        const float gd = (a.offset + wf[e]) * df[e];
        acc[it * V + e] = __builtin_fmaf(df[e], xh, acc[it * V + e]);
        if (e & 1) d1 = __builtin_fmaf(gd, xh, d1);
        else d0 = __builtin_fmaf(gd, xh, d0);
      }
    }
    const float dot = group_sum(d0 + d1, red + (s & 1) * G * wpr + grp * wpr, wpr, tl);
    const float c = dot / (float)N;
    if (valid) {
      S* dxr = static_cast<S*>(a.dx) + row * a.lddx;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int col = (it * TPR + tl) * V;
        if (col >= N) continue;
        Raw rw = (col + V <= N) ? IO::load(wr + col) : IO::load_part(wr + col, N - col);
        float xf[V], df[V], wf[V], o[V];
        IO::unpack(stage[it * TPR + tl], xf);
        IO::unpack(stage[(ITERS + it) * TPR + tl], df);
        IO::unpack(rw, wf);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float xh = xf[e] * rs;
          const float gd = (a.offset + wf[e]) * df[e];
          o[e] = rs * (gd - xh * c);
        }
        const Raw out = IO::pack(o);
        if (col + V <= N) IO::store(dxr + col, out);
        else IO::store_part(dxr + col, out, N - col);
      }
    }
  }

  combine_groups<ITERS * V>(acc, reinterpret_cast<float*>(smem), G, grp, tl, TPR);
  if (grp == 0) store_partial<ITERS, V>(acc, a.part + (int64_t)b * a.ldp, TPR, tl, N);
}

// Any N and any alignment. One row at a time per block (groups = 1); the elementwise pass reads
// x and dy again, and the block's dw partial row accumulates in the workspace itself (each column
// is owned by one thread, rows are added in order).
template <DT D, bool WIDE>
__global__ void __launch_bounds__(1024) bwd_stream_kernel(BwdArgs a) {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int nv = (N + V - 1) / V;
  const int tl = threadIdx.x;
  const int b = blockIdx.x;
  const int64_t r0 = (int64_t)b * a.M / a.P;
  const int64_t r1 = (int64_t)(b + 1) * a.M / a.P;
  float* red = reinterpret_cast<float*>(smem);  // [2][wpr]
  const S* wr = static_cast<const S*>(a.w);
  float* pr = a.part + (int64_t)b * a.ldp;

  for (int v = tl; v < nv; v += TPR) {
    const int col = v * V;
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (col + e < N) pr[col + e] = 0.f;
  }

  int s = 0;
  for (int64_t row = r0; row < r1; ++row, ++s) {
    const S* xr = static_cast<const S*>(a.x) + row * a.ldx;
    const S* dr = static_cast<const S*>(a.dy) + row * a.lddy;
    const float rs = a.rstd[row];
    float d0 = 0.f, d1 = 0.f;
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      const bool full = col + V <= N;
      float xf[V], df[V], wf[V];
      IO::unpack(full ? IO::load(xr + col) : IO::load_part(xr + col, N - col), xf);
      IO::unpack(full ? IO::load(dr + col) : IO::load_part(dr + col, N - col), df);
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = xf[e] * rs;
        const float gd = (a.offset + wf[e]) * df[e];
        if (e & 1) d1 = __builtin_fmaf(gd, xh, d1);
        else d0 = __builtin_fmaf(gd, xh, d0);
      }
    }
    const float dot = group_sum(d0 + d1, red + (s & 1) * wpr, wpr, tl);
    const float c = dot / (float)N;
    S* dxr = static_cast<S*>(a.dx) + row * a.lddx;
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      const bool full = col + V <= N;
      float xf[V], df[V], wf[V], o[V];
      IO::unpack(full ? IO::load(xr + col) : IO::load_part(xr + col, N - col), xf);
      IO::unpack(full ? IO::load(dr + col) : IO::load_part(dr + col, N - col), df);
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = xf[e] * rs;
        const float gd = (a.offset + wf[e]) * df[e];
        o[e] = rs * (gd - xh * c);
        if (col + e < N) pr[col + e] = __builtin_fmaf(df[e], xh, pr[col + e]);
      }
      const auto out = IO::pack(o);
      if (full) IO::store(dxr + col, out);
      else IO::store_part(dxr + col, out, N - col);
    }
  }
}

// dw_j = sum over p of part[p, j], p in a fixed order: wave k of the block adds partial rows
// k, k + 16, ... ; then the 16 wave sums are added in wave order. One column per lane.
__global__ void __launch_bounds__(1024) dw_reduce_kernel(const float* part, int64_t ldp, int P,
                                                         int N, float* dw) {
  __shared__ float buf[16][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (col < N) {
    for (int p = wv; p < P; p += 16) s += part[(int64_t)p * ldp + col];
  }
  buf[wv][lane] = s;
  __syncthreads();
  if (wv == 0 && col < N) {
    float t = buf[0][lane];
#pragma unroll
    for (int k = 1; k < 16; ++k) t += buf[k][lane];
    dw[col] = t;
  }
}

__global__ void fill_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace rmsn
