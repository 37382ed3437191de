// RMSNorm forward kernels.
//
// Per row (blog post "Den dolda avrundningen i RMSNorm", sections "En välbekant operation" and
// "Två ställen att avrunda"):
//   rstd = 1 / sqrt(sum(x^2) / N + eps)           float32; epsilon under the root
//   xhat = x * rstd                                 formed first
//   y    = T(float(T(xhat)) * g)   (round twice)    or   T(xhat * g)   (round once),  g = offset + w
//   y8   = FP8(fl(xhat * g) * scale)                  (8-bit output; the blog post's section "Var
//                                                      implementationerna skiljer sig" and footnote
//                                                      3: normalization, gain and the per-tensor
//                                                      scale in float32, then one cast)
//
// Work decomposition: a row is owned by a group of TPR threads (TPR = 64 * wpr, one or more
// wavefronts); a block holds `groups` such rows. Thread tl of a group owns the 16-byte vectors
// it * TPR + tl (it = 0 .. ITERS-1) of its row, so every wavefront load is one contiguous
// 64 x 16 B = 1 KiB segment. Summation order of the squares is fixed by this mapping: per thread,
// two accumulators (even / odd element of each vector) over it = 0, 1, ...; then the wave
// reduction; then the waves of the row in order. All three kernel families below use the same
// mapping for the same TPR, so their rstd and y are bit-identical.
#pragma once

#include "rmsnorm_common.hpp"

namespace rmsn {

struct FwdArgs {
  const void* x;
  const void* w;
  void* y;      // T elements, or bytes for the 8-bit outputs
  float* rstd;  // may be null
  int64_t ldx, ldy, M;
  int N;
  int tpr;     // threads per row, multiple of 64
  int groups;  // rows per block
  int yvec;    // y and ldy allow one vector store per 16-byte input vector
  int comp;    // streaming kernel: compensated row sums (long per-thread chains)
  float eps, offset, scale;
};

// Output of the forward: the two rounding conventions in T, or an OCP 8-bit format.
enum class Out : int { ONCE = 0, TWICE = 1, E4M3 = 2, E5M2 = 3 };
constexpr bool is_f8(Out o) { return o == Out::E4M3 || o == Out::E5M2; }
constexpr F8 f8_of(Out o) { return o == Out::E4M3 ? F8::E4M3 : F8::E5M2; }

template <DT D, Out O, int V>
__device__ __forceinline__ void apply_gain(const float (&xf)[V], const float (&wf)[V], float rs,
                                           float offset, float scale, float (&yf)[V]) {
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const float xh = xf[e] * rs;
    const float g = offset + wf[e];
    if constexpr (O == Out::TWICE) yf[e] = round_trip<D>(xh) * g;
    else if constexpr (O == Out::ONCE) yf[e] = xh * g;
    else yf[e] = materialize(xh * g) * scale;
  }
}

// Writes V output values at element column `col` of row yr (n valid values): T elements through
// VecIO, or one byte per value for the 8-bit outputs (a 16-byte input vector of 8 16-bit values
// gives 8 bytes, of 4 float32 values 4 bytes). `vec` (uniform) allows the single vector store;
// without it the values go out one element at a time, so the alignment of y never changes the
// kernel's loads or its summation order.
template <DT D, Out O, bool WIDE, int V>
__device__ __forceinline__ void store_out(void* yrow, int col, int n, bool vec,
                                          const float (&yf)[V]) {
  if constexpr (!is_f8(O)) {
    using IO = VecIO<D, WIDE>;
    using S = typename IO::S;
    S* yr = static_cast<S*>(yrow);
    const auto out = IO::pack(yf);
    if (vec && n >= V) IO::store(yr + col, out);
    else IO::store_part(yr + col, out, n);
  } else {
    constexpr F8 F = f8_of(O);
    uint8_t* yr = static_cast<uint8_t*>(yrow) + col;
    if constexpr (V == 8) {
      if (vec && n >= 8) {
        typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t v = {cvt4_f8<F>(yf[0], yf[1], yf[2], yf[3]),
                           cvt4_f8<F>(yf[4], yf[5], yf[6], yf[7])};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(yr));
        return;
      }
    } else if constexpr (V == 4) {
      if (vec && n >= 4) {
        __builtin_nontemporal_store(cvt4_f8<F>(yf[0], yf[1], yf[2], yf[3]),
                                    reinterpret_cast<uint32_t*>(yr));
        return;
      }
    }
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (e < n) yr[e] = cvt1_f8<F>(yf[e]);
  }
}

// Row pointer of the output (element stride ldy; bytes for the 8-bit outputs).
template <DT D, Out O>
__device__ __forceinline__ void* out_row(void* y, int64_t row, int64_t ldy) {
  if constexpr (is_f8(O)) return static_cast<uint8_t*>(y) + row * ldy;
  else return static_cast<typename Elem<D>::S*>(y) + row * ldy;
}

// Row held in registers (STAGE_LDS = false) or staged in LDS (true) between the two passes.
// FULL: the host has checked N = ITERS * TPR * V (the threads' vectors tile the row exactly), and
// the kernel carries no partial-vector code.
// SUB > 0: rows of at most SUB vectors (SUB = 4 to 32) take row groups of SUB lanes, 64 / SUB rows
// per wavefront, summed with segment_sum; the lanes hold the vectors they hold at TPR = 64 and the
// sum comes out bit for bit as wave_sum's, so rstd and y do not change, only how many lanes idle.
template <DT D, int ITERS, Out O, bool STAGE_LDS, bool FULL = false, int SUB = 0>
__global__ void __launch_bounds__(1024) fwd_rows_kernel(FwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  static_assert(SUB == 0 || (ITERS == 1 && !STAGE_LDS), "narrow rows: one vector per lane");
  extern __shared__ uint4 smem[];

  const int TPR = SUB ? SUB : a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;

  float* red = reinterpret_cast<float*>(smem) + grp * wpr;
  Raw* stage = smem + ((a.groups * wpr + 3) >> 2) + (size_t)grp * ITERS * TPR;

  const S* xr = static_cast<const S*>(a.x) + (valid ? row : 0) * a.ldx;
  const S* wr = static_cast<const S*>(a.w);
  Raw raw[ITERS], wraw[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    Raw r = IO::zero(), rw = IO::zero();
    if (valid) {
      if (FULL || col + V <= N) {
        r = IO::load_nt(xr + col);
        rw = IO::load(wr + col);
      } else if (col < N) {
        r = IO::load_part(xr + col, N - col);
        rw = IO::load_part(wr + col, N - col);
      }
    }
    raw[it] = r;
    wraw[it] = rw;
  }
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    float f[V];
    IO::unpack(raw[it], f);
#pragma unroll
    for (int e = 0; e < V; e += 2) {
      acc0 = __builtin_fmaf(f[e], f[e], acc0);
      acc1 = __builtin_fmaf(f[e + 1], f[e + 1], acc1);
    }
    if constexpr (STAGE_LDS) stage[it * TPR + tl] = raw[it];
  }
  float ss;
  if constexpr (SUB > 0) ss = segment_sum<SUB>(acc0 + acc1);
  else ss = group_sum(acc0 + acc1, red, wpr, tl);
  const float rs = 1.0f / __builtin_sqrtf(ss / (float)N + a.eps);
  if (!valid) return;
  if (tl == 0 && a.rstd) a.rstd[row] = rs;

  void* yr = out_row<D, O>(a.y, row, a.ldy);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (!FULL && col >= N) continue;
    const Raw r = STAGE_LDS ? stage[it * TPR + tl] : raw[it];
    float xf[V], wf[V], yf[V];
    IO::unpack(r, xf);
    IO::unpack(wraw[it], wf);
    apply_gain<D, O, V>(xf, wf, rs, a.offset, a.scale, yf);
    store_out<D, O, true, V>(yr, col, FULL ? V : N - col, a.yvec != 0, yf);
  }
}

// Any N and any alignment: the elementwise pass reads x again (from cache) instead of keeping it.
// WIDE selects 16-byte vectors or single elements.
template <DT D, bool WIDE, Out O>
__global__ void __launch_bounds__(1024) fwd_stream_kernel(FwdArgs a) {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int nv = (N + V - 1) / V;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  float* red = reinterpret_cast<float*>(smem) + grp * wpr;

  const S* xr = static_cast<const S*>(a.x) + (valid ? row : 0) * a.ldx;
  const bool comp = a.comp != 0;
  RowAcc acc;
  if (valid) {
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      const auto r = (col + V <= N) ? IO::load(xr + col) : IO::load_part(xr + col, N - col);
      float f[V];
      IO::unpack(r, f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc.fma(e, f[e], f[e], comp);
    }
  }
  const float ss = group_sum(acc.total(), red, wpr, tl);
  const float rs = 1.0f / __builtin_sqrtf(ss / (float)N + a.eps);
  if (!valid) return;
  if (tl == 0 && a.rstd) a.rstd[row] = rs;

  const S* wr = static_cast<const S*>(a.w);
  void* yr = out_row<D, O>(a.y, row, a.ldy);
  for (int v = tl; v < nv; v += TPR) {
    const int col = v * V;
    const bool full = col + V <= N;
    // the row's last read of x: non-temporal
    const auto r = full ? IO::load_nt(xr + col) : IO::load_part(xr + col, N - col);
    const auto wv = full ? IO::load(wr + col) : IO::load_part(wr + col, N - col);
    float xf[V], wf[V], yf[V];
    IO::unpack(r, xf);
    IO::unpack(wv, wf);
    apply_gain<D, O, V>(xf, wf, rs, a.offset, a.scale, yf);
    store_out<D, O, WIDE, V>(yr, col, N - col, a.yvec != 0, yf);
  }
}

// Rows that are not 16-byte aligned (contiguous rows of an odd width, say). A row's first h < V
// elements, up to its first 16-byte boundary, and its last t < V elements go one per lane (lanes
// 0 .. h-1 and 0 .. t-1); the rest moves as whole 16-byte vectors, vector j after the boundary to
// thread j % TPR. h comes from each row's own address, so the thread that holds a column changes
// from row to row. Each thread adds its head element, its vectors in order (even / odd
// accumulators) and its tail element, then the wave and row reductions; compensated sums on long
// chains as the streaming kernel. y takes vector stores when its rows sit at x's offsets from a
// 16-byte boundary (yvec), else element stores. w's columns for a vector are, in most rows, not
// 16-byte aligned: two aligned vectors and a funnel shift by h elements (peel_w).
template <DT D, Out O>
__global__ void __launch_bounds__(1024) fwd_peel_kernel(FwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  float* red = reinterpret_cast<float*>(smem) + grp * wpr;

  const S* xr = static_cast<const S*>(a.x) + (valid ? row : 0) * a.ldx;
  const S* wr = static_cast<const S*>(a.w);
  const bool walign = ((uintptr_t)wr & 15u) == 0;
  const int h = peel_head(xr, N);
  const int nb = (N - h) / V;
  const int t0 = h + nb * V;  // first element of the tail
  const bool comp = a.comp != 0;
  RowAcc acc;
  if (valid) {
    if (tl < h) {
      const float f = to_f32<D>(xr[tl]);
      acc.fma(0, f, f, comp);
    }
    for (int j = tl; j < nb; j += TPR) {
      float f[V];
      IO::unpack(IO::load(at(xr, h + j * V)), f);
#pragma unroll
      for (int e = 0; e < V; ++e) acc.fma(e, f[e], f[e], comp);
    }
    if (tl < N - t0) {
      const float f = to_f32<D>(xr[t0 + tl]);
      acc.fma(0, f, f, comp);
    }
  }
  const float ss = group_sum(acc.total(), red, wpr, tl);
  const float rs = 1.0f / __builtin_sqrtf(ss / (float)N + a.eps);
  if (!valid) return;
  if (tl == 0 && a.rstd) a.rstd[row] = rs;

  void* yr = out_row<D, O>(a.y, row, a.ldy);
  auto one = [&](int col) {
    const float xf[1] = {to_f32<D>(xr[col])}, wf[1] = {to_f32<D>(wr[col])};
    float yf[1];
    apply_gain<D, O, 1>(xf, wf, rs, a.offset, a.scale, yf);
    store_out<D, O, false, 1>(yr, col, 1, false, yf);
  };
  if (tl < h) one(tl);
  for (int j = tl; j < nb; j += TPR) {
    const int col = h + j * V;
    float xf[V], wf[V], yf[V];
    // the row's last read of x: non-temporal
    IO::unpack(IO::load_nt(at(xr, col)), xf);
    peel_w<D, V>(wr, walign, N, h, col, wf);
    apply_gain<D, O, V>(xf, wf, rs, a.offset, a.scale, yf);
    store_out<D, O, true, V>(yr, col, V, a.yvec != 0, yf);
  }
  if (tl < N - t0) one(t0 + tl);
}

}  // namespace rmsn
