// GroupNorm forward and backward kernels for x of shape [B, C, S] (S the flattened spatial size),
// C split into G groups of Cg = C / G adjacent channels; a (batch, group) row is the Cg * S
// contiguous elements of its channels.
//
// Statistics and reductions in float32, mean and rstd cached in float32, inputs upcast on load
// (Liger-Kernel pull request 1608, "fix(group_norm): keep the backward statistics and reductions
// in fp32"); the backward is the derivative of the formula (the layer_norm rule of candle pull
// request 4059 with per-channel weights):
//   y    = T( ((x - mean) * rstd) * w_c + b_c )                 c the element's channel
//   dx   = T( rstd * ((w_c * dy - c1) - xhat * c2) ),  c1 = sum(w_c dy) / n,  c2 = sum(w_c dy xhat) / n
//   dW_c = sum over batch and space of dy * xhat,      dB_c = sum over batch and space of dy
//
// Work is split into chunks of at most CH elements of one (batch, channel) segment, one 256-thread
// block per chunk (one wavefront per chunk for segments of at most CH / 4 elements), so the affine
// weight and bias are one scalar per chunk and rows of any length spread over the whole GPU. Every
// cross-chunk combination runs in a fixed order:
//   forward   gn_stats_kernel writes each chunk's (mean, M2 = sum of squared deviations from the
//             chunk mean, taken in a second pass over registers); gn_fwd_kernel merges the row's
//             chunk statistics with Chan's pairwise update (lane-strided sequential merges, then a
//             fixed shuffle tree) — every block of a row derives the same bits — and normalizes its
//             chunk, reading x a second time.
//   backward  gn_bwd_sums_kernel writes each chunk's (sum dy, sum dy * xhat); gn_bwd_dx_kernel
//             merges c1 = sum_c w_c * (sum dy) and c2 = sum_c w_c * (sum dy * xhat) over the row and
//             writes dx; one block per channel also adds the same per-chunk sums over batch and
//             chunks into dW_c and dB_c. Since w_c is constant over a chunk, w_c * sum(dy) is the
//             row sum of w_c * dy up to float32 rounding order, and one pair of sums per chunk
//             serves both the row constants and the parameter gradients.
#pragma once

#include "rmsnorm_common.hpp"

namespace rmsn {

constexpr int kGnThreads = 256;  // threads per chunk block (4 wavefronts)

// Elements per chunk: four 16-byte vectors per thread (8192 16-bit elements; measured faster
// than two: fewer blocks, each merging its row's chunk statistics once, 37 -> 34 us forward).
template <DT D> constexpr int gn_chunk() { return kGnThreads * 4 * Elem<D>::VEC; }

struct GnArgs {
  const void* x;
  const void* dy;   // backward only
  const void* w;    // [C]
  const void* b;    // [C] or null (forward)
  void* out;        // y (forward) or dx (backward), [B, C, S]
  float* mean;      // [B * G]
  float* rstd;      // [B * G]
  float2* ws;       // [B * C * K] per-chunk pairs
  float* dw;        // [C]
  float* db;        // [C] or null
  int64_t B, C, S;
  int G, Cg, K;     // groups, channels per group, chunks per (batch, channel) segment
  float eps;
  int tpr = 0, rows = 0;  // row kernels: threads per (batch, group) row, rows per block
};

// (count, mean, M2) of a set of values; merge() is Chan et al.'s pairwise update (float32).
struct Moments {
  float n, m, m2;
};
__device__ __forceinline__ Moments merge(Moments a, Moments b) {
  if (b.n == 0.f) return a;
  if (a.n == 0.f) return b;
  const float n = a.n + b.n;
  const float d = b.m - a.m;
  const float fb = b.n / n;
  return {n, a.m + d * fb, (a.m2 + b.m2) + (d * d) * (a.n * fb)};
}
__device__ __forceinline__ Moments shfl_down(Moments v, int off) {
  return {__shfl_down(v.n, off, 64), __shfl_down(v.m, off, 64), __shfl_down(v.m2, off, 64)};
}

// Block-level sums over the 4 wavefronts in wave order (group_sum with one group of 256 threads).
__device__ __forceinline__ float block_sum(float v, float* red) {
  return group_sum(v, red, kGnThreads / 64, threadIdx.x);
}

// The chunk of block u: segment bc = u / K (= batch * C + channel), chunk k = u % K.
struct Chunk {
  int64_t bc, base;  // segment index; element offset of the chunk in x
  int64_t bidx, c;   // batch, channel
  int k, cnt;        // chunk index within the segment, valid elements
};
template <DT D>
__device__ __forceinline__ Chunk chunk_of(const GnArgs& a, int64_t u) {
  constexpr int CH = gn_chunk<D>();
  Chunk ch;
  ch.bc = u / a.K;
  ch.k = (int)(u - ch.bc * a.K);
  ch.bidx = ch.bc / a.C;
  ch.c = ch.bc - ch.bidx * a.C;
  ch.base = ch.bc * a.S + (int64_t)ch.k * CH;
  const int64_t left = a.S - (int64_t)ch.k * CH;
  ch.cnt = (int)(left < CH ? left : CH);
  return ch;
}

// Loads of one chunk: thread t holds vectors t and t + 256 (WIDE) or elements t + 256 i. LAST:
// the kernel's read is the last one of these bytes (the second pass), so whole vectors take
// non-temporal loads; the first pass reads normally and leaves the lines to the caches.
template <DT D, bool WIDE>
struct ChunkIO {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  static constexpr int V = IO::V;
  static constexpr int IT = gn_chunk<D>() / (kGnThreads * V);
  // t: the thread's index among the chunk's `stride` threads (the block's 256, or a wavefront's 64
  // for chunks of at most a quarter of CH).
  template <bool LAST = false>
  static __device__ __forceinline__ void load(const S* p, int cnt, Raw (&r)[IT], int t, int stride) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int col = (it * stride + t) * V;
      r[it] = IO::zero();
      if (col + V <= cnt) r[it] = LAST ? IO::load_nt(p + col) : IO::load(p + col);
      else if (col < cnt) r[it] = IO::load_part(p + col, cnt - col);
    }
  }
};

// The chunk a thread works on. WPC = false: one chunk a block (its 256 threads). WPC: four chunks a
// block, one a wavefront, for segments of at most CH / 4 elements (a whole block would leave at
// least three quarters of its threads idle; a wavefront's lanes hold the same 4 vectors each, and
// its sums need no barrier). Waves past the last chunk have nothing to do (`idle`).
template <bool WPC>
struct ChunkSlot {
  int64_t u;   // chunk index (into the per-chunk pairs)
  int t;       // thread index among the chunk's threads
  int stride;  // the chunk's threads
  bool idle;
  __device__ __forceinline__ explicit ChunkSlot(const GnArgs& a) {
    u = WPC ? (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6) : (int64_t)blockIdx.x;
    t = WPC ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    stride = WPC ? 64 : kGnThreads;
    idle = WPC && u >= a.B * a.C * a.K;
  }
};
// A chunk's sum: the block's (4 wavefronts in order, one barrier) or the wavefront's.
template <bool WPC>
__device__ __forceinline__ float chunk_sum(float v, float* red) {
  return WPC ? wave_sum(v) : block_sum(v, red);
}

// Forward pass 1: per-chunk (mean, M2).
template <DT D, bool WIDE, bool WPC = false>
__global__ void __launch_bounds__(kGnThreads) gn_stats_kernel(GnArgs a) {
  using CI = ChunkIO<D, WIDE>;
  using IO = typename CI::IO;
  constexpr int V = CI::V, IT = CI::IT;
  __shared__ float red[8];
  const ChunkSlot<WPC> sl(a);
  if (sl.idle) return;  // whole wavefronts, and no barrier follows with WPC
  const Chunk ch = chunk_of<D>(a, sl.u);
  typename CI::Raw r[IT];
  CI::load(static_cast<const typename CI::S*>(a.x) + ch.base, ch.cnt, r, sl.t, sl.stride);
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float f[V];
    IO::unpack(r[it], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      if (e & 1) s1 += f[e];
      else s0 += f[e];
    }
  }
  const float m = chunk_sum<WPC>(s0 + s1, red) / (float)ch.cnt;
  float q0 = 0.f, q1 = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int col = (it * sl.stride + sl.t) * V;
    float f[V];
    IO::unpack(r[it], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float d = col + e < ch.cnt ? f[e] - m : 0.f;
      if (e & 1) q1 = __builtin_fmaf(d, d, q1);
      else q0 = __builtin_fmaf(d, d, q0);
    }
  }
  const float m2 = chunk_sum<WPC>(q0 + q1, red + 4);
  if (sl.t == 0) a.ws[sl.u] = make_float2(m, m2);
}

// Chunk statistics of the row (batch, group) merged in a fixed order by wave 0; lane 0 returns it.
template <DT D>
__device__ __forceinline__ Moments row_moments(const GnArgs& a, int64_t bidx, int g) {
  constexpr int CH = gn_chunk<D>();
  const int lane = threadIdx.x & 63;
  const int nent = a.Cg * a.K;
  const int64_t first = (bidx * a.C + (int64_t)g * a.Cg) * a.K;  // the row's entries are adjacent
  Moments acc = {0.f, 0.f, 0.f};
  for (int e = lane; e < nent; e += 64) {
    const int k = e % a.K;
    const int64_t left = a.S - (int64_t)k * CH;
    const float2 v = a.ws[first + e];
    acc = merge(acc, {(float)(left < CH ? left : CH), v.x, v.y});
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const Moments o = shfl_down(acc, off);
    if (lane < off) acc = merge(acc, o);
  }
  return acc;
}

// Forward pass 2: merge the row's statistics, write the caches (first chunk of the row), normalize.
// WPC: each wavefront merges its own chunk's row statistics.
template <DT D, bool WIDE, bool HAS_B, bool WPC = false>
__global__ void __launch_bounds__(kGnThreads) gn_fwd_kernel(GnArgs a) {
  using CI = ChunkIO<D, WIDE>;
  using IO = typename CI::IO;
  using S = typename CI::S;
  constexpr int V = CI::V, IT = CI::IT;
  __shared__ float stat[2];
  const ChunkSlot<WPC> sl(a);
  if (sl.idle) return;  // whole wavefronts, and no barrier follows with WPC
  const Chunk ch = chunk_of<D>(a, sl.u);
  const int g = (int)(ch.c / a.Cg);
  typename CI::Raw r[IT];
  // in flight during the merge
  CI::template load<true>(static_cast<const S*>(a.x) + ch.base, ch.cnt, r, sl.t, sl.stride);
  float mean, rs;
  if (WPC || threadIdx.x < 64) {
    const Moments mo = row_moments<D>(a, ch.bidx, g);  // lane 0 holds the row's moments
    const float m0 = __shfl(mo.m, 0, 64), m2 = __shfl(mo.m2, 0, 64), n0 = __shfl(mo.n, 0, 64);
    mean = m0;
    rs = 1.0f / __builtin_sqrtf(m2 / n0 + a.eps);
    if ((threadIdx.x & 63) == 0) {
      if (!WPC) {
        stat[0] = mean;
        stat[1] = rs;
      }
      if (ch.k == 0 && ch.c == (int64_t)g * a.Cg) {
        const int64_t row = ch.bidx * a.G + g;
        if (a.mean) a.mean[row] = mean;
        if (a.rstd) a.rstd[row] = rs;
      }
    }
  }
  if constexpr (!WPC) {
    __syncthreads();
    mean = stat[0];
    rs = stat[1];
  }
  const float wc = to_f32<D>(static_cast<const S*>(a.w)[ch.c]);
  const float bc = HAS_B ? to_f32<D>(static_cast<const S*>(a.b)[ch.c]) : 0.f;
  S* yp = static_cast<S*>(a.out) + ch.base;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int col = (it * sl.stride + sl.t) * V;
    if (col >= ch.cnt) continue;
    float f[V], o[V];
    IO::unpack(r[it], f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float xh = (f[e] - mean) * rs;
      o[e] = HAS_B ? xh * wc + bc : xh * wc;
    }
    const auto out = IO::pack(o);
    if (col + V <= ch.cnt) IO::store(yp + col, out);
    else IO::store_part(yp + col, out, ch.cnt - col);
  }
}

// Backward pass 1: per-chunk (sum dy, sum dy * xhat).
template <DT D, bool WIDE, bool WPC = false>
__global__ void __launch_bounds__(kGnThreads) gn_bwd_sums_kernel(GnArgs a) {
  using CI = ChunkIO<D, WIDE>;
  using IO = typename CI::IO;
  using S = typename CI::S;
  constexpr int V = CI::V, IT = CI::IT;
  __shared__ float red[8];
  const ChunkSlot<WPC> sl(a);
  if (sl.idle) return;  // whole wavefronts, and no barrier follows with WPC
  const Chunk ch = chunk_of<D>(a, sl.u);
  const int64_t row = ch.bidx * a.G + ch.c / a.Cg;
  const float mean = a.mean[row], rs = a.rstd[row];
  typename CI::Raw rx[IT], rd[IT];
  CI::load(static_cast<const S*>(a.x) + ch.base, ch.cnt, rx, sl.t, sl.stride);
  CI::load(static_cast<const S*>(a.dy) + ch.base, ch.cnt, rd, sl.t, sl.stride);
  float s0 = 0.f, s1 = 0.f, t0 = 0.f, t1 = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float xf[V], df[V];
    IO::unpack(rx[it], xf);
    IO::unpack(rd[it], df);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float xh = (xf[e] - mean) * rs;  // padding: dy = 0 adds nothing
      if (e & 1) {
        s1 += df[e];
        t1 = __builtin_fmaf(df[e], xh, t1);
      } else {
        s0 += df[e];
        t0 = __builtin_fmaf(df[e], xh, t0);
      }
    }
  }
  const float sdy = chunk_sum<WPC>(s0 + s1, red);
  const float sdx = chunk_sum<WPC>(t0 + t1, red + 4);
  if (sl.t == 0) a.ws[sl.u] = make_float2(sdy, sdx);
}

// dW_c = sum over (batch, chunk) of sum(dy * xhat), dB_c of sum(dy), by one wavefront: lane-strided
// sequential sums then a fixed shuffle tree.
__device__ __forceinline__ void gn_param_sums(const GnArgs& a, int64_t c) {
  const int lane = threadIdx.x & 63;
  const int64_t nent = a.B * a.K;
  float u1 = 0.f, u2 = 0.f;
  for (int64_t e = lane; e < nent; e += 64) {
    const int64_t bidx = e / a.K, k = e - bidx * a.K;
    const float2 v = a.ws[(bidx * a.C + c) * a.K + k];
    u1 += v.x;
    u2 += v.y;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o1 = __shfl_down(u1, off, 64), o2 = __shfl_down(u2, off, 64);
    if (lane < off) {
      u1 += o1;
      u2 += o2;
    }
  }
  if (lane == 0) {
    a.dw[c] = u2;
    if (a.db) a.db[c] = u1;
  }
}

// Backward pass 2: row constants from the chunk sums (fixed order), then dx for the chunk.
template <DT D, bool WIDE, bool WPC = false>
__global__ void __launch_bounds__(kGnThreads) gn_bwd_dx_kernel(GnArgs a) {
  using CI = ChunkIO<D, WIDE>;
  using IO = typename CI::IO;
  using S = typename CI::S;
  constexpr int V = CI::V, IT = CI::IT;
  __shared__ float cst[2];
  const ChunkSlot<WPC> sl(a);
  if (sl.idle) return;  // whole wavefronts, and no barrier follows with WPC
  const Chunk ch = chunk_of<D>(a, sl.u);
  const int g = (int)(ch.c / a.Cg);
  const int64_t row = ch.bidx * a.G + g;
  const float mean = a.mean[row], rs = a.rstd[row];
  const S* wp = static_cast<const S*>(a.w);
  typename CI::Raw rx[IT], rd[IT];
  CI::template load<true>(static_cast<const S*>(a.x) + ch.base, ch.cnt, rx, sl.t, sl.stride);
  CI::template load<true>(static_cast<const S*>(a.dy) + ch.base, ch.cnt, rd, sl.t, sl.stride);
  // The row constants from the chunk sums, by the block's first wavefront (WPC: every wavefront
  // for its own chunk's row).
  float c1 = 0.f, c2 = 0.f;
  if (WPC || threadIdx.x < 64) {
    const int lane = threadIdx.x & 63;
    const int nent = a.Cg * a.K;
    const int64_t first = (ch.bidx * a.C + (int64_t)g * a.Cg) * a.K;
    float u1 = 0.f, u2 = 0.f;
    for (int e = lane; e < nent; e += 64) {
      const float wc = to_f32<D>(wp[(int64_t)g * a.Cg + e / a.K]);
      const float2 v = a.ws[first + e];
      u1 += wc * v.x;
      u2 += wc * v.y;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o1 = __shfl_down(u1, off, 64), o2 = __shfl_down(u2, off, 64);
      if (lane < off) {
        u1 += o1;
        u2 += o2;
      }
    }
    const float n = (float)(a.Cg * a.S);
    c1 = __shfl(u1, 0, 64) / n;
    c2 = __shfl(u2, 0, 64) / n;
    if (!WPC && lane == 0) {
      cst[0] = c1;
      cst[1] = c2;
    }
  }
  // The first chunk of batch 0 of each channel also sums that channel's dW and dB (the per-chunk
  // sums are complete since the previous kernel): in the block's second wavefront, or with WPC in
  // the chunk's own wavefront.
  if (ch.bidx == 0 && ch.k == 0) {
    if (WPC) gn_param_sums(a, ch.c);
    else if (threadIdx.x >= 64 && threadIdx.x < 128) gn_param_sums(a, ch.c);
  }
  if constexpr (!WPC) {
    __syncthreads();
    c1 = cst[0];
    c2 = cst[1];
  }
  const float wc = to_f32<D>(wp[ch.c]);
  S* dxp = static_cast<S*>(a.out) + ch.base;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int col = (it * sl.stride + sl.t) * V;
    if (col >= ch.cnt) continue;
    float xf[V], df[V], o[V];
    IO::unpack(rx[it], xf);
    IO::unpack(rd[it], df);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float xh = (xf[e] - mean) * rs;
      o[e] = rs * ((wc * df[e] - c1) - xh * c2);
    }
    const auto out = IO::pack(o);
    if (col + V <= ch.cnt) IO::store(dxp + col, out);
    else IO::store_part(dxp + col, out, ch.cnt - col);
  }
}

// ---- (batch, group) rows that fit one row group's registers ------------------------------------
// Many channels of a small spatial size (7 x 7 to 32 x 32, say) make rows of a few thousand
// elements and (batch, channel) segments of a few dozen: one block per segment chunk would leave
// each block almost no work. Rows of n = Cg * S elements up to ITERS values per lane (16-byte
// vectors when n * sizeof(T) is a multiple of 16 and the tensors are 16-byte aligned, else single
// elements) are instead held whole by TPR threads, a.rows rows per block (row r = b * G + g starts
// at element r * n; element j of it belongs to channel g * Cg + j / S).
//   forward   mean = sum(x) / n, var = sum((x - mean)^2) / n over the registers (plain float32
//             sums: even and odd values of a lane, the lanes, then the waves in order), y from the
//             same registers: x read once.
//   backward  p1 = dy and p2 = fl(dy * xhat) go to LDS; each (batch, channel) segment is summed by
//             one wavefront (lane l the segment's elements l, l + 64, ... in order, then the wave
//             sum) into the same per-chunk pairs as the chunked kernels (one chunk per segment);
//             c1 = sum_c w_c * (sum dy) / n and c2 likewise over the row's Cg entries in the
//             chunked kernel's order (lane-strided, then the shuffle tree); dx from the registers.
//             dW and dB then come from the pairs as before (gn_params_kernel).
// w_c (and b_c) of the elements col .. col + V - 1 of a (batch, group) row (channel = element / Sl
// within the row): with Sl >= V a vector crosses at most one channel boundary, so one division
// and two loads per parameter serve the vector (elements from nb on take the next channel's);
// smaller spatial sizes divide per element. Elements past n take some channel's value, unused.
template <DT D, int V, bool HAS_B>
__device__ __forceinline__ void row_params(const typename Elem<D>::S* wp,
                                           const typename Elem<D>::S* bp, int col, int n, int Sl,
                                           int Cg, float (&wv)[V], float (&bv)[V]) {
  if (Sl >= V) {
    const int c0 = col / Sl, nb = (c0 + 1) * Sl - col;
    const int c1 = c0 + 1 < Cg ? c0 + 1 : c0;
    const float w0 = to_f32<D>(wp[c0]), w1 = to_f32<D>(wp[c1]);
    float b0 = 0.f, b1 = 0.f;
    if constexpr (HAS_B) {
      b0 = to_f32<D>(bp[c0]);
      b1 = to_f32<D>(bp[c1]);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      wv[e] = e < nb ? w0 : w1;
      bv[e] = e < nb ? b0 : b1;
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int c = (col + e < n ? col + e : col) / Sl;
      wv[e] = to_f32<D>(wp[c]);
      bv[e] = HAS_B ? to_f32<D>(bp[c]) : 0.f;
    }
  }
}

template <DT D, bool WIDE, int ITERS>
struct GnRowIO {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  static constexpr int V = IO::V;
  // The lane's values of row r (zeros past n).
  static __device__ __forceinline__ void load(const S* p, int n, int TPR, int tl, Raw (&r)[ITERS]) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      r[it] = IO::zero();
      if (col + V <= n) r[it] = IO::load(p + col);
      else if (col < n) r[it] = IO::load_part(p + col, n - col);
    }
  }
};

template <DT D, bool WIDE, int ITERS, bool HAS_B>
__global__ void __launch_bounds__(1024) gn_rows_fwd_kernel(GnArgs a) {
  using RI = GnRowIO<D, WIDE, ITERS>;
  using IO = typename RI::IO;
  using S = typename RI::S;
  constexpr int V = RI::V;
  extern __shared__ uint4 smem[];
  const int TPR = a.tpr, wpr = TPR >> 6;
  const int tid = threadIdx.x;
  const int grp = wave_group(tid, TPR);
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.rows + grp;
  const bool valid = row < a.B * a.G;
  const int n = a.Cg * (int)a.S;
  float* red = reinterpret_cast<float*>(smem) + grp * 2 * wpr;
  const S* xr = static_cast<const S*>(a.x) + (valid ? row : 0) * n;
  typename RI::Raw r[ITERS];
  RI::load(xr, n, TPR, tl, r);
  float f[ITERS][V];
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    IO::unpack(r[it], f[it]);
#pragma unroll
    for (int e = 0; e < V; ++e) {  // values past n are zeros
      if (e & 1) s1 += f[it][e];
      else s0 += f[it][e];
    }
  }
  const float mean = group_sum(s0 + s1, red, wpr, tl) / (float)n;
  float q0 = 0.f, q1 = 0.f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float d = col + e < n ? f[it][e] - mean : 0.f;
      if (e & 1) q1 = __builtin_fmaf(d, d, q1);
      else q0 = __builtin_fmaf(d, d, q0);
    }
  }
  const float var = group_sum(q0 + q1, red + wpr, wpr, tl) / (float)n;
  const float rs = 1.0f / __builtin_sqrtf(var + a.eps);
  if (!valid) return;
  if (tl == 0) {
    if (a.mean) a.mean[row] = mean;
    if (a.rstd) a.rstd[row] = rs;
  }
  const int g = (int)(row % a.G);
  const S* wp = static_cast<const S*>(a.w) + (int64_t)g * a.Cg;
  const S* bp = HAS_B ? static_cast<const S*>(a.b) + (int64_t)g * a.Cg : nullptr;
  const int Sl = (int)a.S;
  S* yr = static_cast<S*>(a.out) + row * n;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (col >= n) continue;
    float o[V], wv[V], bv[V];
    row_params<D, V, HAS_B>(wp, bp, col, n, Sl, a.Cg, wv, bv);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float xh = (f[it][e] - mean) * rs;
      o[e] = HAS_B ? xh * wv[e] + bv[e] : xh * wv[e];
    }
    const auto out = IO::pack(o);
    if (col + V <= n) IO::store(yr + col, out);
    else IO::store_part(yr + col, out, n - col);
  }
}

// LDS of the backward row kernel, per row group: two reduction slots and the row constants
// (4 * wpr + 2 floats, rounded to 4), the segment pairs (2 * Cg), then p1 and p2 (m each: n
// elements, or n / V vector sums with VSEG).
__host__ __device__ inline int gn_rows_bwd_lds_floats(int wpr, int Cg, int m) {
  return ((4 * wpr + 2 + 3) & ~3) + ((2 * Cg + 3) & ~3) + 2 * ((m + 3) & ~3);
}

// VSEG (16-byte vectors, S a multiple of V, so no vector straddles two channels): each lane first
// adds the V values of each of its vectors in element order, and p1, p2 hold these vector sums
// (n / V each): a segment's wavefront then adds S / V of them (lane l the vector sums l, l + 64,
// ... in order, then the wave sum) instead of S single values, and the row's LDS shrinks V-fold,
// which lets rows of up to 4 vectors a lane (bf16 32768 elements) keep their pairs in LDS.
template <DT D, bool WIDE, int ITERS, bool VSEG = false>
__global__ void __launch_bounds__(1024) gn_rows_bwd_kernel(GnArgs a) {
  static_assert(!VSEG || WIDE, "vector sums need 16-byte vectors");
  using RI = GnRowIO<D, WIDE, ITERS>;
  using IO = typename RI::IO;
  using S = typename RI::S;
  constexpr int V = RI::V;
  extern __shared__ uint4 smem[];
  const int TPR = a.tpr, wpr = TPR >> 6;
  const int tid = threadIdx.x;
  const int grp = wave_group(tid, TPR);
  const int tl = tid - grp * TPR;
  const int lane = tl & 63, wave = tl >> 6;
  const int64_t row = (int64_t)blockIdx.x * a.rows + grp;
  const bool valid = row < a.B * a.G;
  const int Cg = a.Cg, Sl = (int)a.S, n = Cg * Sl;
  const int m = VSEG ? n / V : n;  // staged values per row
  float* base = reinterpret_cast<float*>(smem) + (size_t)grp * gn_rows_bwd_lds_floats(wpr, Cg, m);
  float* cst = base + 4 * wpr;                 // c1, c2
  float* seg = base + ((4 * wpr + 2 + 3) & ~3);  // [Cg][2]
  float* p1 = seg + ((2 * Cg + 3) & ~3);       // [m]
  float* p2 = p1 + ((m + 3) & ~3);             // [m]
  const int64_t r = valid ? row : 0;
  const float mean = a.mean[r], rs = a.rstd[r];
  typename RI::Raw rx[ITERS], rd[ITERS];
  RI::load(static_cast<const S*>(a.x) + r * n, n, TPR, tl, rx);
  RI::load(static_cast<const S*>(a.dy) + r * n, n, TPR, tl, rd);
  float xh[ITERS][V], df[ITERS][V];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    float xf[V];
    IO::unpack(rx[it], xf);
    IO::unpack(rd[it], df[it]);
    float q[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      xh[it][e] = (xf[e] - mean) * rs;
      q[e] = df[it][e] * xh[it][e];
    }
    if constexpr (VSEG) {  // n is a multiple of V: a lane's vector is whole or absent
      if (col < n) {
        float u1 = df[it][0], u2 = q[0];
#pragma unroll
        for (int e = 1; e < V; ++e) {
          u1 += df[it][e];
          u2 += q[e];
        }
        p1[col / V] = u1;
        p2[col / V] = u2;
      }
      continue;
    }
    bool staged = false;
    if constexpr (WIDE) {  // whole vectors: 16-byte LDS stores (p1, p2, col multiples of 4 floats)
      if (col + V <= n) {
#pragma unroll
        for (int e = 0; e < V; e += 4) {
          *reinterpret_cast<float4*>(p1 + col + e) =
              make_float4(df[it][e], df[it][e + 1], df[it][e + 2], df[it][e + 3]);
          *reinterpret_cast<float4*>(p2 + col + e) =
              make_float4(q[e], q[e + 1], q[e + 2], q[e + 3]);
        }
        staged = true;
      }
    }
    if (!staged) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (col + e < n) {
          p1[col + e] = df[it][e];
          p2[col + e] = q[e];
        }
      }
    }
  }
  lds_barrier();
  // one wavefront per (batch, channel) segment of the row
  const int ms = VSEG ? Sl / V : Sl;  // staged values per segment
  for (int k = wave; k < Cg; k += wpr) {
    float u1 = 0.f, u2 = 0.f;
    for (int j = lane; j < ms; j += 64) {
      u1 += p1[k * ms + j];
      u2 += p2[k * ms + j];
    }
    u1 = wave_sum(u1);
    u2 = wave_sum(u2);
    if (lane == 0) {
      seg[2 * k] = u1;
      seg[2 * k + 1] = u2;
      if (valid) a.ws[r * Cg + k] = make_float2(u1, u2);
    }
  }
  lds_barrier();
  const int g = (int)(r % a.G);
  const S* wp = static_cast<const S*>(a.w) + (int64_t)g * Cg;
  if (wave == 0) {
    float u1 = 0.f, u2 = 0.f;
    for (int e = lane; e < Cg; e += 64) {
      const float wc = to_f32<D>(wp[e]);
      u1 += wc * seg[2 * e];
      u2 += wc * seg[2 * e + 1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o1 = __shfl_down(u1, off, 64), o2 = __shfl_down(u2, off, 64);
      if (lane < off) {
        u1 += o1;
        u2 += o2;
      }
    }
    if (lane == 0) {
      cst[0] = u1 / (float)n;
      cst[1] = u2 / (float)n;
    }
  }
  lds_barrier();
  if (!valid) return;
  const float c1 = cst[0], c2 = cst[1];
  S* dxr = static_cast<S*>(a.out) + row * n;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (col >= n) continue;
    float o[V], wv[V], bv[V];
    row_params<D, V, false>(wp, nullptr, col, n, Sl, Cg, wv, bv);
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = rs * ((wv[e] * df[it][e] - c1) - xh[it][e] * c2);
    const auto out = IO::pack(o);
    if (col + V <= n) IO::store(dxr + col, out);
    else IO::store_part(dxr + col, out, n - col);
  }
}

// dW and dB from the per-chunk pairs: one wavefront per channel.
__global__ void __launch_bounds__(256) gn_params_kernel(GnArgs a) {
  const int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c < a.C) gn_param_sums(a, c);
}

}  // namespace rmsn
