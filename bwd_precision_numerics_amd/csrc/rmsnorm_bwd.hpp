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
// With AG (autograd casts; 16-bit T, round twice): g*dy is rounded to T before it enters the row
// reduction and dx, and dw sums dy * T(xhat): the casts of differentiating the round-twice forward
// computed in T (the Liger RMSNorm pull request, "feat: correct casts in RMSNorm to match
// references", reproduces the references' casts in its backward).
//
// dw without atomics: block b of a persistent grid of P blocks owns rows b, b + P, b + 2P, ... (P
// depends only on M, so the result does not depend on the device). Interleaving keeps the whole
// grid on one contiguous stretch of rows at a time, which spreads DRAM traffic evenly; a block
// owning one contiguous chunk instead makes 256 far-apart streams and leaves some compute units
// starved. A block's threads keep float32 column accumulators in registers while they walk their
// rows, combine them across the block's row groups in a fixed tree order, and write one partial
// row of a [P, ldp] float32 workspace. A second kernel adds the P partial rows in a fixed order.
#pragma once

#include "rmsnorm_common.hpp"

namespace rmsn {

// Partial rows of the dw workspace: one per block; a function of M only.
constexpr int kMaxPartials = 256;
inline int64_t num_partials(int64_t M) { return M < kMaxPartials ? M : kMaxPartials; }
// Rows owned by block b of P: b, b + P, ... below M.
__device__ __forceinline__ int64_t block_rows(int64_t M, int P, int b) { return (M - b + P - 1) / P; }
// Row stride of the workspace in floats (16-byte aligned rows).
inline int64_t partial_ld(int64_t N) { return (N + 3) & ~int64_t(3); }
// Column sums in LDS indexed by a lane's 16-byte vector at an element offset h (rows not 16-byte
// aligned): one pad float after every 8, so the lanes' stride of 8 floats becomes 9 and a 32-bit
// LDS access of 64 lanes meets every bank at most once per pass instead of 8 or 16 lanes on one.
__host__ __device__ __forceinline__ int peel_col(int c) { return c + (c >> 3); }
// Floats of such a sums array for ldp columns.
__host__ __device__ inline int64_t peel_sum_floats(int64_t ldp) { return ldp + (ldp >> 3) + 1; }

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
  int comp;    // streaming kernel: compensated row sums (long per-thread chains)
  float offset;
  int dxvec = 0;  // unaligned-row kernel: dx rows sit at x's offsets from a 16-byte boundary
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

// Column sums of the 1024 / tpr row groups of a block (lane tl of a group holds the V columns
// tl V .. tl V + V - 1, so C = tpr * V columns) through LDS in at most two rounds instead of the
// pairwise tree, whose 2 log2(groups) barriers cost 0.55-0.9 us of a rows kernel with 4 to 64
// groups. Every group writes its sums as row grp of a [groups][C] array. With C >= 1024 columns
// thread t adds all groups' rows of columns t, t + 1024, ... in group order; with fewer, thread t
// adds rows q V .. q V + V - 1 of column t % C in order (q = t / C), and thread c < C adds the
// 1024 / C results of column c in order. Column c < N of the result goes to out[c] (non-temporal).
// LDS: combine_columns_floats(V) floats. Every thread of the 1024-thread block must call it.
constexpr int combine_columns_floats(int V) { return 1024 * V + 1024; }
template <int V>
__device__ __forceinline__ void combine_columns(const float (&acc)[V], float* buf, int grp, int tl,
                                                int tpr, float* out, int N) {
  const int C = tpr * V, G = 1024 / tpr, t = threadIdx.x;
  float* rows = buf;               // [G][C] = 1024 * V floats
  float* parts = buf + 1024 * V;   // [1024 / C][C] when C < 1024
  lds_barrier();  // earlier users of the LDS are done
  float* row = rows + grp * C + tl * V;
#pragma unroll
  for (int k = 0; k < V; k += 4)
    *reinterpret_cast<float4*>(row + k) = make_float4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
  lds_barrier();
  if (C >= 1024) {  // block-uniform
    for (int c = t; c < C; c += 1024) {
      float s = rows[c];
      for (int g = 1; g < G; ++g) s += rows[g * C + c];
      if (c < N) __builtin_nontemporal_store(s, out + c);
    }
    return;
  }
  const int c = t % C, q = t / C;
  float s = rows[(q * V) * C + c];
#pragma unroll
  for (int i = 1; i < V; ++i) s += rows[(q * V + i) * C + c];
  parts[q * C + c] = s;
  lds_barrier();
  if (t < C) {
    float total = parts[t];
    for (int j = 1; j < 1024 / C; ++j) total += parts[j * C + t];
    if (t < N) __builtin_nontemporal_store(total, out + t);
  }
}

// Write a block's combined column accumulators as partial row b of the workspace (group 0 only).
// Non-temporal (streaming cache policy) 16-byte stores: every block writes its row in the kernel's
// last moments, with no input stream left to overlap, and the reduction launch that follows reads
// them back sooner than rows written with the default policy (bf16 4096 x 4096, rows kernel then
// reduction: LayerNorm's two partial rows 25.85 -> 25.24 us, RMSNorm's one 22.52 -> 22.38 us).
template <int ITERS, int V>
__device__ __forceinline__ void store_partial(const float (&acc)[ITERS * V], float* pr, int TPR,
                                              int tl, int N) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const BufRsrc r = buf_rsrc(pr);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (col + V <= N) {
#pragma unroll
      for (int q = 0; q < V; q += 4) {
        const float4 v = make_float4(acc[it * V + q], acc[it * V + q + 1], acc[it * V + q + 2],
                                     acc[it * V + q + 3]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r,
                                               (uint32_t)(col + q) * 4u, 0, kBufNonTemporal);
      }
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (col + e < N) pr[col + e] = acc[it * V + e];
    }
  }
}

// A block's G row groups' column sums (ITERS vectors of V a lane) into partial row `out`: the
// column combine for one vector a lane and four or more groups, else the pairwise tree and group
// 0's stores. G is block-uniform. Every thread of the block must call it.
template <int ITERS, int V>
__device__ __forceinline__ void combine_block(float (&acc)[ITERS * V], float* buf, int G, int grp,
                                              int tl, int tpr, float* out, int N) {
  if constexpr (ITERS == 1) {
    if (G >= 4) {
      combine_columns<V>(acc, buf, grp, tl, tpr, out, N);
      return;
    }
  }
  combine_groups<ITERS * V>(acc, buf, G, grp, tl, tpr);
  if (grp == 0) store_partial<ITERS, V>(acc, out, tpr, tl, N);
}

// Sums of RB values over the TPR threads of one row group, with the order of group_sum for each:
// one LDS round trip and one barrier serve the whole batch. Every thread of the block must call it.
// W > 0: the row group's wave count is known at compile time (wpr == W).
template <int RB, int W = 0>
__device__ __forceinline__ void group_sum_batch(float (&v)[RB], float* red, int wpr, int tl) {
#pragma unroll
  for (int k = 0; k < RB; ++k) v[k] = wave_sum(v[k]);
  if (W > 1 || (W == 0 && wpr > 1)) {
    if ((tl & 63) == 0) {
#pragma unroll
      for (int k = 0; k < RB; ++k) red[(tl >> 6) * RB + k] = v[k];
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < RB; ++k)
      v[k] = W > 1 ? ordered_sum<(W > 1 ? W : 2), RB>(red + k) : waves_sum<RB>(red + k, wpr);
  }
}

// g * dy and the value dw multiplies dy by, under the two backward readings.
template <DT D, bool AG>
__device__ __forceinline__ float gain_dy(float g, float dy) {
  return AG ? round_trip<D>(g * dy) : g * dy;
}
template <DT D, bool AG>
__device__ __forceinline__ float dw_factor(float xh) {
  return AG ? round_trip<D>(xh) : xh;
}

// How a row's 16-byte vectors fall on a row group's lanes.
enum class Tail : int {
  FULL = 0,    // N = ITERS * TPR * V: every lane has ITERS whole vectors
  WHOLE = 1,   // N % V == 0: whole vectors, the last lanes may have none (idle)
  RAGGED = 2,  // N % V != 0 (a padded row stride): one lane's last vector is partial
};

// Register kernel. A row group takes its block's rows in batches of RB rows (local index
// (s * RB + k) * groups + grp for step s and batch index k; row = b + local * P) and keeps a ring of
// DEPTH + 1 batches of raw (x, dy) and their rstd in registers: while batch s is reduced and
// written, batches s + 1 .. s + DEPTH are in flight, and one barrier serves all RB rows of a batch.
// Pass 1 upcasts a raw row to form its dot product and its dw contributions; pass 2 either reuses
// xhat and g*dy kept from pass 1 (KEEP) or upcasts the raw row again. The gain g = offset + w stays
// in registers.
//
// Loads are straight-line code: every step issues its batch's loads unconditionally; rows past the
// block's share (and the empty steps that pad the last round of the ring) read w instead, which is
// cache-resident, and lanes without a whole vector read the row's first one. Only the arithmetic and
// the stores are guarded. Were the loads guarded too, the compiler would have to assume that any
// later step might have skipped its loads, and it would wait for every outstanding load at each
// step, leaving one row in flight whatever the ring depth. x, dy and dx move through buffer
// instructions: the row's descriptor sits in scalar registers and each lane keeps one 32-bit byte
// offset per vector, so no per-lane 64-bit addresses compete with the ring for registers (a
// 64-bit address built in a ring slot's registers also forces the same full wait).
//
// WPR > 0 fixes the row group at WPR wavefronts (TPR = 64 * WPR, 1024 / TPR groups per block) at
// compile time, so the row indices fold and the wave sums are read in one batch; WPR = 0 takes the
// shape from the arguments.
//
// SUB > 0: rows of at most SUB whole vectors (SUB = 4 to 32) take row groups of SUB lanes, 64 / SUB
// rows per wavefront and 1024 / SUB per block, summed with segment_sum (bit for bit the TPR = 64
// sums, so dx does not change); the groups' dw sums meet in combine_columns. A wavefront's rows are then local indices g0 .. g0 + 64 / SUB - 1,
// P rows apart: the buffer descriptor holds the wavefront's first row and each lane adds its own
// row's distance, dg * P row strides (the host checks that these offsets fit in 31 bits).
template <DT D, int ITERS, int DEPTH, int RB, bool AG, bool KEEP, Tail TAIL, int WPR, int SUB = 0>
__global__ void __launch_bounds__(1024) bwd_rows_kernel(BwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  constexpr int RING = DEPTH + 1;
  static_assert(SUB == 0 || (ITERS == 1 && TAIL != Tail::RAGGED),
                "narrow rows: at most one whole vector per lane");
  extern __shared__ uint4 smem[];

  const int TPR = SUB ? SUB : WPR ? 64 * WPR : a.tpr, wpr = SUB ? 1 : WPR ? WPR : TPR >> 6;
  const int G = SUB ? 1024 / SUB : WPR ? 1024 / (64 * WPR) : a.groups, N = a.N;
  const int tid = threadIdx.x;
  // Row group: wave-uniform (row indices and row pointers are scalar) unless SUB; g0 is the group
  // of the wavefront's first lane and dg = grp - g0 the lane's row within the wavefront.
  const int grp = SUB ? tid / TPR : wave_group(tid, TPR);
  const int g0 = SUB ? wave_group(tid & ~63, TPR) : grp;
  const int dg = grp - g0;
  const int tl = tid - grp * TPR;
  // Byte distance between a wavefront's consecutive rows in x, dy and dx.
  const uint32_t dx_step = SUB ? (uint32_t)((int64_t)a.P * a.ldx * (int64_t)sizeof(S)) : 0u;
  const uint32_t dd_step = SUB ? (uint32_t)((int64_t)a.P * a.lddy * (int64_t)sizeof(S)) : 0u;
  const uint32_t do_step = SUB ? (uint32_t)((int64_t)a.P * a.lddx * (int64_t)sizeof(S)) : 0u;
  const int b = blockIdx.x, P = a.P;
  const int64_t nloc = block_rows(a.M, P, b);
  const int64_t span = (int64_t)G * RB;
  const int nsteps = (int)((nloc + span - 1) / span);
  float* red = reinterpret_cast<float*>(smem);  // [2][G][wpr][RB]

  const S* wr = static_cast<const S*>(a.w);
  // Lane's vector `it`: byte offset in the row (0 for a lane without a whole vector, whose loads
  // are never used), whether it is whole, and whether the lane has any element of it.
  bool whole[ITERS], live[ITERS];
  uint32_t voff[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    // Only the last vector of a row can be absent or partial (ITERS = ceil(vectors / TPR)).
    const bool last = it == ITERS - 1;
    live[it] = TAIL == Tail::FULL || !last || col < N;
    // With N % V == 0 a lane's vector is whole or absent; said so, the element paths compile away.
    whole[it] = TAIL == Tail::RAGGED && last ? col + V <= N : live[it];
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
      float wf[V];
      IO::unpack(r, wf);
#pragma unroll
      for (int e = 0; e < V; ++e) g[it][e] = a.offset + wf[e];
    }
  }
  float acc[ITERS * V];
#pragma unroll
  for (int k = 0; k < ITERS * V; ++k) acc[k] = 0.f;

  Raw rx[RING][RB][ITERS], rd[RING][RB][ITERS];
  float rr[RING][RB];  // the rows' rstd travels with their data: no dependent load per step
  auto load_batch = [&](int slot, int s) {
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int64_t l0 = ((int64_t)s * RB + k) * G + g0, li = l0 + dg;
      const bool ok0 = s < nsteps && l0 < nloc, ok = s < nsteps && li < nloc;
      const int64_t row0 = b + (ok0 ? l0 : 0) * P;
      const S* xr = ok0 ? static_cast<const S*>(a.x) + row0 * a.ldx : wr;
      const S* dr = ok0 ? static_cast<const S*>(a.dy) + row0 * a.lddy : wr;
      const BufRsrc xb = buf_rsrc(xr), db = buf_rsrc(dr);
      // A lane whose own row lies past the block's share reads the wavefront's first row (or w).
      const uint32_t ex = SUB && ok ? (uint32_t)dg * dx_step : 0u;
      const uint32_t ed = SUB && ok ? (uint32_t)dg * dd_step : 0u;
      rr[slot][k] = a.rstd[SUB ? b + (ok ? li : 0) * P : row0];
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        rx[slot][k][it] = IO::load_b_nt(xb, voff[it] + ex, 0);
        rd[slot][k][it] = IO::load_b_nt(db, voff[it] + ed, 0);
        if constexpr (TAIL == Tail::RAGGED) {
          // The lane holding the row's partial vector reads it element by element (zeros past
          // N); these lane-dependent loads cost this instantiation some of its rows in flight.
          const int col = (it * TPR + tl) * V;
          if (!whole[it] && live[it]) {
            rx[slot][k][it] = IO::load_part(at(xr, col), N - col);
            rd[slot][k][it] = IO::load_part(at(dr, col), N - col);
          }
        }
      }
    }
  };
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) load_batch(j, j);

  // c = dot / N. Exactly tiled rows are a power of two wide (ITERS, TPR and V are), so 1/N is
  // exact and the product has the quotient's bits; other widths divide.
  const float inv_n = 1.0f / (float)N;

  for (int s0 = 0; s0 < nsteps; s0 += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      const int s = s0 + j;
      load_batch((j + DEPTH) % RING, s + DEPTH);
      if (s < nsteps) {  // block-uniform
        float rs[RB], dot[RB];
        float kx[KEEP ? RB : 1][KEEP ? ITERS * V : 1], kg[KEEP ? RB : 1][KEEP ? ITERS * V : 1];
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          const int64_t li = ((int64_t)s * RB + k) * G + grp;
          rs[k] = rr[j][k];
          float d0 = 0.f, d1 = 0.f;
          if (li < nloc) {  // wave-uniform unless SUB
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
              if (!live[it]) continue;
              float xf[V], df[V];
              IO::unpack(rx[j][k][it], xf);
              IO::unpack(rd[j][k][it], df);
#pragma unroll
              for (int e = 0; e < V; e += 2) {
                const float xh0 = xf[e] * rs[k], xh1 = xf[e + 1] * rs[k];
                const float gd0 = gain_dy<D, AG>(g[it][e], df[e]);
                const float gd1 = gain_dy<D, AG>(g[it][e + 1], df[e + 1]);
                acc[it * V + e] = __builtin_fmaf(df[e], dw_factor<D, AG>(xh0), acc[it * V + e]);
                acc[it * V + e + 1] =
                    __builtin_fmaf(df[e + 1], dw_factor<D, AG>(xh1), acc[it * V + e + 1]);
                if constexpr (KEEP) {
                  kx[k][it * V + e] = xh0;
                  kx[k][it * V + e + 1] = xh1;
                  kg[k][it * V + e] = gd0;
                  kg[k][it * V + e + 1] = gd1;
                }
                d0 = __builtin_fmaf(gd0, xh0, d0);
                d1 = __builtin_fmaf(gd1, xh1, d1);
              }
            }
          }
          dot[k] = d0 + d1;
        }
        if constexpr (SUB > 0) {
#pragma unroll
          for (int k = 0; k < RB; ++k) dot[k] = segment_sum<SUB>(dot[k]);
        } else {
          group_sum_batch<RB, WPR>(dot, red + ((s & 1) * G + grp) * wpr * RB, wpr, tl);
        }
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          const int64_t l0 = ((int64_t)s * RB + k) * G + g0, li = l0 + dg;
          if (li >= nloc) continue;
          const int64_t row0 = b + l0 * P;  // l0 <= li: the wavefront's first row is valid too
          const float c = TAIL == Tail::FULL ? dot[k] * inv_n : dot[k] / (float)N;
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
                o[e] = rs[k] * (kg[k][it * V + e] - kx[k][it * V + e] * c);
            } else {
              float xf[V], df[V];
              IO::unpack(rx[j][k][it], xf);
              IO::unpack(rd[j][k][it], df);
#pragma unroll
              for (int e = 0; e < V; ++e) {
                const float xh = xf[e] * rs[k];
                const float gd = gain_dy<D, AG>(g[it][e], df[e]);
                o[e] = rs[k] * (gd - xh * c);
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

  // Four or more row groups (rows of at most 256 lanes) meet in the column combine; one or two in
  // the pairwise tree (one level at two groups).
  combine_block<ITERS, V>(acc, reinterpret_cast<float*>(smem), G, grp, tl, TPR,
                          a.part + (int64_t)b * a.ldp, N);
}

// LDS-staged kernel for rows too wide to keep in registers (e.g. N = 32768 in 16-bit types): the
// raw x and dy of the current row sit in LDS for both passes while the registers hold the next
// row's loads in flight (a two-row pipeline), so registers carry the column accumulators and one
// row of raw data. The gain is re-read from w (cache-resident) in each pass. Same thread-to-element
// mapping and summation order as the register kernel, so dx is bit-identical to it for the same
// shape. TAIL as for the register kernel: whole vectors on every lane, whole vectors or none
// (idle lanes), or a partial last vector. The next row's loads are straight-line code (a block's
// last step reads w instead), so the compiler waits only for them, not for the stores in flight.
template <DT D, int ITERS, bool AG, Tail TAIL, int TPRC = 0>
__global__ void __launch_bounds__(1024) bwd_lds_kernel(BwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  // TPRC > 0: one row group of TPRC threads (the whole block), known at compile time, so the
  // stage slots of a thread sit at constant offsets from two base addresses.
  const int TPR = TPRC > 0 ? TPRC : a.tpr, G = TPRC > 0 ? 1 : a.groups;
  const int wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = wave_group(tid, TPR);
  const int tl = tid - grp * TPR;
  const int b = blockIdx.x, P = a.P;
  const int64_t nloc = block_rows(a.M, P, b);
  const int nsteps = (int)((nloc + G - 1) / G);
  float* red = reinterpret_cast<float*>(smem);                                    // [2][G * wpr]
  Raw* stage = smem + ((2 * G * wpr + 3) >> 2) + (size_t)grp * 2 * ITERS * TPR;  // [G][2][ITERS*TPR]

  const S* wr = static_cast<const S*>(a.w);
  const BufRsrc wbuf = buf_rsrc(wr);
  // Lane's vector it: byte offset in the row (vector it * TPR + tl; 0 for a lane without a whole
  // vector, whose loads are never used), whole / any elements, as in the register kernel.
  bool whole[ITERS], live[ITERS];
  uint32_t voff[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    // Only the last vector of a row can be absent or partial (ITERS = ceil(vectors / TPR)).
    const bool last = it == ITERS - 1;
    live[it] = TAIL == Tail::FULL || !last || col < N;
    whole[it] = TAIL == Tail::RAGGED && last ? col + V <= N : live[it];
    voff[it] = whole[it] ? (uint32_t)col * (uint32_t)sizeof(S) : 0u;
  }
  float acc[ITERS * V];
#pragma unroll
  for (int k = 0; k < ITERS * V; ++k) acc[k] = 0.f;

  // Registers carry the next row's raw x and dy (and rstd) while the current one is processed
  // from the stage.
  Raw rx[ITERS], rd[ITERS];
  float rs_next = 0.f;
  auto load_row = [&](int s) {
    const int64_t li = (int64_t)s * G + grp;
    const bool ok = s < nsteps && li < nloc;
    const int64_t row = b + (ok ? li : 0) * P;
    const S* xr = ok ? static_cast<const S*>(a.x) + row * a.ldx : wr;
    const S* dr = ok ? static_cast<const S*>(a.dy) + row * a.lddy : wr;
    const BufRsrc xb = buf_rsrc(xr), db = buf_rsrc(dr);
    rs_next = a.rstd[row];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      rx[it] = IO::load_b_nt(xb, voff[it], 0);
      rd[it] = IO::load_b_nt(db, voff[it], 0);
      if constexpr (TAIL == Tail::RAGGED) {
        const int col = (it * TPR + tl) * V;
        if (!whole[it] && live[it]) {
          rx[it] = IO::load_part(at(xr, col), N - col);
          rd[it] = IO::load_part(at(dr, col), N - col);
        }
      }
    }
  };
  load_row(0);

  // c = dot / N: a multiply for exactly tiled rows (a power of two wide), else a division.
  const float inv_n = 1.0f / (float)N;

  for (int s = 0; s < nsteps; ++s) {
    const int64_t li = (int64_t)s * G + grp;
    const bool valid = li < nloc;  // wave-uniform
    const int64_t row = b + (valid ? li : 0) * P;
    // Each thread reads back only the stage slots it wrote, so no barrier guards the stage.
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      stage[it * TPR + tl] = rx[it];
      stage[(ITERS + it) * TPR + tl] = rd[it];
    }
    const float rs = rs_next;
    load_row(s + 1);
    // Opaque copies of the lane's stage index and w offsets. Without them the compiler would
    // forward the values just stored to the stage instead of reading them back (keeping this
    // row's raw data live next to the next row's loads), and would hoist the w loads (the same for
    // every row) out of the row loop, holding the whole gain in registers.
    int tl1 = tl;
    uint32_t wv1[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) wv1[it] = voff[it];
    asm volatile("" : "+v"(tl1));
#pragma unroll
    for (int it = 0; it < ITERS; ++it) asm volatile("" : "+v"(wv1[it]));
    float d0 = 0.f, d1 = 0.f;
    if (valid) {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        if (!live[it]) continue;
        const int col = (it * TPR + tl) * V;
        Raw rw = IO::load_b(wbuf, wv1[it], 0);
        if (TAIL == Tail::RAGGED && !whole[it]) rw = IO::load_part(at(wr, col), N - col);
        float xf[V], df[V], wf[V];
        IO::unpack(stage[it * TPR + tl1], xf);
        IO::unpack(stage[(ITERS + it) * TPR + tl1], df);
        IO::unpack(rw, wf);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float xh = xf[e] * rs;
          const float gd = gain_dy<D, AG>(a.offset + wf[e], df[e]);
          acc[it * V + e] = __builtin_fmaf(df[e], dw_factor<D, AG>(xh), acc[it * V + e]);
          if (e & 1) d1 = __builtin_fmaf(gd, xh, d1);
          else d0 = __builtin_fmaf(gd, xh, d0);
        }
        // One vector at a time, with its dw updates done here: left to itself the compiler sinks
        // them past the reduction and keeps every vector's xhat and dy live until then, which the
        // accumulators and the next row's loads leave no registers for.
#pragma unroll
        for (int e = 0; e < V; ++e) asm volatile("" : "+v"(acc[it * V + e]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float dot = group_sum(d0 + d1, red + (s & 1) * G * wpr + grp * wpr, wpr, tl);
    const float c = TAIL == Tail::FULL ? dot * inv_n : dot / (float)N;
    // Fresh opaque copies for the second pass, which reads the same addresses as the first:
    // otherwise the first pass's values stay live across the reduction.
    int tl2 = tl;
    uint32_t wv2[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) wv2[it] = voff[it];
    asm volatile("" : "+v"(tl2));
#pragma unroll
    for (int it = 0; it < ITERS; ++it) asm volatile("" : "+v"(wv2[it]));
    if (valid) {
      S* dxr = static_cast<S*>(a.dx) + row * a.lddx;
      const BufRsrc dxb = buf_rsrc(dxr);
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        if (!live[it]) continue;
        const int col = (it * TPR + tl) * V;
        Raw rw = IO::load_b(wbuf, wv2[it], 0);
        if (TAIL == Tail::RAGGED && !whole[it]) rw = IO::load_part(at(wr, col), N - col);
        float xf[V], df[V], wf[V], o[V];
        IO::unpack(stage[it * TPR + tl2], xf);
        IO::unpack(stage[(ITERS + it) * TPR + tl2], df);
        IO::unpack(rw, wf);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float xh = xf[e] * rs;
          const float gd = gain_dy<D, AG>(a.offset + wf[e], df[e]);
          o[e] = rs * (gd - xh * c);
        }
        const Raw out = IO::pack(o);
        if (whole[it]) IO::store_b(dxb, voff[it], 0, out);
        else IO::store_part(at(dxr, col), out, N - col);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // The register kernel's combine for the same shape (so the two give the same dw bits).
  combine_block<ITERS, V>(acc, reinterpret_cast<float*>(smem), G, grp, tl, TPR,
                          a.part + (int64_t)b * a.ldp, N);
}

// Any N and any alignment. One row at a time per block (groups = 1); the elementwise pass reads
// x and dy again (from the caches). KREG = 0: the block's dw partial row accumulates in LDS when
// LACC (rows up to kStreamLdsAccFloats wide; each column is owned by one thread, rows are added in
// order) and is written once at the end, else in the workspace itself. KREG > 0 (16-byte vectors,
// at most KREG per thread: rows past the LDS-staged kernel's reach, up to 8192 vectors): the same
// sums in registers — per row the workspace round trip would move twice the row's float32 width
// (the kernel ran at 1.3 TB/s that way). Same operations in the same order every way, so dx and
// dw are bit-identical between them.
constexpr int kStreamLdsAccFloats = 36 * 1024;  // 144 KiB of LDS, after the 128-byte reduction area
template <DT D, bool WIDE, bool AG, int KREG = 0, bool LACC = false>
__global__ void __launch_bounds__(1024) bwd_stream_kernel(BwdArgs a) {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  static_assert(KREG == 0 || WIDE, "register sums take 16-byte vectors");
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int nv = (N + V - 1) / V;
  const int tl = threadIdx.x;
  const int b = blockIdx.x, P = a.P;
  float* red = reinterpret_cast<float*>(smem);  // [2][wpr]
  const S* wr = static_cast<const S*>(a.w);
  float* const pg = a.part + (int64_t)b * a.ldp;
  static_assert(!LACC || KREG == 0, "LDS sums replace the workspace sums");
  // The row's dw sums: LDS (after the 32-float reduction area) or the workspace row itself.
  float* const pr = LACC ? reinterpret_cast<float*>(smem) + 32 : pg;
  constexpr int K = KREG > 0 ? KREG * V : 1;
  float acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = 0.f;

  if constexpr (KREG == 0) {
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (col + e < N) pr[col + e] = 0.f;
    }
  }

  int s = 0;
  for (int64_t row = b; row < a.M; row += P, ++s) {
    const S* xr = static_cast<const S*>(a.x) + row * a.ldx;
    const S* dr = static_cast<const S*>(a.dy) + row * a.lddy;
    const float rs = a.rstd[row];
    RowAcc d;
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
        const float gd = gain_dy<D, AG>(a.offset + wf[e], df[e]);
        d.fma(e, gd, xh, a.comp != 0);
      }
    }
    const float dot = group_sum(d.total(), red + (s & 1) * wpr, wpr, tl);
    const float c = dot / (float)N;
    S* dxr = static_cast<S*>(a.dx) + row * a.lddx;
    auto elementwise = [&](int v, float* accv) {
      const int col = v * V;
      const bool full = col + V <= N;
      float xf[V], df[V], wf[V], o[V];
      // the row's last read of x and dy: non-temporal
      IO::unpack(full ? IO::load_nt(xr + col) : IO::load_part(xr + col, N - col), xf);
      IO::unpack(full ? IO::load_nt(dr + col) : IO::load_part(dr + col, N - col), df);
      IO::unpack(full ? IO::load(wr + col) : IO::load_part(wr + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = xf[e] * rs;
        const float gd = gain_dy<D, AG>(a.offset + wf[e], df[e]);
        o[e] = rs * (gd - xh * c);
        if constexpr (KREG > 0) {
          accv[e] = __builtin_fmaf(df[e], dw_factor<D, AG>(xh), accv[e]);
        } else {
          if (col + e < N) pr[col + e] = __builtin_fmaf(df[e], dw_factor<D, AG>(xh), pr[col + e]);
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
        if (v < nv) elementwise(v, acc + k * V);
        // One vector at a time, its dw sums done here (the compiler would otherwise keep every
        // vector's loads and operands live at once next to the accumulators).
#pragma unroll
        for (int e = 0; e < V; ++e) asm volatile("" : "+v"(acc[k * V + e]));
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int v = tl; v < nv; v += TPR) elementwise(v, nullptr);
    }
  }

  if constexpr (KREG > 0) {
#pragma unroll
    for (int k = 0; k < KREG; ++k) {
      const int col = (tl + k * TPR) * V;
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (col + e < N) pg[col + e] = acc[k * V + e];
    }
  } else if constexpr (LACC) {
    // each thread copies the columns it summed: no barrier needed
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (col + e < N) pg[col + e] = pr[col + e];
    }
  }
}

// Rows that are not 16-byte aligned whose x and dy rows sit at the same offset from a 16-byte
// boundary (equal base offsets, equal row strides modulo 16 bytes: contiguous rows of an odd width,
// say), as the forward's unaligned-row kernel: per row, h < V head and t < V tail elements one per
// lane, whole 16-byte vectors between them, vector j after the boundary to thread j % TPR, h from
// the row's address. One row per block at a time, two passes as the streaming kernel (the second
// re-reads x and dy non-temporally; w as in the forward, peel_w). The thread that holds a column changes
// from row to row, so the dw sums sit in LDS (N floats after the reduction area): each column gets
// one addition per row, rows in the block's order, ordered by the barrier of the next row's
// reduction; the block's partial row is written once at the end. dx takes vector stores when its
// rows sit at x's offsets (dxvec), else element stores.
template <DT D, bool AG>
__global__ void __launch_bounds__(1024) bwd_peel_kernel(BwdArgs a) {
  using IO = VecIO<D, true>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];

  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int tl = threadIdx.x;
  const int b = blockIdx.x, P = a.P;
  float* red = reinterpret_cast<float*>(smem);            // [2][wpr], at most 32 floats
  float* const sums = reinterpret_cast<float*>(smem) + 32;  // dw sums, columns at peel_col
  const S* wr = static_cast<const S*>(a.w);
  const bool walign = ((uintptr_t)wr & 15u) == 0;
  const bool comp = a.comp != 0;
  for (int c = tl; c < N; c += TPR) sums[peel_col(c)] = 0.f;

  int s = 0;
  for (int64_t row = b; row < a.M; row += P, ++s) {
    const S* xr = static_cast<const S*>(a.x) + row * a.ldx;
    const S* dr = static_cast<const S*>(a.dy) + row * a.lddy;
    S* dxr = static_cast<S*>(a.dx) + row * a.lddx;
    const float rs = a.rstd[row];
    const int h = peel_head(xr, N);
    const int nb = (N - h) / V;
    const int t0 = h + nb * V;
    RowAcc d;
    auto first = [&](int col) {
      const float xh = to_f32<D>(xr[col]) * rs;
      const float gd = gain_dy<D, AG>(a.offset + to_f32<D>(wr[col]), to_f32<D>(dr[col]));
      d.fma(0, gd, xh, comp);
    };
    if (tl < h) first(tl);
    for (int j = tl; j < nb; j += TPR) {
      const int col = h + j * V;
      float xf[V], df[V], wf[V];
      IO::unpack(IO::load(at(xr, col)), xf);
      IO::unpack(IO::load(at(dr, col)), df);
      peel_w<D, V>(wr, walign, N, h, col, wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = xf[e] * rs;
        const float gd = gain_dy<D, AG>(a.offset + wf[e], df[e]);
        d.fma(e, gd, xh, comp);
      }
    }
    if (tl < N - t0) first(t0 + tl);
    const float dot = group_sum(d.total(), red + (s & 1) * wpr, wpr, tl);
    const float c = dot / (float)N;
    auto second = [&](int col) {
      const float dyv = to_f32<D>(dr[col]);
      const float xh = to_f32<D>(xr[col]) * rs;
      const float gd = gain_dy<D, AG>(a.offset + to_f32<D>(wr[col]), dyv);
      dxr[col] = from_f32<D>(rs * (gd - xh * c));
      const int k = peel_col(col);
      sums[k] = __builtin_fmaf(dyv, dw_factor<D, AG>(xh), sums[k]);
    };
    if (tl < h) second(tl);
    for (int j = tl; j < nb; j += TPR) {
      const int col = h + j * V;
      float xf[V], df[V], wf[V], o[V];
      // the row's last read of x and dy: non-temporal
      IO::unpack(IO::load_nt(at(xr, col)), xf);
      IO::unpack(IO::load_nt(at(dr, col)), df);
      peel_w<D, V>(wr, walign, N, h, col, wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float xh = xf[e] * rs;
        const float gd = gain_dy<D, AG>(a.offset + wf[e], df[e]);
        o[e] = rs * (gd - xh * c);
        const int k = peel_col(col + e);
        sums[k] = __builtin_fmaf(df[e], dw_factor<D, AG>(xh), sums[k]);
      }
      const auto out = IO::pack(o);
      if (a.dxvec) IO::store(at(dxr, col), out);
      else IO::store_part(at(dxr, col), out, V);
    }
    if (tl < N - t0) second(t0 + tl);
  }
  lds_barrier();  // the last row's sums were added by other threads
  float* const pg = a.part + (int64_t)b * a.ldp;
  for (int c = tl; c < N; c += TPR) pg[c] = sums[peel_col(c)];
}

// Rows that are not 16-byte aligned, as bwd_peel_kernel, of at most one whole 16-byte vector per
// lane, on the register kernel's persistent grid and row order: G row groups of TPR threads, step s
// of block b giving its group row b + (s * G + grp) * P. A lane holds the row's whole vector tl
// (the vectors start h elements into the row, h from the row's address), lanes below h and below t
// the head and tail elements, in registers for both passes. One step ahead the next row's x, dy,
// rstd and gain are loaded, all unconditionally (a lane without a whole vector reads the row's first
// one, head and tail indices are clamped into the row; the two aligned gain vectors that the funnel
// shift by h takes come through a descriptor bounded at w's last 16-byte granule, so the one past
// w's end reads zeros), so the compiler waits only for the row in use. The thread that holds a
// column changes with h, so each row group keeps its dw sums in LDS (past the reduction slots,
// columns at peel_col): per row one fma per column from one lane, in the group's row order, which the
// barrier of the next row's reduction keeps. The block's partial row is the groups' sums added in
// group order. w must be 16-byte aligned.
template <DT D, bool AG>
__global__ void __launch_bounds__(1024) bwd_peel_rows_kernel(BwdArgs a) {
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
  float* red = reinterpret_cast<float*>(smem);                  // [2][G][wpr]
  const int stride = (int)peel_sum_floats(a.ldp);
  float* const sums0 = red + ((2 * G * wpr + 3) & ~3);  // [G][stride], columns at peel_col
  float* const sums = sums0 + (size_t)grp * stride;
  for (int c = tl; c < N; c += TPR) sums[peel_col(c)] = 0.f;

  const S* wr = static_cast<const S*>(a.w);
  const BufRsrc wb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<S*>(wr), 0, (N * (int)sizeof(S) + 15) & ~15, kBufDword3);

  Raw rx[2], rd[2], wa[2], wv[2];
  S hx[2], hd[2], hw[2], tx[2], td[2], tw[2];
  float rr[2];
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
      const float rs = rr[j];
      float xh[V], gd[V], df[V];
      float hxh = 0.f, hgd = 0.f, txh = 0.f, tgd = 0.f;
      float d0 = 0.f, d1 = 0.f;
      {
        float xf[V], wf[V];
        IO::unpack(rx[j], xf);
        IO::unpack(rd[j], df);
        IO::unpack(peel_vec<D>(h, wa[j], wv[j]), wf);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xh[e] = xf[e] * rs;
          gd[e] = gain_dy<D, AG>(a.offset + wf[e], df[e]);
        }
      }
      if (valid) {
        if (tl < h) {
          hxh = to_f32<D>(hx[j]) * rs;
          hgd = gain_dy<D, AG>(a.offset + to_f32<D>(hw[j]), to_f32<D>(hd[j]));
          d0 = __builtin_fmaf(hgd, hxh, d0);
        }
        if (tl < nb) {
#pragma unroll
          for (int e = 0; e < V; e += 2) {
            d0 = __builtin_fmaf(gd[e], xh[e], d0);
            d1 = __builtin_fmaf(gd[e + 1], xh[e + 1], d1);
          }
        }
        if (tl < t) {
          txh = to_f32<D>(tx[j]) * rs;
          tgd = gain_dy<D, AG>(a.offset + to_f32<D>(tw[j]), to_f32<D>(td[j]));
          d1 = __builtin_fmaf(tgd, txh, d1);
        }
      }
      float dot[1] = {d0 + d1};
      group_sum_batch<1>(dot, red + ((s & 1) * G + grp) * wpr, wpr, tl);
      if (wpr == 1) lds_barrier();  // orders the LDS sums of consecutive rows (no barrier above)
      if (!valid) continue;
      const float c = dot[0] / (float)N;
      S* dxr = static_cast<S*>(a.dx) + (b + li * P) * a.lddx;
      if (tl < h) {
        dxr[tl] = from_f32<D>(rs * (hgd - hxh * c));
        sums[peel_col(tl)] =
            __builtin_fmaf(to_f32<D>(hd[j]), dw_factor<D, AG>(hxh), sums[peel_col(tl)]);
      }
      if (tl < nb) {
        const int col = h + tl * V;
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          o[e] = rs * (gd[e] - xh[e] * c);
          const int k = peel_col(col + e);
          sums[k] = __builtin_fmaf(df[e], dw_factor<D, AG>(xh[e]), sums[k]);
        }
        const Raw out = IO::pack(o);
        if (a.dxvec) IO::store(at(dxr, col), out);
        else IO::store_part(at(dxr, col), out, V);
      }
      if (tl < t) {
        dxr[t0 + tl] = from_f32<D>(rs * (tgd - txh * c));
        const int k = peel_col(t0 + tl);
        sums[k] = __builtin_fmaf(to_f32<D>(td[j]), dw_factor<D, AG>(txh), sums[k]);
      }
    }
  }
  lds_barrier();  // every group's last sums are in LDS
  float* const pg = a.part + (int64_t)b * a.ldp;
  for (int c = tid; c < N; c += G * TPR) {
    float v = sums0[peel_col(c)];
    for (int g = 1; g < G; ++g) v += sums0[(size_t)g * stride + peel_col(c)];
    pg[c] = v;
  }
}

// dw_j = sum over p of part[p, j] in a fixed order, spread over many compute units: a block of
// 4 wavefronts owns 16 columns. Lane l of wave k reads column l % 16 of partial rows
// p = 16 * i + 4 * k + l / 16 (i = 0 .. kMaxPartials / 16 - 1, all loads in flight together) and
// adds them in order of i; the four lanes of a column (l / 16 = 0..3) are then added in order, and
// finally the four waves in order. blockIdx.y selects one of gridDim.y sets of partial rows,
// set_stride floats apart, and its output (dw, or dw2 for the second set).
// The float64 RMSNorm reduces its double partials with it; float32 partials take
// dw_reduce32_kernel or dw_reduce4_kernel below.
static_assert(kMaxPartials % 16 == 0, "dw_reduce_kernel reads partial rows in groups of 16");
template <typename T>
__global__ void __launch_bounds__(256) dw_reduce_kernel(const T* part, int64_t ldp, int P, int N,
                                                        T* dw, T* dw2, int64_t set_stride) {
  if (blockIdx.y) {
    part += set_stride;
    dw = dw2;
  }
  constexpr int L = kMaxPartials / 16;
  __shared__ T buf[4][16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int col = blockIdx.x * 16 + c;
  T v[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int p = 16 * i + 4 * wv + q;
    v[i] = (col < N && p < P) ? part[(int64_t)p * ldp + col] : T(0);
  }
  T s = v[0];
#pragma unroll
  for (int i = 1; i < L; ++i) s += v[i];
  // lanes c, c+16, c+32, c+48 hold the four row phases of column c: add them in order q = 0..3
  const T s1 = __shfl(s, c + 16, 64), s2 = __shfl(s, c + 32, 64), s3 = __shfl(s, c + 48, 64);
  const T t = ((s + s1) + s2) + s3;
  if (q == 0) buf[wv][c] = t;
  __syncthreads();
  if (wv == 0 && q == 0 && col < N) dw[col] = ((buf[0][c] + buf[1][c]) + buf[2][c]) + buf[3][c];
}

// The float32 version with 16-byte loads: the same partial rows per lane and the same order of
// additions per column, but each lane reads 4 consecutive columns (16 lanes cover 64 columns, 256
// contiguous bytes of a partial row, instead of 64), so a block owns 64 columns. Partial rows are
// padded to a multiple of 4 floats (partial_ld), so a vector that starts below N stays inside its
// row. It adds in the order dw_reduce_kernel would for float partials.
inline __global__ void __launch_bounds__(256) dw_reduce4_kernel(const float* part, int64_t ldp,
                                                                int P, int N, float* dw,
                                                                float* dw2, int64_t set_stride) {
  if (blockIdx.y) {
    part += set_stride;
    dw = dw2;
  }
  constexpr int L = kMaxPartials / 16;
  __shared__ float4 buf[4][16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int col = (blockIdx.x * 16 + c) * 4;
  float4 v[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int p = 16 * i + 4 * wv + q;
    v[i] = (col < N && p < P) ? *reinterpret_cast<const float4*>(part + (int64_t)p * ldp + col)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 t = v[0];
#pragma unroll
  for (int i = 1; i < L; ++i) {
    t.x += v[i].x;
    t.y += v[i].y;
    t.z += v[i].z;
    t.w += v[i].w;
  }
  // lanes c, c+16, c+32, c+48 hold the four row phases of columns col..col+3: add them in order
  float4 u[4];
  u[0] = t;
#pragma unroll
  for (int k = 1; k < 4; ++k)
    u[k] = make_float4(__shfl(t.x, c + 16 * k, 64), __shfl(t.y, c + 16 * k, 64),
                       __shfl(t.z, c + 16 * k, 64), __shfl(t.w, c + 16 * k, 64));
  if (q == 0)
    buf[wv][c] = make_float4(((u[0].x + u[1].x) + u[2].x) + u[3].x,
                             ((u[0].y + u[1].y) + u[2].y) + u[3].y,
                             ((u[0].z + u[1].z) + u[2].z) + u[3].z,
                             ((u[0].w + u[1].w) + u[2].w) + u[3].w);
  __syncthreads();
  if (wv == 0 && q == 0 && col < N) {
    const float4 a = buf[0][c], b = buf[1][c], d = buf[2][c], e = buf[3][c];
    const float r[4] = {((a.x + b.x) + d.x) + e.x, ((a.y + b.y) + d.y) + e.y,
                        ((a.z + b.z) + d.z) + e.z, ((a.w + b.w) + d.w) + e.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (col + k < N) dw[col + k] = r[k];
  }
}

// The float32 reduction for rows below kReduce4MinN: a block owns 32 columns, one whole 128-byte
// line of every partial row (16 columns of 4 bytes left each line half used, and the neighbouring
// block, on another XCD, fetched the same line again: the counters read twice the partial bytes).
// Lane l of wave k reads columns 4 * (l % 8) .. + 3 of partial rows p = 32 * i + 8 * k + l / 8
// (i = 0 .. kMaxPartials / 32 - 1, all loads in flight together) and adds them in order of i; the
// eight row phases of a wave (l / 8) are added by a butterfly over lane bits 3, 4, 5 (IEEE addition
// commutes, so every lane ends with the same bits), then the four waves in order.
static_assert(kMaxPartials % 32 == 0, "dw_reduce32_kernel reads partial rows in groups of 32");
inline __global__ void __launch_bounds__(256) dw_reduce32_kernel(const float* part, int64_t ldp,
                                                                 int P, int N, float* dw,
                                                                 float* dw2, int64_t set_stride) {
  if (blockIdx.y) {
    part += set_stride;
    dw = dw2;
  }
  constexpr int L = kMaxPartials / 32;
  __shared__ float4 buf[4][8];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c4 = lane & 7, ph = lane >> 3;
  const int col = blockIdx.x * 32 + c4 * 4;
  float4 v[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int p = 32 * i + 8 * wv + ph;
    v[i] = (col < N && p < P) ? *reinterpret_cast<const float4*>(part + (int64_t)p * ldp + col)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 t = v[0];
#pragma unroll
  for (int i = 1; i < L; ++i) {
    t.x += v[i].x;
    t.y += v[i].y;
    t.z += v[i].z;
    t.w += v[i].w;
  }
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
    t.x += __shfl_xor(t.x, m, 64);
    t.y += __shfl_xor(t.y, m, 64);
    t.z += __shfl_xor(t.z, m, 64);
    t.w += __shfl_xor(t.w, m, 64);
  }
  if (ph == 0) buf[wv][c4] = t;
  __syncthreads();
  if (wv == 0 && ph == 0 && col < N) {
    const float4 a = buf[0][c4], b = buf[1][c4], d = buf[2][c4], e = buf[3][c4];
    const float r[4] = {((a.x + b.x) + d.x) + e.x, ((a.y + b.y) + d.y) + e.y,
                        ((a.z + b.z) + d.z) + e.z, ((a.w + b.w) + d.w) + e.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (col + k < N) dw[col + k] = r[k];
  }
}

// Host side: the fixed-order float32 reduction of P partial rows into dw (and of the next P rows,
// set_stride floats on, into dw2 when sets = 2). Rows below kReduce4MinN take the 32-column kernel
// (N = 4096: 3.18 -> 2.82 us against 16 columns of 4-byte loads; N = 8192: 3.21 us against 3.32 for
// the 64-column kernel); from kReduce4MinN on the 64-column kernel is as fast or faster (N = 32768:
// 7.6 us against 8.2). The two add in different orders, each fixed, and the choice depends on N
// alone, so dw stays a function of the inputs.
constexpr int kReduce4MinN = 16384;
inline void launch_dw_reduce(const float* part, int64_t ldp, int P, int N, float* dw, float* dw2,
                             int64_t set_stride, unsigned sets, hipStream_t s) {
  if (N >= kReduce4MinN)
    hipLaunchKernelGGL(dw_reduce4_kernel, dim3((unsigned)((N + 63) / 64), sets), dim3(256), 0, s,
                       part, ldp, P, N, dw, dw2, set_stride);
  else
    hipLaunchKernelGGL(dw_reduce32_kernel, dim3((unsigned)((N + 31) / 32), sets), dim3(256), 0, s,
                       part, ldp, P, N, dw, dw2, set_stride);
}

inline __global__ void fill_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace rmsn
