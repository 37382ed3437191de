// Softmax over the last dimension (forward and backward) and the float64 RMSNorm.
//
// Candle pull request 4059, "Add backward passes to the fused rms_norm, layer_norm and
// softmax_last_dim ops": the softmax forward computes in float32 for the 16-bit types and rounds
// once at the store; the backward is dx = y * (dy - sum(dy * y)) with the sum in float32 for the
// 16-bit types and float64 for float64; float64 kernels accumulate in float64 (a float accumulator
// made the float64 forward's statistics differ from the backward's).
//
//   forward   m = max_j x_j,  e_j = exp(x_j - m),  y_j = T(e_j * r),  r = 1 / sum_k e_k
// (one division per row; each y is within about three float32 ulps of the exact quotient before
// the cast, against nine vector instructions per element for an IEEE division). The float32 exp
// is the device library's, or on rows whose every e_j is a normal float32 a shorter evaluation of
// the same function to about two ulps (exp_row_normal below): the library's range reduction and
// its over- and underflow handling cost more vector instructions per element than the memory
// traffic leaves room for.
//   backward  s = sum_j dy_j * y_j,  dx_j = T(y_j * (dy_j - s))
//
// A is the compute type: float for float32 / float16 / bfloat16 I/O, double for float64.
#pragma once

#include "rmsnorm_bwd.hpp"

namespace rmsn {

template <DT D> struct Acc { using A = float; };
template <> struct Acc<DT::F64> { using A = double; };

// 16-byte vector or single-element I/O in the compute type.
template <DT D, bool WIDE> struct NumIO {
  using IO = VecIO<D, WIDE>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  static constexpr int V = IO::V;
  static __device__ __forceinline__ Raw load(const S* p, int n) {
    return n >= V ? IO::load(p) : IO::load_part(p, n);
  }
  // Non-temporal for full vectors: streams read exactly once.
  static __device__ __forceinline__ Raw load_nt(const S* p, int n) {
    return n >= V ? IO::load_nt(p) : IO::load_part(p, n);
  }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&f)[V]) { IO::unpack(r, f); }
  static __device__ __forceinline__ void store(S* p, const float (&f)[V], int n) {
    const Raw r = IO::pack(f);
    if (n >= V) IO::store(p, r);
    else IO::store_part(p, r, n);
  }
};
template <> struct NumIO<DT::F64, true> {
  using S = double;
  using Raw = uint4;
  static constexpr int V = 2;
  static __device__ __forceinline__ Raw load(const S* p, int n) {
    if (n >= 2) return *reinterpret_cast<const uint4*>(p);
    const uint2 u = __builtin_bit_cast(uint2, n > 0 ? p[0] : 0.0);
    return make_uint4(u.x, u.y, 0u, 0u);
  }
  static __device__ __forceinline__ Raw load_nt(const S* p, int n) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    if (n >= 2)
      return __builtin_bit_cast(uint4,
                                __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
    return load(p, n);
  }
  static __device__ __forceinline__ void unpack(const Raw& r, double (&f)[2]) {
    f[0] = __builtin_bit_cast(double, make_uint2(r.x, r.y));
    f[1] = __builtin_bit_cast(double, make_uint2(r.z, r.w));
  }
  static __device__ __forceinline__ void store(S* p, const double (&f)[2], int n) {
    if (n >= 2) {
      typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
      const uint2 a = __builtin_bit_cast(uint2, f[0]), b = __builtin_bit_cast(uint2, f[1]);
      const u32x4_t v = {a.x, a.y, b.x, b.y};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
    } else if (n > 0) {
      p[0] = f[0];
    }
  }
};
template <> struct NumIO<DT::F64, false> {
  using S = double;
  using Raw = double;
  static constexpr int V = 1;
  static __device__ __forceinline__ Raw load(const S* p, int) { return *p; }
  static __device__ __forceinline__ Raw load_nt(const S* p, int) { return *p; }
  static __device__ __forceinline__ void unpack(const Raw& r, double (&f)[1]) { f[0] = r; }
  static __device__ __forceinline__ void store(S* p, const double (&f)[1], int) { *p = f[0]; }
};

// Wave reductions by xor butterfly: at every step each lane combines the same two operands as its
// partner (a + b == b + a in IEEE arithmetic), so all lanes end with the same bits; the order of
// additions is fixed.
template <typename A> __device__ __forceinline__ A shfl_xor_any(A v, int m) {
  if constexpr (sizeof(A) == 8) {
    const int2 i = __builtin_bit_cast(int2, v);
    return __builtin_bit_cast(A, make_int2(__shfl_xor(i.x, m, 64), __shfl_xor(i.y, m, 64)));
  } else {
    return __shfl_xor(v, m, 64);
  }
}
template <typename A> __device__ __forceinline__ A wave_sum_x(A v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += shfl_xor_any(v, m);
  return v;
}
template <typename A> __device__ __forceinline__ A wave_max_x(A v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmax(v, shfl_xor_any(v, m));
  return v;
}
// float: the DPP reductions (register moves, result broadcast from lane 63); double: butterflies.
__device__ __forceinline__ float wave_sum_a(float v) { return wave_sum(v); }
__device__ __forceinline__ double wave_sum_a(double v) { return wave_sum_x(v); }
__device__ __forceinline__ float wave_max_a(float v) { return wave_max(v); }
__device__ __forceinline__ double wave_max_a(double v) { return wave_max_x(v); }

// Sum (MAX = false) or maximum over the TPR = 64 * wpr threads of a row group: waves publish their
// results in red[wave] and every thread combines them in wave order. Every thread of the block
// must call it when wpr > 1.
template <bool MAX, typename A>
__device__ __forceinline__ A group_reduce(A v, A* red, int wpr, int tl) {
  v = MAX ? wave_max_a(v) : wave_sum_a(v);
  if (wpr > 1) {
    if ((tl & 63) == 0) red[tl >> 6] = v;
    lds_barrier();
    v = red[0];
    for (int k = 1; k < wpr; ++k) v = MAX ? fmax(v, red[k]) : v + red[k];
  }
  return v;
}

// exp in the compute type (the accurate device library functions).
__device__ __forceinline__ float exp_a(float v) { return expf(v); }
__device__ __forceinline__ double exp_a(double v) { return exp(v); }

// exp(v) for -kSmNormalSpan < v <= 0, where the result is a normal float32. Method: a two-term
// (Cody-Waite style) split of the exponent. v * log2(e) = hi + lo with hi = fl(v * L),
// L = fl32(log2 e); the fma yields the rounding error of that product exactly, and v * Llo adds
// the part of log2(e) that L leaves out. The hardware base-2 exponential (v_exp_f32, about one
// ulp for normal results; it flushes results below 2^-126, hence the span) gives 2^hi, and
// 2^lo = 1 + lo * ln 2 + O(lo^2) with |lo| < 2^-16 leaves a second-order term below 2^-33.
// Emulated on the CPU with a correctly rounded 2^hi the error is at most 1.0 ulp; with the
// hardware's, about two. No special values: callers use it only on rows known to qualify.
constexpr float kSmNormalSpan = 87.0f;  // exp(-87) = 1.6e-38 > 2^-126
__device__ __forceinline__ float exp_row_normal(float v) {
  constexpr float kL = 0x1.715476p+0f;     // log2(e) rounded to float32
  constexpr float kLlo = 0x1.4ae0cp-26f;   // log2(e) - kL, rounded to float32
  constexpr float kLn2 = 0x1.62e43p-1f;    // ln(2) rounded to float32
  const float hi = v * kL;
  const float lo = __builtin_fmaf(v, kLlo, __builtin_fmaf(v, kL, -hi));
  const float p = __builtin_amdgcn_exp2f(hi);
  return __builtin_fmaf(p, lo * kLn2, p);
}

// Max of u and of v over the TPR threads of a row group in one LDS round: red holds 2 * wpr
// slots. Every thread of the block must call it when wpr > 1.
template <typename A>
__device__ __forceinline__ void group_max2(A& u, A& v, A* red, int wpr, int tl) {
  u = wave_max_a(u);
  v = wave_max_a(v);
  if (wpr > 1) {
    if ((tl & 63) == 0) {
      red[tl >> 6] = u;
      red[wpr + (tl >> 6)] = v;
    }
    lds_barrier();
    u = red[0];
    v = red[wpr];
    for (int k = 1; k < wpr; ++k) {
      u = fmax(u, red[k]);
      v = fmax(v, red[wpr + k]);
    }
  }
}

template <bool B> struct Flag { static constexpr bool value = B; };

struct SmArgs {
  const void* x;   // forward input, or the forward's output y (backward)
  const void* dy;  // backward only
  void* out;       // y (forward) or dx (backward)
  int64_t ldx, lddy, ldo, M;
  int N;
  int tpr, groups;
  int comp;  // streaming kernels: compensated float32 row sums (long per-thread chains)
};

// Two interleaved accumulators in the compute type; float sums of long chains are compensated
// (RowAcc), float64 sums are plain (a float64 chain of 2^24 terms stays far inside the tolerance).
template <typename A> struct SmAcc {
  A s0 = 0, s1 = 0;
  __device__ __forceinline__ void add(int e, A v, bool) { (e & 1 ? s1 : s0) += v; }
  __device__ __forceinline__ void fma(int e, A x, A y, bool) {
    A& s = e & 1 ? s1 : s0;
    s = ::fma(x, y, s);
  }
  __device__ __forceinline__ A total() const { return s0 + s1; }
};
template <> struct SmAcc<float> : RowAcc {};

// One element of a row in the compute type, and its store.
template <DT D>
__device__ __forceinline__ typename Acc<D>::A elem_in(const typename Elem<D>::S* p) {
  if constexpr (D == DT::F64) return *p;
  else return to_f32<D>(*p);
}
template <DT D>
__device__ __forceinline__ void elem_out(typename Elem<D>::S* p, typename Acc<D>::A v) {
  if constexpr (D == DT::F64) *p = v;
  else *p = from_f32<D>(v);
}

// Forward. Register kernel (ITERS > 0: the row's exp values stay in registers between the
// reductions and the store) or streaming (ITERS = 0: each pass reads x again from the caches).
// FULL (register kernel): the host has checked that N = ITERS * TPR * V, so every vector of every
// thread lies inside the row and the kernel carries no code for partial vectors or padding (that
// code alone would push the 8-vector kernel past its register budget).
// PEEL (16-byte vectors, rows not 16-byte aligned, y rows at x's offsets from a 16-byte boundary):
// the row's whole vectors start h < V elements in (h from the row's address); the vector mapping
// covers them, lanes 0 .. h-1 hold the h head elements and lanes 0 .. t-1 the t < V tail elements
// after the last whole vector. A lane's head element opens its even sum and its tail element
// closes its odd sum, in both kernel families, so they keep giving the same bits. The host sizes
// the mapping for floor(N / V) vectors: a row with one vector fewer leaves the last iteration's
// lanes idle, never an earlier one.
// The max pass also finds the row's minimum: when max - min < kSmNormalSpan (false for rows with
// infinities or only NaN), every e_j is a normal float32 and the float32 kernels use
// exp_row_normal, else the library exp. The choice is made per row from exact values, so the two
// kernel families take the same one. LDS: three reduction slots of wpr compute-type values per
// row group (max and -min, then the sum).
// SUB > 0 (float32 compute, rows of at most SUB vectors, one per lane): row groups of SUB lanes,
// 64 / SUB rows per wavefront, reduced with segment_max and segment_sum; each lane holds what it
// holds at one wavefront per row and the sums keep their bits, so y does not change. No LDS.
template <DT D, bool WIDE, int ITERS, bool FULL = false, bool PEEL = false, int SUB = 0>
__global__ void __launch_bounds__(1024) softmax_fwd_kernel(SmArgs a) {
  using A = typename Acc<D>::A;
  using IO = NumIO<D, WIDE>;
  using S = typename IO::S;
  constexpr int V = IO::V;
  constexpr bool F32 = sizeof(A) == 4;
  static_assert(!FULL || (ITERS > 0 && WIDE), "FULL applies to the register kernel");
  static_assert(!PEEL || (WIDE && !FULL), "PEEL takes 16-byte vectors and partial rows");
  static_assert(SUB == 0 || (F32 && WIDE && ITERS == 1 && !PEEL), "narrow rows: one vector a lane");
  extern __shared__ uint4 smem[];
  const int TPR = SUB ? SUB : a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  A* red = reinterpret_cast<A*>(smem) + grp * 3 * wpr;
  // Rows past M read row 0 (in bounds) and store nothing.
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
  constexpr int R = ITERS > 0 ? ITERS : 1;
  A ev[R][V];

  A mx = -INFINITY, nmn = -INFINITY;  // max and -min over the row
  A hx = -INFINITY, tx = -INFINITY;   // PEEL: the lane's head and tail elements
  if constexpr (PEEL) {
    if (tl < h) hx = elem_in<D>(xr + tl);
    if (tl < t) tx = elem_in<D>(xv + NV + tl);
    mx = fmax(hx, tx);
    if constexpr (F32) nmn = fmax(tl < h ? -hx : (A)-INFINITY, tl < t ? -tx : (A)-INFINITY);
  }
  if constexpr (ITERS > 0) {
    if constexpr (FULL) {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int col = (it * TPR + tl) * V;
        IO::unpack(IO::load_nt(xv + col, V), ev[it]);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          mx = fmax(mx, ev[it][e]);
          if constexpr (F32) nmn = fmax(nmn, -ev[it][e]);
        }
      }
    } else {
      // Only a row's last vector can be partial or absent (ITERS = ceil(vectors / TPR)): the
      // other iterations take the whole-vector code.
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int col = (it * TPR + tl) * V;
        if (it < ITERS - 1) {
          IO::unpack(IO::load(xv + col, V), ev[it]);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            mx = fmax(mx, ev[it][e]);
            if constexpr (F32) nmn = fmax(nmn, -ev[it][e]);
          }
          continue;
        }
        A f[V];
        if (col < NV) IO::unpack(IO::load(xv + col, NV - col), f);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const bool in = col + e < NV;
          ev[it][e] = in ? f[e] : (A)-INFINITY;
          mx = fmax(mx, ev[it][e]);
          if constexpr (F32) nmn = fmax(nmn, in ? -f[e] : (A)-INFINITY);
        }
      }
    }
  } else {
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      A f[V];
      IO::unpack(IO::load(xv + col, NV - col), f);
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (col + e < NV) {
          mx = fmax(mx, f[e]);
          if constexpr (F32) nmn = fmax(nmn, -f[e]);
        }
    }
  }
  if constexpr (SUB > 0) {
    mx = segment_max<SUB>(mx);
    nmn = segment_max<SUB>(nmn);
  } else if constexpr (F32) {
    group_max2(mx, nmn, red, wpr, tl);
  } else {
    mx = group_reduce<true>(mx, red, wpr, tl);
  }
  const bool fast = F32 && mx + nmn < (A)kSmNormalSpan;
  auto ex = [&](auto fast_tag, A v) -> A {
    if constexpr (F32 && decltype(fast_tag)::value) return exp_row_normal(v);
    else return exp_a(v);
  };

  // The register kernels keep the row only on the short-exp path. Otherwise they, like the
  // streaming kernel, read x again for the sum and for the store (from the caches), with the same
  // element-to-thread mapping and order, so register values are not held across the library exp.
  const bool in_regs = ITERS > 0 && fast;
  A s0 = 0, s1 = 0;
  A he = 0, te = 0;  // PEEL: exp of the lane's head and tail elements
  if (in_regs) {
    if constexpr (PEEL) {
      if (tl < h) he = ex(Flag<true>{}, hx - mx);
      if (tl < t) te = ex(Flag<true>{}, tx - mx);
      s0 = he;
    }
    // Padding lanes (partial rows) hold -inf, which the short exp does not take: select 0.
#pragma unroll
    for (int it = 0; it < R; ++it) {
      const int col = (it * TPR + tl) * V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        A q = ex(Flag<true>{}, ev[it][e] - mx);
        if (!FULL && it == R - 1) q = col + e < NV ? q : (A)0;
        ev[it][e] = q;
        if (e & 1) s1 += q;
        else s0 += q;
      }
    }
    if constexpr (PEEL) s1 += te;
  } else if (valid) {
    SmAcc<A> acc;
    auto sum_pass = [&](auto fast_tag) {
      if constexpr (PEEL) {
        if (tl < h) acc.add(0, ex(fast_tag, hx - mx), a.comp != 0);
      }
      for (int v = tl; v < nv; v += TPR) {
        const int col = v * V;
        A f[V];
        IO::unpack(IO::load(xv + col, NV - col), f);
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (col + e < NV) acc.add(e, ex(fast_tag, f[e] - mx), a.comp != 0);
      }
      if constexpr (PEEL) {
        if (tl < t) acc.add(1, ex(fast_tag, tx - mx), a.comp != 0);
      }
    };
    if (fast) sum_pass(Flag<true>{});
    else sum_pass(Flag<false>{});
    s0 = acc.total();
  }
  A sum;
  if constexpr (SUB > 0) sum = segment_sum<SUB>(s0 + s1);
  else sum = group_reduce<false>(s0 + s1, red + 2 * wpr, wpr, tl);
  if (!valid) return;
  const A r = (A)1 / sum;
  S* yr = static_cast<S*>(a.out) + row * a.ldo;
  S* yv = yr + h;
  if (in_regs) {
    if constexpr (PEEL) {
      if (tl < h) elem_out<D>(yr + tl, he * r);
      if (tl < t) elem_out<D>(yv + NV + tl, te * r);
    }
#pragma unroll
    for (int it = 0; it < R; ++it) {
      const int col = (it * TPR + tl) * V;
      const bool last = !FULL && it == R - 1;
      if (last && col >= NV) continue;
      A o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = ev[it][e] * r;
      IO::store(yv + col, o, last ? NV - col : V);
    }
  } else {
    auto store_pass = [&](auto fast_tag) {
      if constexpr (PEEL) {
        if (tl < h) elem_out<D>(yr + tl, ex(fast_tag, hx - mx) * r);
        if (tl < t) elem_out<D>(yv + NV + tl, ex(fast_tag, tx - mx) * r);
      }
      for (int v = tl; v < nv; v += TPR) {
        const int col = v * V;
        A f[V], o[V];
        IO::unpack(IO::load(xv + col, NV - col), f);
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = ex(fast_tag, f[e] - mx) * r;
        IO::store(yv + col, o, NV - col);
      }
    };
    if (fast) store_pass(Flag<true>{});
    else store_pass(Flag<false>{});
  }
}

// Backward: s = sum(dy * y) over the row, dx = T(y * (dy - s)). Register kernel (ITERS > 0: y and
// dy stay in registers) or streaming (ITERS = 0: read again for the elementwise pass). PEEL as
// for the forward (y, dy and dx rows at one offset from a 16-byte boundary): the lane's head
// product opens its even sum, its tail product closes its odd sum.
// SUB > 0: row groups of SUB lanes on narrow rows, as in the forward.
template <DT D, bool WIDE, int ITERS, bool PEEL = false, int SUB = 0>
__global__ void __launch_bounds__(1024) softmax_bwd_kernel(SmArgs a) {
  using A = typename Acc<D>::A;
  using IO = NumIO<D, WIDE>;
  using S = typename IO::S;
  using Raw = typename IO::Raw;
  constexpr int V = IO::V;
  static_assert(!PEEL || WIDE, "PEEL takes 16-byte vectors");
  static_assert(SUB == 0 || (sizeof(A) == 4 && WIDE && ITERS == 1 && !PEEL),
                "narrow rows: one vector a lane");
  extern __shared__ uint4 smem[];
  const int TPR = SUB ? SUB : a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  A* red = reinterpret_cast<A*>(smem) + grp * wpr;
  const S* yr = static_cast<const S*>(a.x) + (valid ? row : 0) * a.ldx;
  const S* dr = static_cast<const S*>(a.dy) + (valid ? row : 0) * a.lddy;
  int h = 0, t = 0;
  if constexpr (PEEL) {
    h = peel_head(yr, N);
    t = (N - h) % V;
  }
  const S* yv = yr + h;
  const S* dv = dr + h;
  const int NV = N - h - t;
  const int nv = (NV + V - 1) / V;
  constexpr int R = ITERS > 0 ? ITERS : 1;
  Raw ry[R], rd[R];

  A s0 = 0, s1 = 0;
  A hy = 0, hd = 0, ty = 0, td = 0;  // PEEL: the lane's head and tail elements of y and dy
  if constexpr (PEEL) {
    if (valid && tl < h) {
      hy = elem_in<D>(yr + tl);
      hd = elem_in<D>(dr + tl);
    }
    if (valid && tl < t) {
      ty = elem_in<D>(yv + NV + tl);
      td = elem_in<D>(dv + NV + tl);
    }
  }
  if constexpr (ITERS > 0) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      if (valid && col < NV) {
        ry[it] = IO::load_nt(yv + col, NV - col);
        rd[it] = IO::load_nt(dv + col, NV - col);
      } else {
        ry[it] = IO::load(yr, 0);
        rd[it] = IO::load(dr, 0);
      }
    }
    if constexpr (PEEL) {
      if (tl < h) s0 = fma(hd, hy, s0);
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      if (!(valid && col < NV)) continue;
      A yf[V], df[V];
      IO::unpack(ry[it], yf);
      IO::unpack(rd[it], df);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (e & 1) s1 = fma(df[e], yf[e], s1);
        else s0 = fma(df[e], yf[e], s0);
      }
    }
    if constexpr (PEEL) {
      if (tl < t) s1 = fma(td, ty, s1);
    }
  } else if (valid) {
    SmAcc<A> acc;
    if constexpr (PEEL) {
      if (tl < h) acc.fma(0, hd, hy, a.comp != 0);
    }
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      A yf[V], df[V];
      IO::unpack(IO::load(yv + col, NV - col), yf);
      IO::unpack(IO::load(dv + col, NV - col), df);
#pragma unroll
      for (int e = 0; e < V; ++e) acc.fma(e, df[e], yf[e], a.comp != 0);
    }
    if constexpr (PEEL) {
      if (tl < t) acc.fma(1, td, ty, a.comp != 0);
    }
    s0 = acc.total();
  }
  A s;
  if constexpr (SUB > 0) s = segment_sum<SUB>(s0 + s1);
  else s = group_reduce<false>(s0 + s1, red, wpr, tl);
  if (!valid) return;
  S* xr = static_cast<S*>(a.out) + row * a.ldo;
  S* xv = xr + h;
  if constexpr (PEEL) {
    if (tl < h) elem_out<D>(xr + tl, hy * (hd - s));
    if (tl < t) elem_out<D>(xv + NV + tl, ty * (td - s));
  }
  if constexpr (ITERS > 0) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      if (col >= NV) continue;
      A yf[V], df[V], o[V];
      IO::unpack(ry[it], yf);
      IO::unpack(rd[it], df);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = yf[e] * (df[e] - s);
      IO::store(xv + col, o, NV - col);
    }
  } else {
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      A yf[V], df[V], o[V];
      IO::unpack(IO::load(yv + col, NV - col), yf);
      IO::unpack(IO::load(dv + col, NV - col), df);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = yf[e] * (df[e] - s);
      IO::store(xv + col, o, NV - col);
    }
  }
}

// ---- float64 RMSNorm ------------------------------------------------------------------------------
// rstd = 1 / sqrt(sum(x^2) / N + eps), y = (x * rstd) * (offset + w); backward
// c = sum((offset + w) * dy * xhat) / N, dx = rstd * ((offset + w) * dy - xhat * c),
// dw = sum over rows of dy * xhat; all in float64. Two passes over each row (the second reads it
// again from the caches); the backward runs on the persistent grid of the 16-bit backward, its
// float64 partial rows of dw accumulated in the workspace and then summed in a fixed order.
struct F64Args {
  const double* x;
  const double* dy;
  const double* w;
  double* rstd;  // forward: written (may be null); backward: read
  double* out;   // y or dx
  double* part;  // [P, N] backward partials
  double* dw;
  int64_t ldx, lddy, ldo, M;
  int N, P, tpr, groups;
  double eps, offset;
};

template <bool WIDE>
__global__ void __launch_bounds__(1024) rms_f64_fwd_kernel(F64Args a) {
  using IO = NumIO<DT::F64, WIDE>;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];
  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int nv = (N + V - 1) / V;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  double* red = reinterpret_cast<double*>(smem) + grp * wpr;
  const double* xr = a.x + (valid ? row : 0) * a.ldx;
  double q0 = 0, q1 = 0;
  if (valid) {
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      double f[V];
      IO::unpack(IO::load(xr + col, N - col), f);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (e & 1) q1 = fma(f[e], f[e], q1);
        else q0 = fma(f[e], f[e], q0);
      }
    }
  }
  const double ss = group_reduce<false>(q0 + q1, red, wpr, tl);
  const double rs = 1.0 / sqrt(ss / (double)N + a.eps);
  if (!valid) return;
  if (tl == 0 && a.rstd) a.rstd[row] = rs;
  double* yr = a.out + row * a.ldo;
  for (int v = tl; v < nv; v += TPR) {
    const int col = v * V;
    double f[V], wf[V], o[V];
    IO::unpack(IO::load(xr + col, N - col), f);
    IO::unpack(IO::load(a.w + col, N - col), wf);
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = (f[e] * rs) * (a.offset + wf[e]);
    IO::store(yr + col, o, N - col);
  }
}

// KREG > 0 (16-byte vectors, at most KREG per thread): the dw sums stay in registers and are
// written once, instead of a float64 round trip through the workspace per row; same operations in
// the same order, bit-identical.
template <bool WIDE, int KREG = 0>
__global__ void __launch_bounds__(1024) rms_f64_bwd_kernel(F64Args a) {
  using IO = NumIO<DT::F64, WIDE>;
  constexpr int V = IO::V;
  static_assert(KREG == 0 || WIDE, "register sums take 16-byte vectors");
  extern __shared__ uint4 smem[];
  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int nv = (N + V - 1) / V;
  const int tl = threadIdx.x;
  const int b = blockIdx.x, P = a.P;
  double* red = reinterpret_cast<double*>(smem);  // [2][wpr]
  double* pr = a.part + (int64_t)b * N;
  constexpr int K = KREG > 0 ? KREG * V : 1;
  double acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = 0.0;
  if constexpr (KREG == 0) {
    // zeroed by the thread that owns each column below (same mapping, program order)
    for (int v = tl; v < nv; v += TPR) {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (v * V + e < N) pr[v * V + e] = 0.0;
    }
  }
  int s = 0;
  for (int64_t row = b; row < a.M; row += P, ++s) {
    const double* xr = a.x + row * a.ldx;
    const double* dr = a.dy + row * a.lddy;
    const double rs = a.rstd[row];
    double d0 = 0, d1 = 0;
    for (int v = tl; v < nv; v += TPR) {
      const int col = v * V;
      double f[V], df[V], wf[V];
      IO::unpack(IO::load(xr + col, N - col), f);
      IO::unpack(IO::load(dr + col, N - col), df);
      IO::unpack(IO::load(a.w + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const double xh = f[e] * rs, gd = (a.offset + wf[e]) * df[e];
        if (e & 1) d1 = fma(gd, xh, d1);
        else d0 = fma(gd, xh, d0);
      }
    }
    const double c = group_reduce<false>(d0 + d1, red + (s & 1) * wpr, wpr, tl) / (double)N;
    double* xo = a.out + row * a.ldo;
    auto elementwise = [&](int v, double* accv) {
      const int col = v * V;
      double f[V], df[V], wf[V], o[V];
      IO::unpack(IO::load(xr + col, N - col), f);
      IO::unpack(IO::load(dr + col, N - col), df);
      IO::unpack(IO::load(a.w + col, N - col), wf);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const double xh = f[e] * rs, gd = (a.offset + wf[e]) * df[e];
        o[e] = rs * (gd - xh * c);
        if constexpr (KREG > 0) accv[e] = fma(df[e], xh, accv[e]);
        else if (col + e < N) pr[col + e] = fma(df[e], xh, pr[col + e]);
      }
      IO::store(xo + col, o, N - col);
    };
    if constexpr (KREG > 0) {
#pragma unroll
      for (int k = 0; k < KREG; ++k) {
        const int v = tl + k * TPR;
        if (v < nv) elementwise(v, acc + k * V);
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
        if (col + e < N) pr[col + e] = acc[k * V + e];
    }
  }
}

__global__ void fill_zero_f64_kernel(double* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0;
}

// Register forward: a row of at most ITERS 16-byte vectors per thread stays in registers (with w)
// between the reduction and the store; x is read once.
template <int ITERS>
__global__ void __launch_bounds__(1024) rms_f64_fwd_rows_kernel(F64Args a) {
  using IO = NumIO<DT::F64, true>;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];
  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int tid = threadIdx.x;
  const int grp = tid / TPR;
  const int tl = tid - grp * TPR;
  const int64_t row = (int64_t)blockIdx.x * a.groups + grp;
  const bool valid = row < a.M;
  double* red = reinterpret_cast<double*>(smem) + grp * wpr;
  const double* xr = a.x + (valid ? row : 0) * a.ldx;
  uint4 rx[ITERS], rw[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    const bool ok = valid && col < N;
    rx[it] = IO::load_nt(xr + (ok ? col : 0), ok ? N - col : 0);
    rw[it] = IO::load(a.w + (ok ? col : 0), ok ? N - col : 0);
  }
  double q0 = 0, q1 = 0;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    double f[V];
    IO::unpack(rx[it], f);
    q0 = fma(f[0], f[0], q0);
    q1 = fma(f[1], f[1], q1);
  }
  const double ss = group_reduce<false>(q0 + q1, red, wpr, tl);
  const double rs = 1.0 / sqrt(ss / (double)N + a.eps);
  if (!valid) return;
  if (tl == 0 && a.rstd) a.rstd[row] = rs;
  double* yr = a.out + row * a.ldo;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    if (col >= N) continue;
    double f[V], wf[V], o[V];
    IO::unpack(rx[it], f);
    IO::unpack(rw[it], wf);
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = (f[e] * rs) * (a.offset + wf[e]);
    IO::store(yr + col, o, N - col);
  }
}

// Register backward on the persistent grid (block b of P owns rows b, b + P, ...; one row at a
// time per block, the next row's x, dy and rstd loaded while the current one is reduced). The dw
// column sums stay in registers and are written once as partial row b of the [P, N] workspace.
template <int ITERS>
__global__ void __launch_bounds__(1024) rms_f64_bwd_rows_kernel(F64Args a) {
  using IO = NumIO<DT::F64, true>;
  constexpr int V = IO::V;
  extern __shared__ uint4 smem[];
  const int TPR = a.tpr, wpr = TPR >> 6, N = a.N;
  const int tl = threadIdx.x;
  const int b = blockIdx.x, P = a.P;
  double* red = reinterpret_cast<double*>(smem);  // [2][wpr]
  double g[ITERS][V], acc[ITERS][V];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
    double wf[V];
    IO::unpack(IO::load(a.w + (col < N ? col : 0), col < N ? N - col : 0), wf);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      g[it][e] = a.offset + wf[e];
      acc[it][e] = 0.0;
    }
  }
  uint4 rx[2][ITERS], rd[2][ITERS];
  double rr[2];
  auto load_row = [&](int slot, int64_t row) {
    rr[slot] = a.rstd[row];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int col = (it * TPR + tl) * V;
      const bool ok = col < N;
      rx[slot][it] = IO::load_nt(a.x + row * a.ldx + (ok ? col : 0), ok ? N - col : 0);
      rd[slot][it] = IO::load_nt(a.dy + row * a.lddy + (ok ? col : 0), ok ? N - col : 0);
    }
  };
  const int64_t nloc = block_rows(a.M, P, b);
  if (nloc > 0) load_row(0, b);
  for (int64_t s0 = 0; s0 < nloc; s0 += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t s = s0 + j;
      if (s < nloc) {  // block-uniform
        if (s + 1 < nloc) load_row(j ^ 1, b + (s + 1) * P);
        const double rs = rr[j];
        double d0 = 0, d1 = 0;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
          double f[V], df[V];
          IO::unpack(rx[j][it], f);
          IO::unpack(rd[j][it], df);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const double xh = f[e] * rs, gd = g[it][e] * df[e];
            acc[it][e] = fma(df[e], xh, acc[it][e]);
            if (e & 1) d1 = fma(gd, xh, d1);
            else d0 = fma(gd, xh, d0);
          }
        }
        const double c = group_reduce<false>(d0 + d1, red + (s & 1) * wpr, wpr, tl) / (double)N;
        double* xo = a.out + (b + s * P) * a.ldo;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
          const int col = (it * TPR + tl) * V;
          if (col >= N) continue;
          double f[V], df[V], o[V];
          IO::unpack(rx[j][it], f);
          IO::unpack(rd[j][it], df);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const double xh = f[e] * rs;
            o[e] = rs * (g[it][e] * df[e] - xh * c);
          }
          IO::store(xo + col, o, N - col);
        }
      }
    }
  }
  double* pr = a.part + (int64_t)b * N;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int col = (it * TPR + tl) * V;
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (col + e < N) pr[col + e] = acc[it][e];
  }
}

}  // namespace rmsn
