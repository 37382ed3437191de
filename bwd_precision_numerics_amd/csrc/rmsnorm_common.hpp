// Shared device helpers for the RMSNorm kernels (gfx950, wave64).
//
// Element I/O: 16-bit types travel as 16-byte vectors of 8 elements and fp32 as 16-byte vectors
// of 4; the element-wise ("narrow") path moves one element at a time and serves any alignment.
// Upcasts are exact; downcasts are round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 under the default round mode).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace rmsn {

enum class DT : int { F32 = 0, F16 = 1, BF16 = 2, F64 = 3 };

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <DT D> struct Elem;
template <> struct Elem<DT::F32> { using S = float; static constexpr int VEC = 4; };
template <> struct Elem<DT::F16> { using S = uint16_t; static constexpr int VEC = 8; };
template <> struct Elem<DT::BF16> { using S = uint16_t; static constexpr int VEC = 8; };
template <> struct Elem<DT::F64> { using S = double; static constexpr int VEC = 2; };

// The narrowing conversions below take their float32 operand through `materialize`: an empty asm
// with a register constraint (no instruction is emitted). It stops the backend from folding a
// float32 multiply into the conversion (gfx950 v_fma_mixlo_f16 rounds the exact product once to
// binary16), so every product is rounded to float32 first and then to the 16-bit type, as the
// contract states: y = T(fl(a * b)).
__device__ __forceinline__ float materialize(float v) {
  asm("" : "+v"(v));
  return v;
}

// ---- scalar conversions ------------------------------------------------------------------------
template <DT D> __device__ __forceinline__ float to_f32(typename Elem<D>::S s);
template <> __device__ __forceinline__ float to_f32<DT::F32>(float s) { return s; }
template <> __device__ __forceinline__ float to_f32<DT::F16>(uint16_t s) {
  return (float)__builtin_bit_cast(_Float16, s);
}
template <> __device__ __forceinline__ float to_f32<DT::BF16>(uint16_t s) {
  return __uint_as_float((uint32_t)s << 16);
}

template <DT D> __device__ __forceinline__ typename Elem<D>::S from_f32(float f);
template <> __device__ __forceinline__ float from_f32<DT::F32>(float f) { return f; }
template <> __device__ __forceinline__ uint16_t from_f32<DT::F16>(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)materialize(f));
}
template <> __device__ __forceinline__ uint16_t from_f32<DT::BF16>(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)materialize(f));
}

// ---- packed pairs (one 32-bit word holds two 16-bit elements) -----------------------------------
template <DT D> __device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi);
template <> __device__ __forceinline__ void unpack2<DT::BF16>(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ void unpack2<DT::F16>(uint32_t w, float& lo, float& hi) {
  f32x2_t f = __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
  lo = f.x;
  hi = f.y;
}
template <DT D> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<DT::BF16>(float lo, float hi) {
  f32x2_t f = {materialize(lo), materialize(hi)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
template <> __device__ __forceinline__ uint32_t pack2<DT::F16>(float lo, float hi) {
  f32x2_t f = {materialize(lo), materialize(hi)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
}

// ---- vector I/O --------------------------------------------------------------------------------
// VecIO<D, true>: 16-byte vectors (requires 16-byte aligned addresses).
// VecIO<D, false>: single elements.
template <DT D, bool WIDE> struct VecIO;

// Raw (untyped) buffer access: a 128-bit descriptor in scalar registers holds a row's base address,
// and each access names a 32-bit lane offset (one vector register shared by all of a thread's
// accesses) plus a wave-uniform 32-bit offset in a scalar register. Dword 3 sets the descriptor's
// data format field (bits 15-18) to 4 (32 bits), without which untyped accesses return zero on
// gfx9-family GPUs; no swizzle, no index. The record count is left at 2^31 - 1: callers address
// only bytes of the row they own (partial vectors take the element-wise path).
using BufRsrc = __amdgpu_buffer_rsrc_t;
constexpr int kBufDword3 = 0x00020000;
constexpr int kBufNonTemporal = 2;  // cache-policy operand: non-temporal (nt) accesses
template <typename T>
__device__ __forceinline__ BufRsrc buf_rsrc(const T* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, 0x7fffffff, kBufDword3);
}

template <DT D> struct VecIO<D, true> {
  using S = typename Elem<D>::S;
  static constexpr int V = Elem<D>::VEC;
  using Raw = uint4;
  static __device__ __forceinline__ Raw zero() { return make_uint4(0u, 0u, 0u, 0u); }
  // 16 bytes at byte offset voff + soff of the buffer (soff wave-uniform).
  static __device__ __forceinline__ Raw load_b(BufRsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  static __device__ __forceinline__ void store_b(BufRsrc r, uint32_t voff, uint32_t soff, Raw v) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, soff,
                                           kBufNonTemporal);
  }
  static __device__ __forceinline__ Raw load(const S* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  // Non-temporal (nt) load, for streams read exactly once whose lines need not stay in the caches.
  static __device__ __forceinline__ Raw load_nt(const S* p) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(uint4,
                              __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  }
  static __device__ __forceinline__ Raw load_b_nt(BufRsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff,
                                                                           kBufNonTemporal));
  }
  static __device__ __forceinline__ Raw load_part(const S* p, int n) {
    S tmp[V];
#pragma unroll
    for (int i = 0; i < V; ++i) tmp[i] = (i < n) ? p[i] : S(0);
    return __builtin_bit_cast(uint4, tmp);
  }
  // Outputs are written once and not re-read by the kernel: non-temporal 16-byte stores keep
  // them from displacing the input stream in the caches.
  static __device__ __forceinline__ void store(S* p, Raw r) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, r), reinterpret_cast<u32x4_t*>(p));
  }
  static __device__ __forceinline__ void store_part(S* p, Raw r, int n) {
    S tmp[V];
    __builtin_memcpy(tmp, &r, sizeof(r));
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (i < n) p[i] = tmp[i];
  }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&f)[V]) {
    if constexpr (D == DT::F32) {
      f[0] = __uint_as_float(r.x);
      f[1] = __uint_as_float(r.y);
      f[2] = __uint_as_float(r.z);
      f[3] = __uint_as_float(r.w);
    } else {
      unpack2<D>(r.x, f[0], f[1]);
      unpack2<D>(r.y, f[2], f[3]);
      unpack2<D>(r.z, f[4], f[5]);
      unpack2<D>(r.w, f[6], f[7]);
    }
  }
  static __device__ __forceinline__ Raw pack(const float (&f)[V]) {
    if constexpr (D == DT::F32) {
      return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                        __float_as_uint(f[3]));
    } else {
      return make_uint4(pack2<D>(f[0], f[1]), pack2<D>(f[2], f[3]), pack2<D>(f[4], f[5]),
                        pack2<D>(f[6], f[7]));
    }
  }
};

template <DT D> struct VecIO<D, false> {
  using S = typename Elem<D>::S;
  static constexpr int V = 1;
  using Raw = S;
  static __device__ __forceinline__ Raw zero() { return S(0); }
  static __device__ __forceinline__ Raw load(const S* p) { return *p; }
  static __device__ __forceinline__ Raw load_nt(const S* p) { return *p; }
  static __device__ __forceinline__ Raw load_part(const S* p, int) { return *p; }
  static __device__ __forceinline__ void store(S* p, Raw r) { *p = r; }
  static __device__ __forceinline__ void store_part(S* p, Raw r, int) { *p = r; }
  static __device__ __forceinline__ void unpack(const Raw& r, float (&f)[1]) { f[0] = to_f32<D>(r); }
  static __device__ __forceinline__ Raw pack(const float (&f)[1]) { return from_f32<D>(f[0]); }
};

// ---- OCP 8-bit outputs ----------------------------------------------------------------------------
// gfx950 converts packed float32 pairs to e4m3 (fp8) or e5m2 (bf8) with round-to-nearest-even;
// overflow gives NaN in e4m3 (no infinities) and an infinity in e5m2.
enum class F8 : int { E4M3 = 0, E5M2 = 1 };

template <F8 F>
__device__ __forceinline__ uint32_t cvt_pair_f8(float a, float b, uint32_t old, bool hi) {
  a = materialize(a);
  b = materialize(b);
  if constexpr (F == F8::E4M3) {
    return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
              : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
  } else {
    return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, true)
              : (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, false);
  }
}
template <F8 F>
__device__ __forceinline__ uint32_t cvt4_f8(float a, float b, float c, float d) {
  return cvt_pair_f8<F>(c, d, cvt_pair_f8<F>(a, b, 0u, false), true);
}
template <F8 F>
__device__ __forceinline__ uint8_t cvt1_f8(float a) {
  return (uint8_t)(cvt_pair_f8<F>(a, 0.f, 0u, false) & 0xffu);
}

// float -> T -> float (the inner cast of the round-twice convention); identity for fp32.
template <DT D> __device__ __forceinline__ float round_trip(float f) {
  if constexpr (D == DT::F32) {
    return f;
  } else {
    return to_f32<D>(from_f32<D>(f));
  }
}

// Row group of a thread in a block of row groups of tpr threads. tpr is a multiple of 64, so all
// lanes of a wavefront share the group; reading it from the first lane makes it, and every row
// index and row pointer derived from it, wave-uniform (scalar registers), so row addresses need no
// per-lane 64-bit registers.
__device__ __forceinline__ int wave_group(int tid, int tpr) {
  return __builtin_amdgcn_readfirstlane(tid / tpr);
}

// Element col of a row: the byte offset is formed in 32 bits (unsigned; rows are far below 4 GiB),
// so with a wave-uniform row pointer the compiler addresses the element as scalar base + one 32-bit
// lane offset instead of a 64-bit per-lane address. Precondition: col >= 0.
template <typename T>
__device__ __forceinline__ T* at(T* row, int col) {
  using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
  return reinterpret_cast<T*>(reinterpret_cast<B*>(row) + (uint32_t)col * (uint32_t)sizeof(T));
}

// Elements of a row before its first 16-byte boundary (at most V - 1, at most N): the head a
// kernel for rows that are not 16-byte aligned moves element by element before whole vectors.
template <typename S>
__device__ __forceinline__ int peel_head(const S* row, int N) {
  const int h = (int)(((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) / (uint32_t)sizeof(S));
  return h < N ? h : N;
}

// The 16-byte vector of a row's elements [c, c + V) for c = 16-byte column + h (0 < h < V), from
// the aligned vectors A = [c - h, c - h + V) and B = [c - h + V, c - h + 2V): a funnel shift by h
// elements (H a compile-time constant; peel_vec dispatches on the block-uniform h).
template <DT D, int H>
__device__ __forceinline__ uint4 funnel_vec(uint4 A, uint4 B) {
  const uint32_t c[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
  if constexpr (D == DT::F32) {
    return make_uint4(c[H], c[H + 1], c[H + 2], c[H + 3]);
  } else {
    constexpr int m = H / 2;
    if constexpr (H % 2 == 0) {
      return make_uint4(c[m], c[m + 1], c[m + 2], c[m + 3]);
    } else {  // odd element shift: the high half of dword k and the low half of dword k + 1
      return make_uint4(__builtin_amdgcn_alignbyte(c[m + 1], c[m], 2),
                        __builtin_amdgcn_alignbyte(c[m + 2], c[m + 1], 2),
                        __builtin_amdgcn_alignbyte(c[m + 3], c[m + 2], 2),
                        __builtin_amdgcn_alignbyte(c[m + 4], c[m + 3], 2));
    }
  }
}
template <DT D>
__device__ __forceinline__ uint4 peel_vec(int h, uint4 A, uint4 B) {
  switch (h) {
    case 1: return funnel_vec<D, 1>(A, B);
    case 2: return funnel_vec<D, 2>(A, B);
    case 3: return funnel_vec<D, 3>(A, B);
    default: break;
  }
  if constexpr (D != DT::F32) {
    switch (h) {
      case 4: return funnel_vec<D, 4>(A, B);
      case 5: return funnel_vec<D, 5>(A, B);
      case 6: return funnel_vec<D, 6>(A, B);
      case 7: return funnel_vec<D, 7>(A, B);
      default: break;
    }
  }
  return A;  // h = 0
}

// The gain elements [col, col + V) of a peeled row's vector (col = h + j * V, h the row's head):
// one aligned vector when h = 0; two and a funnel shift when w is 16-byte aligned and the second
// vector lies inside w; else element by element (w misaligned, or the row's last vectors).
template <DT D, int V>
__device__ __forceinline__ void peel_w(const typename Elem<D>::S* wr, bool walign, int N, int h,
                                       int col, float (&wf)[V]) {
  using IO = VecIO<D, true>;
  static_assert(V == IO::V, "16-byte vectors");
  const int base = col - h;  // a multiple of V: w + base is 16-byte aligned when w is
  if (walign && (h == 0 || base + 2 * V <= N)) {
    const uint4 A = IO::load(at(wr, base));
    const uint4 B = h ? IO::load(at(wr, base + V)) : A;
    IO::unpack(peel_vec<D>(h, A, B), wf);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) wf[e] = to_f32<D>(wr[col + e]);
  }
}

// ---- reductions ----------------------------------------------------------------------------------
// Sum over the 64 lanes of a wave with DPP lane moves (register-to-register, no LDS round trip):
// pairs and quads (quad_perm), then rows of 16 (row_shr 4 and 8), then rows 0+1 and 2+3
// (row_bcast 15) and all four rows (row_bcast 31); lane 63 ends with the total, which is read into
// a scalar register, so every lane gets the same bits. The order of additions is fixed.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, BOUND_ZERO));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xb1, 0xf, true>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4e, 0xf, true>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x114, 0xf, true>(v);  // row_shr:4 (lanes 0-3 of a row add 0)
  v += dpp_move<0x118, 0xf, true>(v);  // row_shr:8: lane 15 of each row holds the row sum
  v += dpp_move<0x142, 0xa, false>(v); // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc, false>(v); // row_bcast:31 into rows 2 and 3: lane 63 holds the total
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over each aligned segment of SUB lanes (SUB = 4, 8, 16 or 32; a row group narrower than a
// wave), every lane getting its segment's sum. The moves are wave_sum's first steps: after the
// quad moves lane 3 of each quad holds its quad's sum, after row_shr:4 lane 7 of each 8 lanes,
// after row_shr:8 lane 15 of each row, after row_bcast:15 into rows 1 and 3 lanes 31 and 63 their
// halves'. A segment's last lane then holds exactly what wave_sum makes of the same lanes with
// every other lane of the wave zero, which only goes on to add +0 to it: adding one +0 here (turns
// a -0 sum into +0, changes nothing else) gives bit for bit wave_sum's result for a row whose
// vectors fill only the wave's first SUB lanes. The sum is spread over the segment with a
// cross-lane read (ds_bpermute, no LDS memory).
template <int SUB>
__device__ __forceinline__ float segment_sum(float v) {
  static_assert(SUB == 4 || SUB == 8 || SUB == 16 || SUB == 32, "segment of 4 to 32 lanes");
  v += dpp_move<0xb1, 0xf, true>(v);
  v += dpp_move<0x4e, 0xf, true>(v);
  if constexpr (SUB >= 8) v += dpp_move<0x114, 0xf, true>(v);
  if constexpr (SUB >= 16) v += dpp_move<0x118, 0xf, true>(v);
  if constexpr (SUB == 32) v += dpp_move<0x142, 0xa, false>(v);
  const int lane = (int)__lane_id();
  v = __shfl(v, (lane & ~(SUB - 1)) + SUB - 1, 64);
  return v + 0.0f;
}

// Maximum over the 64 lanes with the same moves; here a lane without a source keeps its own value
// (max(v, v) = v) instead of reading 0. Every lane gets lane 63's result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_keep(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_keep<0xb1, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x4e, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x114, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x118, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  v = fmaxf(v, dpp_keep<0x143, 0xc>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Maximum over each aligned segment of SUB lanes with segment_sum's moves (lanes without a source
// keep their value), spread over the segment. Every order gives the same maximum.
template <int SUB>
__device__ __forceinline__ float segment_max(float v) {
  static_assert(SUB == 4 || SUB == 8 || SUB == 16 || SUB == 32, "segment of 4 to 32 lanes");
  v = fmaxf(v, dpp_keep<0xb1, 0xf>(v));
  v = fmaxf(v, dpp_keep<0x4e, 0xf>(v));
  if constexpr (SUB >= 8) v = fmaxf(v, dpp_keep<0x114, 0xf>(v));
  if constexpr (SUB >= 16) v = fmaxf(v, dpp_keep<0x118, 0xf>(v));
  if constexpr (SUB == 32) v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  const int lane = (int)__lane_id();
  return __shfl(v, (lane & ~(SUB - 1)) + SUB - 1, 64);
}

// A thread's share of a row sum in two interleaved float32 accumulators (even / odd elements of a
// vector). Chains of at most kPlainChainVectors vectors per thread add plainly, in the order the
// register kernels use; longer chains (the streaming kernels on very wide rows) set `comp` and
// compensate every addition (Kahan: c carries the low-order part lost so far), so that a row of
// 2^24 elements keeps its float32 sums within a few ulps of the exact value instead of drifting by
// about sqrt(chain length) ulps.
constexpr int kPlainChainVectors = 8;
struct RowAcc {
  float s0 = 0.f, s1 = 0.f, c0 = 0.f, c1 = 0.f;
  static __device__ __forceinline__ void kahan(float& s, float& c, float v) {
    const float y = v - c;
    const float t = s + y;
    c = (t - s) - y;
    s = t;
  }
  // s += v for element parity e
  __device__ __forceinline__ void add(int e, float v, bool comp) {
    float& s = (e & 1) ? s1 : s0;
    if (comp) kahan(s, (e & 1) ? c1 : c0, v);
    else s += v;
  }
  // s += a * b (one fused multiply-add on the plain path)
  __device__ __forceinline__ void fma(int e, float a, float b, bool comp) {
    float& s = (e & 1) ? s1 : s0;
    if (comp) kahan(s, (e & 1) ? c1 : c0, a * b);
    else s = __builtin_fmaf(a, b, s);
  }
  // s0 + s1 on the plain path (c0 = c1 = 0), bit for bit
  __device__ __forceinline__ float total() const { return (s0 + s1) - (c0 + c1); }
};

// Workgroup barrier that orders LDS only: outstanding global loads stay in flight across it, so a
// row prefetched before the barrier keeps streaming while the current row is reduced.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// red[0], red[STRIDE], ..., red[(W - 1) * STRIDE] added in that order. All W reads are issued
// before the first addition (one LDS wait instead of one per value).
template <int W, int STRIDE>
__device__ __forceinline__ float ordered_sum(const float* red) {
  float v[W];
#pragma unroll
  for (int w = 0; w < W; ++w) v[w] = red[w * STRIDE];
  float t = v[0];
#pragma unroll
  for (int w = 1; w < W; ++w) t += v[w];
  return t;
}
// The same for a wave count known only at run time: wpr is a power of two up to 16 (row groups
// of 64 to 1024 threads).
template <int STRIDE>
__device__ __forceinline__ float waves_sum(const float* red, int wpr) {
  switch (wpr) {
    case 2: return ordered_sum<2, STRIDE>(red);
    case 4: return ordered_sum<4, STRIDE>(red);
    case 8: return ordered_sum<8, STRIDE>(red);
    case 16: return ordered_sum<16, STRIDE>(red);
    default: {
      float t = red[0];
      for (int w = 1; w < wpr; ++w) t += red[w * STRIDE];
      return t;
    }
  }
}

// Sum of a value over the TPR threads of one row group (TPR = 64 * wpr). Waves publish their wave
// sums in red[slot * wpr + wave] and every thread adds them in wave order, so all threads of the
// group end with the same bits. Must be reached by every thread of the block when wpr > 1.
__device__ __forceinline__ float group_sum(float v, float* red, int wpr, int tl) {
  v = wave_sum(v);
  if (wpr > 1) {
    if ((tl & 63) == 0) red[tl >> 6] = v;
    lds_barrier();
    v = waves_sum<1>(red, wpr);
  }
  return v;
}

}  // namespace rmsn
