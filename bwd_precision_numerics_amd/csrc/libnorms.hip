// LayerNorm (and GroupNorm) C interface: argument validation, kernel selection and launches.
//
// Same conventions as the RMSNorm entry points: every argument check runs before the first HIP
// call, nothing is allocated, work is enqueued on the caller's stream.
#include "groupnorm.hpp"
#include "host_common.hpp"
#include "layernorm.hpp"

using namespace rmsn;

namespace {

// Forward register kernel: one wavefront per row up to 8 vectors a thread (w and b then loaded
// at the store), x, w and b all held up to 4.
constexpr int kLnFwdMaxIters = 8;
constexpr int kLnFwdEarlyWbIters = 4;
constexpr int kLnBwdBlockThreads = 1024;
constexpr int kLnBwdRegMaxIters = 2;
// Rows in flight ahead of the current one, and whether xhat and w * dy are kept between the
// passes, per vectors-per-thread of the register backward.
// Streaming backward with dw and db sums in registers: up to 4 vectors per thread (4096 vectors a
// row at 1024 threads, e.g. N = 32768 in 16-bit types).
constexpr int kLnStreamRegVectors = 4;
template <int ITERS> struct LnBwdPipe;
template <> struct LnBwdPipe<1> {
  static constexpr int DEPTH = 1;
  static constexpr bool KEEP = true;
};
template <> struct LnBwdPipe<2> {
  static constexpr int DEPTH = 1;
  static constexpr bool KEEP = false;
};

size_t ln_workspace_bytes(int64_t M, int64_t N) {
  return 2 * (size_t)num_partials(M) * (size_t)partial_ld(N) * sizeof(float);
}

// ---- LayerNorm forward ----------------------------------------------------------------------------
// A wavefront per row up to 4 vectors a thread; wider rows get more wavefronts (x, w and b stay in
// registers through the two reductions). Both families use the same threads per row for 16-byte
// rows, so they sum in the same order.
void ln_fwd_shape(int64_t nv, int* tpr, int* iters) {
  *tpr = (int)clamp64(pow2_ceil(ceil_div(nv, kLnFwdMaxIters)), 64, 1024);
  *iters = (int)ceil_div(nv, *tpr);
}

// peel_ok: rows not 16-byte aligned (N >= 2 * V) take the streaming kernel with 16-byte vectors
// between an element-wise head and tail.
rmsnorm_status plan_ln_fwd(int64_t M, int64_t N, rmsnorm_dtype dtype, bool wide_ok,
                           rmsnorm_variant req, Plan* p, bool peel_ok = false) {
  const int64_t nv_wide = ceil_div(N, vec_elems(dtype));
  int tpr, iters;
  ln_fwd_shape(nv_wide, &tpr, &iters);
  const bool reg_ok = wide_ok && iters <= kLnFwdMaxIters;
  rmsnorm_variant v = req;
  if (v == RMSNORM_VARIANT_AUTO) v = reg_ok ? RMSNORM_VARIANT_REGISTERS : RMSNORM_VARIANT_STREAMING;
  if (v == RMSNORM_VARIANT_LDS || (v == RMSNORM_VARIANT_REGISTERS && !reg_ok))
    return RMSNORM_ERR_UNSUPPORTED;
  p->variant = v;
  p->wide = v == RMSNORM_VARIANT_REGISTERS || wide_ok;
  if (v == RMSNORM_VARIANT_STREAMING) {
    p->peel = !wide_ok && peel_ok;
    ln_fwd_shape(wide_ok || p->peel ? nv_wide : N, &tpr, &iters);
    iters = 0;
  } else if ((p->sub = narrow_lanes(nv_wide)) > 0) {
    tpr = p->sub;  // narrow rows: segments of lanes, 64 / sub rows per wavefront
  }
  p->tpr = tpr;
  p->iters = iters;
  p->groups = tpr >= kFwdBlockThreads ? 1 : kFwdBlockThreads / tpr;
  p->lds = round16(sizeof(float) * 2 * (size_t)p->groups * (tpr / 64));
  p->grid = ceil_div(M, p->groups);
  if (p->grid > INT32_MAX) return RMSNORM_ERR_UNSUPPORTED;
  return RMSNORM_OK;
}

template <DT D, bool HAS_B>
rmsnorm_status ln_fwd_dispatch(const Plan& p, const LnFwdArgs& a, hipStream_t s) {
  const int block = p.groups * p.tpr;
  if (p.variant == RMSNORM_VARIANT_STREAMING) {
    if (p.peel) return launch(ln_fwd_stream_kernel<D, true, HAS_B, true>, p.grid, block, p.lds, s, a);
    return p.wide ? launch(ln_fwd_stream_kernel<D, true, HAS_B>, p.grid, block, p.lds, s, a)
                  : launch(ln_fwd_stream_kernel<D, false, HAS_B>, p.grid, block, p.lds, s, a);
  }
  static_assert(kLnFwdEarlyWbIters == 4, "cases below");
  // Rows that the threads' vectors tile exactly take the FULL instantiation (no partial-vector
  // code; the same arithmetic).
  const bool full = (int64_t)p.iters * p.tpr * Elem<D>::VEC == a.N;
  if (p.sub > 0) {
#define RMSN_LNF_SUB(SB)                                                                         \
  (full ? launch(ln_fwd_rows_kernel<D, 1, HAS_B, false, true, SB>, p.grid, block, p.lds, s, a)   \
        : launch(ln_fwd_rows_kernel<D, 1, HAS_B, false, false, SB>, p.grid, block, p.lds, s, a))
    switch (p.sub) {
      case 4: return RMSN_LNF_SUB(4);
      case 8: return RMSN_LNF_SUB(8);
      case 16: return RMSN_LNF_SUB(16);
      case 32: return RMSN_LNF_SUB(32);
      default: return RMSNORM_ERR_UNSUPPORTED;
    }
#undef RMSN_LNF_SUB
  }
#define RMSN_LNF(IT, LATE)                                                                    \
  (full ? launch(ln_fwd_rows_kernel<D, IT, HAS_B, LATE, true>, p.grid, block, p.lds, s, a)  \
        : launch(ln_fwd_rows_kernel<D, IT, HAS_B, LATE>, p.grid, block, p.lds, s, a))
  switch (p.iters) {
    case 1: return RMSN_LNF(1, false);
    case 2: return RMSN_LNF(2, false);
    case 3: return RMSN_LNF(3, false);
    case 4: return RMSN_LNF(4, false);
    case 5: return RMSN_LNF(5, true);
    case 6: return RMSN_LNF(6, true);
    case 7: return RMSN_LNF(7, true);
    case 8: return RMSN_LNF(8, true);
    default: return RMSNORM_ERR_UNSUPPORTED;
  }
#undef RMSN_LNF
}

template <bool HAS_B>
rmsnorm_status ln_fwd_by_dtype(rmsnorm_dtype dtype, const Plan& p, const LnFwdArgs& a,
                               hipStream_t s) {
  switch (dtype) {
    case RMSNORM_DTYPE_F32: return ln_fwd_dispatch<DT::F32, HAS_B>(p, a, s);
    case RMSNORM_DTYPE_F16: return ln_fwd_dispatch<DT::F16, HAS_B>(p, a, s);
    case RMSNORM_DTYPE_BF16: return ln_fwd_dispatch<DT::BF16, HAS_B>(p, a, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

rmsnorm_status ln_fwd_impl(const void* x, int64_t ldx, const void* w, const void* b, void* y,
                           int64_t ldy, float* mean, float* rstd, int64_t M, int64_t N,
                           rmsnorm_dtype dtype, float eps, rmsnorm_variant variant, void* stream) {
  rmsnorm_status st = check_common(M, N, dtype, eps, 0.f);
  if (st != RMSNORM_OK) return st;
  if (!variant_ok(variant)) return RMSNORM_ERR_INVALID_ARG;
  if (variant == RMSNORM_VARIANT_LDS) return RMSNORM_ERR_UNSUPPORTED;  // no LDS-staged family
  const int eb = elem_bytes(dtype);
  if ((st = check_matrix(x, ldx, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(y, ldy, M, N, eb)) != RMSNORM_OK) return st;
  if (M > 0 && w == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(w, (uintptr_t)eb) || !aligned(b, (uintptr_t)eb) || !aligned(mean, 4) ||
      !aligned(rstd, 4))
    return RMSNORM_ERR_MISALIGNED;
  const bool wide = wide_fits(x, ldx, eb) && aligned(w, 16) && aligned(b, 16);
  // Otherwise whole 16-byte vectors of x between an element-wise head and tail (w and b funnel-
  // shifted, or element by element when they are not 16-byte aligned).
  const bool peel_ok = N >= 2 * vec_elems(dtype);
  Plan p;
  if ((st = plan_ln_fwd(M, N, dtype, wide, variant, &p, peel_ok)) != RMSNORM_OK) return st;
  if (M == 0) return RMSNORM_OK;

  LnFwdArgs a;
  a.x = x; a.w = w; a.b = b; a.y = y; a.mean = mean; a.rstd = rstd;
  a.ldx = ldx; a.ldy = ldy; a.M = M; a.N = (int)N;
  a.tpr = p.tpr; a.groups = p.groups; a.eps = eps;
  a.yvec = p.peel ? same_row_phase(x, ldx, y, ldy, eb) : wide_fits(y, ldy, eb);
  a.comp = p.variant == RMSNORM_VARIANT_STREAMING && long_chain(N, dtype, p.wide || p.peel, p.tpr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return b ? ln_fwd_by_dtype<true>(dtype, p, a, s) : ln_fwd_by_dtype<false>(dtype, p, a, s);
}

// ---- LayerNorm backward ---------------------------------------------------------------------------
// peel_regs_ok: rows not 16-byte aligned with x and dy rows at one offset from a 16-byte boundary
// and w 16-byte aligned; at most one whole vector per lane (floor(N / V) <= 1024) takes the
// peeled register kernel.
// narrow_ok: a wavefront's rows on narrow rows (up to 15 workspace-row counts of strides apart)
// are addressable as 32-bit byte offsets from its first row.
rmsnorm_status plan_ln_bwd(int64_t M, int64_t N, rmsnorm_dtype dtype, bool wide_ok,
                           rmsnorm_variant req, Plan* p, bool peel_regs_ok = false,
                           bool narrow_ok = false) {
  const int64_t nv_wide = ceil_div(N, vec_elems(dtype));
  int tpr, iters;
  bwd_shape(nv_wide, &tpr, &iters);
  const int64_t nv_peel = N / vec_elems(dtype);
  const bool peel_regs = !wide_ok && peel_regs_ok && nv_peel <= kLnBwdBlockThreads;
  const bool reg_ok = (wide_ok && iters <= kLnBwdRegMaxIters) || peel_regs;
  rmsnorm_variant v = req;
  if (v == RMSNORM_VARIANT_AUTO) v = reg_ok ? RMSNORM_VARIANT_REGISTERS : RMSNORM_VARIANT_STREAMING;
  if (v == RMSNORM_VARIANT_LDS) return RMSNORM_ERR_UNSUPPORTED;
  if (v == RMSNORM_VARIANT_REGISTERS && !reg_ok) return RMSNORM_ERR_UNSUPPORTED;
  p->variant = v;
  p->grid = num_partials(M);
  if (v == RMSNORM_VARIANT_STREAMING) {
    p->wide = wide_ok;
    bwd_shape(wide_ok ? nv_wide : N, &tpr, &iters);
    p->tpr = tpr;
    p->iters = 0;
    p->groups = 1;
    p->lds = round16(sizeof(float) * 2 * 2 * (tpr / 64));
    return RMSNORM_OK;
  }
  if (!wide_ok) {  // registers on peeled rows: one vector per lane, dw and db sums in LDS
    p->peel = true;
    p->wide = true;
    p->tpr = (int)clamp64(pow2_ceil(nv_peel), 64, kLnBwdBlockThreads);
    p->iters = 1;
    p->groups = kLnBwdBlockThreads / p->tpr;
    p->lds = round16(sizeof(float) * 2 * (size_t)p->groups * (p->tpr / 64) * 2) +
             2 * sizeof(float) * (size_t)p->groups * (size_t)peel_sum_floats(partial_ld(N));
    return RMSNORM_OK;
  }
  p->wide = true;
  const int V = vec_elems(dtype);
  if (v == RMSNORM_VARIANT_REGISTERS && narrow_ok && N % V == 0 &&
      (p->sub = narrow_lanes(nv_wide)) > 0) {
    // Narrow rows of whole vectors: 1024 / sub row groups of sub lanes; LDS only for the column
    // combine of the groups' dw and db sums (one after the other).
    p->tpr = p->sub;
    p->iters = 1;
    p->groups = kLnBwdBlockThreads / p->sub;
    p->lds = sizeof(float) * (size_t)combine_columns_floats(V);
    return RMSNORM_OK;
  }
  p->tpr = tpr;
  p->iters = iters;
  p->groups = kLnBwdBlockThreads / tpr;
  const size_t red_bytes = round16(sizeof(float) * 2 * (size_t)p->groups * (tpr / 64) * 2);
  // The combine's slices for the dw and the db sums sit past the row sums (the last step fills
  // them while its row sums are in use).
  const size_t combine_bytes =
      sizeof(float) * (size_t)(p->groups / 2) * tpr * iters * vec_elems(dtype);
  p->lds = red_bytes + 2 * combine_bytes;
  // Four or more groups at one vector a lane combine through the column combine's array instead,
  // from the start of the LDS, after the last row.
  const size_t columns_bytes = sizeof(float) * (size_t)combine_columns_floats(V);
  if (iters == 1 && p->groups >= 4 && p->lds < columns_bytes) p->lds = columns_bytes;
  return RMSNORM_OK;
}

template <DT D, bool HAS_DB>
rmsnorm_status ln_bwd_dispatch(const Plan& p, const LnBwdArgs& a, hipStream_t s) {
  const int block = p.groups * p.tpr;
  if (p.variant == RMSNORM_VARIANT_STREAMING) {
    // 16-byte rows of at most kLnStreamRegVectors vectors per thread keep dw, db in registers.
    if (p.wide && ceil_div(ceil_div(a.N, Elem<D>::VEC), p.tpr) <= kLnStreamRegVectors)
      return launch(ln_bwd_stream_kernel<D, true, HAS_DB, kLnStreamRegVectors>, p.grid, block,
                    p.lds, s, a);
    // Other rows keep the dw and db sums in LDS when both fit there (as the RMSNorm kernel).
    if (2 * (int64_t)a.ldp <= kStreamLdsAccFloats) {
      const size_t lds = 256 + 2 * sizeof(float) * (size_t)a.ldp;
      return p.wide
                 ? launch(ln_bwd_stream_kernel<D, true, HAS_DB, 0, true>, p.grid, block, lds, s, a)
                 : launch(ln_bwd_stream_kernel<D, false, HAS_DB, 0, true>, p.grid, block, lds, s, a);
    }
    return p.wide ? launch(ln_bwd_stream_kernel<D, true, HAS_DB>, p.grid, block, p.lds, s, a)
                  : launch(ln_bwd_stream_kernel<D, false, HAS_DB>, p.grid, block, p.lds, s, a);
  }
  if (p.peel) return launch(ln_bwd_peel_rows_kernel<D, HAS_DB>, p.grid, block, p.lds, s, a);
  const bool full = (int64_t)p.iters * p.tpr * Elem<D>::VEC == a.N;
  // The tail layouts and compile-time row-group widths of the RMSNorm register backward.
  const Tail tail = full ? Tail::FULL : (a.N % Elem<D>::VEC == 0 ? Tail::WHOLE : Tail::RAGGED);
  const int wpr = p.tpr / 64;
  if (block != kLnBwdBlockThreads) return RMSNORM_ERR_UNSUPPORTED;
  if (p.sub > 0) {  // narrow rows of whole vectors, one per lane
#define RMSN_LNB_SUB(T, SB)                                                                    \
  launch(ln_bwd_rows_kernel<D, 1, LnBwdPipe<1>::DEPTH, HAS_DB, LnBwdPipe<1>::KEEP, T, 0, SB>, \
         p.grid, block, p.lds, s, a)
#define RMSN_LNB_SUBT(SB) \
  (tail == Tail::FULL ? RMSN_LNB_SUB(Tail::FULL, SB) : RMSN_LNB_SUB(Tail::WHOLE, SB))
    if (tail == Tail::RAGGED) return RMSNORM_ERR_UNSUPPORTED;
    switch (p.sub) {
      case 4: return RMSN_LNB_SUBT(4);
      case 8: return RMSN_LNB_SUBT(8);
      case 16: return RMSN_LNB_SUBT(16);
      case 32: return RMSN_LNB_SUBT(32);
      default: return RMSNORM_ERR_UNSUPPORTED;
    }
#undef RMSN_LNB_SUBT
#undef RMSN_LNB_SUB
  }
#define RMSN_LNB(IT, T, W)                                                                      \
  launch(ln_bwd_rows_kernel<D, IT, LnBwdPipe<IT>::DEPTH, HAS_DB, LnBwdPipe<IT>::KEEP, T, W>, \
         p.grid, block, p.lds, s, a)
#define RMSN_LNB_WPR(IT, T)                         \
  (wpr == 1   ? RMSN_LNB(IT, T, 1)                  \
   : wpr == 2 ? RMSN_LNB(IT, T, 2)                  \
   : wpr == 4 ? RMSN_LNB(IT, T, 4)                  \
   : wpr == 8 ? RMSN_LNB(IT, T, 8)                  \
              : RMSN_LNB(IT, T, 16))
  switch (p.iters) {
    case 1:
      return tail == Tail::FULL    ? RMSN_LNB_WPR(1, Tail::FULL)
             : tail == Tail::WHOLE ? RMSN_LNB_WPR(1, Tail::WHOLE)
                                   : RMSN_LNB(1, Tail::RAGGED, 0);
    case 2:
      // Exactly tiled rows take the WHOLE instantiation here: the FULL one spilled registers at two
      // vectors a thread, and for these power-of-two widths dot / N and dot * (1 / N) agree.
      return tail != Tail::RAGGED ? RMSN_LNB(2, Tail::WHOLE, 16) : RMSN_LNB(2, Tail::RAGGED, 0);
    default: return RMSNORM_ERR_UNSUPPORTED;
  }
#undef RMSN_LNB_WPR
#undef RMSN_LNB
}

template <bool HAS_DB>
rmsnorm_status ln_bwd_by_dtype(rmsnorm_dtype dtype, const Plan& p, const LnBwdArgs& a,
                               hipStream_t s) {
  switch (dtype) {
    case RMSNORM_DTYPE_F32: return ln_bwd_dispatch<DT::F32, HAS_DB>(p, a, s);
    case RMSNORM_DTYPE_F16: return ln_bwd_dispatch<DT::F16, HAS_DB>(p, a, s);
    case RMSNORM_DTYPE_BF16: return ln_bwd_dispatch<DT::BF16, HAS_DB>(p, a, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

// Fixed-order column sums of P partial rows (stride ldp) into out[N], and of the next P rows into
// out2[N] when out2 is not null, in one launch; zeros when there are no rows.
rmsnorm_status reduce_partials(const float* part, int64_t P, int64_t N, float* out, float* out2,
                               hipStream_t s) {
  if (P == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s, out,
                       (int)N);
    if (out2)
      hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s,
                         out2, (int)N);
  } else {
    launch_dw_reduce(part, partial_ld(N), (int)P, (int)N, out, out2, P * partial_ld(N),
                     out2 ? 2u : 1u, s);
  }
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}

rmsnorm_status ln_bwd_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                           const void* w, const float* mean, const float* rstd, void* dx,
                           int64_t lddx, float* dw, float* db, void* workspace,
                           size_t workspace_bytes_given, int64_t M, int64_t N,
                           rmsnorm_dtype dtype, rmsnorm_variant variant, void* stream) {
  rmsnorm_status st = check_common(M, N, dtype, 0.f, 0.f);
  if (st != RMSNORM_OK) return st;
  if (!variant_ok(variant)) return RMSNORM_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  if ((st = check_matrix(dy, lddy, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(x, ldx, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(dx, lddx, M, N, eb)) != RMSNORM_OK) return st;
  if (dw == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (M > 0 && (w == nullptr || mean == nullptr || rstd == nullptr || workspace == nullptr))
    return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(w, (uintptr_t)eb) || !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(dw, 4) ||
      !aligned(db, 4) || !aligned(workspace, 16))
    return RMSNORM_ERR_MISALIGNED;
  if (workspace_bytes_given < ln_workspace_bytes(M, N)) return RMSNORM_ERR_WORKSPACE;
  const bool wide = wide_fits(dy, lddy, eb) && wide_fits(x, ldx, eb) && wide_fits(dx, lddx, eb) &&
                    aligned(w, 16);
  // Otherwise x and dy rows at one offset from a 16-byte boundary (and w 16-byte aligned) move
  // whole vectors between an element-wise head and tail.
  const bool peel_regs_ok = same_row_phase(x, ldx, dy, lddy, eb) && N >= 2 * vec_elems(dtype) &&
                            aligned(w, 16);
  const int64_t ld_max = ldx > lddy ? (ldx > lddx ? ldx : lddx) : (lddy > lddx ? lddy : lddx);
  const bool narrow_ok =
      ((int64_t)(64 / 4 - 1) * num_partials(M) * ld_max + N) * eb <= (int64_t)INT32_MAX;
  Plan p;
  if ((st = plan_ln_bwd(M, N, dtype, wide, variant, &p, peel_regs_ok, narrow_ok)) != RMSNORM_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t P = num_partials(M);
  float* part = static_cast<float*>(workspace);
  if (M > 0) {
    LnBwdArgs a;
    a.dy = dy; a.x = x; a.w = w; a.mean = mean; a.rstd = rstd; a.dx = dx; a.part = part;
    a.lddy = lddy; a.ldx = ldx; a.lddx = lddx; a.M = M;
    a.N = (int)N; a.ldp = (int)partial_ld(N); a.P = (int)P;
    a.tpr = p.tpr; a.groups = p.groups;
    a.comp = p.variant == RMSNORM_VARIANT_STREAMING && long_chain(N, dtype, p.wide, p.tpr);
    a.dxvec = p.peel && same_row_phase(x, ldx, dx, lddx, eb);
    st = db ? ln_bwd_by_dtype<true>(dtype, p, a, s) : ln_bwd_by_dtype<false>(dtype, p, a, s);
    if (st != RMSNORM_OK) return st;
  }
  return reduce_partials(part, P, N, dw, db, s);
}

// ---- GroupNorm -----------------------------------------------------------------------------------
int gn_chunk_elems(rmsnorm_dtype d) {
  return d == RMSNORM_DTYPE_F32 ? gn_chunk<DT::F32>() : gn_chunk<DT::BF16>();
}

// Validates the shape; on success *chunks = B * C * K (one block per chunk) and *K.
rmsnorm_status gn_shape(int64_t B, int64_t C, int64_t S, int64_t G, int dtype, int64_t* K,
                        int64_t* chunks) {
  if (!dtype_ok(dtype)) return RMSNORM_ERR_INVALID_ARG;
  if (B < 0 || C < 1 || S < 1 || G < 1 || C % G != 0) return RMSNORM_ERR_INVALID_ARG;
  if (C > INT32_MAX) return RMSNORM_ERR_UNSUPPORTED;
  const int64_t Cg = C / G;
  if (S > RMSNORM_MAX_N || Cg > RMSNORM_MAX_N / S) return RMSNORM_ERR_UNSUPPORTED;  // group size
  *K = ceil_div(S, gn_chunk_elems((rmsnorm_dtype)dtype));
  if (B > 0 && C > (INT64_MAX / B) / S) return RMSNORM_ERR_INVALID_ARG;  // element count
  if (B > 0 && (C > INT32_MAX / *K || B > INT32_MAX / (C * *K))) return RMSNORM_ERR_UNSUPPORTED;
  *chunks = B * C * *K;
  return RMSNORM_OK;
}

rmsnorm_status gn_common(const void* x, const void* w, const void* out, const float* mean,
                         const float* rstd, void* workspace, size_t wsb, int64_t B, int64_t C,
                         int64_t S, int64_t G, rmsnorm_dtype dtype, int64_t* K, int64_t* chunks) {
  rmsnorm_status st = gn_shape(B, C, S, G, dtype, K, chunks);
  if (st != RMSNORM_OK) return st;
  if (B > 0 && (x == nullptr || w == nullptr || out == nullptr || workspace == nullptr))
    return RMSNORM_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  if (!aligned(x, (uintptr_t)eb) || !aligned(w, (uintptr_t)eb) || !aligned(out, (uintptr_t)eb) ||
      !aligned(mean, 4) || !aligned(rstd, 4) || !aligned(workspace, 16))
    return RMSNORM_ERR_MISALIGNED;
  if (wsb < (size_t)*chunks * sizeof(float2)) return RMSNORM_ERR_WORKSPACE;
  return RMSNORM_OK;
}

GnArgs gn_args(int64_t B, int64_t C, int64_t S, int64_t G, int64_t K, void* workspace) {
  GnArgs a = {};
  a.B = B; a.C = C; a.S = S; a.G = (int)G; a.Cg = (int)(C / G); a.K = (int)K;
  a.ws = static_cast<float2*>(workspace);
  return a;
}

// Segments of at most a quarter chunk (S <= CH / 4) take one chunk per wavefront, four a block
// (WPC): bf16 (2, 1280, 32 x 32), 32 groups, 1024-element segments, had filled a quarter of each
// 256-thread chunk block.
template <DT D, bool WIDE, bool WPC>
rmsnorm_status gn_fwd_launch_as(const GnArgs& a, int64_t chunks, hipStream_t s) {
  const unsigned grid = (unsigned)(WPC ? ceil_div(chunks, 4) : chunks);
  hipLaunchKernelGGL((gn_stats_kernel<D, WIDE, WPC>), dim3(grid), dim3(kGnThreads), 0, s, a);
  if (a.b)
    hipLaunchKernelGGL((gn_fwd_kernel<D, WIDE, true, WPC>), dim3(grid), dim3(kGnThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gn_fwd_kernel<D, WIDE, false, WPC>), dim3(grid), dim3(kGnThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}
template <DT D, bool WIDE>
rmsnorm_status gn_fwd_launch(const GnArgs& a, int64_t chunks, hipStream_t s) {
  return a.S <= gn_chunk<D>() / 4 ? gn_fwd_launch_as<D, WIDE, true>(a, chunks, s)
                                  : gn_fwd_launch_as<D, WIDE, false>(a, chunks, s);
}

template <DT D, bool WIDE, bool WPC>
rmsnorm_status gn_bwd_launch_as(const GnArgs& a, int64_t chunks, hipStream_t s) {
  const unsigned grid = (unsigned)(WPC ? ceil_div(chunks, 4) : chunks);
  hipLaunchKernelGGL((gn_bwd_sums_kernel<D, WIDE, WPC>), dim3(grid), dim3(kGnThreads), 0, s, a);
  hipLaunchKernelGGL((gn_bwd_dx_kernel<D, WIDE, WPC>), dim3(grid), dim3(kGnThreads), 0, s,
                     a);  // also writes dW, dB
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}
template <DT D, bool WIDE>
rmsnorm_status gn_bwd_launch(const GnArgs& a, int64_t chunks, hipStream_t s) {
  return a.S <= gn_chunk<D>() / 4 ? gn_bwd_launch_as<D, WIDE, true>(a, chunks, s)
                                  : gn_bwd_launch_as<D, WIDE, false>(a, chunks, s);
}

template <bool FWD, bool WIDE>
rmsnorm_status gn_by_dtype(rmsnorm_dtype dtype, const GnArgs& a, int64_t chunks, hipStream_t s) {
  switch (dtype) {
    case RMSNORM_DTYPE_F32:
      return FWD ? gn_fwd_launch<DT::F32, WIDE>(a, chunks, s) : gn_bwd_launch<DT::F32, WIDE>(a, chunks, s);
    case RMSNORM_DTYPE_F16:
      return FWD ? gn_fwd_launch<DT::F16, WIDE>(a, chunks, s) : gn_bwd_launch<DT::F16, WIDE>(a, chunks, s);
    case RMSNORM_DTYPE_BF16:
      return FWD ? gn_fwd_launch<DT::BF16, WIDE>(a, chunks, s) : gn_bwd_launch<DT::BF16, WIDE>(a, chunks, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

// 16-byte accesses: every chunk starts 16-byte aligned when the bases are and S * sizeof(T) is a
// multiple of 16 (chunks are whole numbers of vectors).
bool gn_wide(const void* p, int64_t S, int eb) { return aligned(p, 16) && (S * eb) % 16 == 0; }

// (batch, group) rows held whole by one row group (one launch per forward, x read once) instead of
// chunks, when the spatial size fits one chunk (the per-chunk pairs then hold one chunk per segment,
// the layout the parameter sums read) and the backward's LDS for one row (p1, p2 and the segment
// pairs, and its reduction slots, 2 * (m + Cg) + 128 floats) stays within kGnRowsLdsFloats:
//   GN_ROWS_VEC   16-byte vectors and S a multiple of V: p1, p2 hold per-vector sums (m = n / V),
//                 rows of up to 4 vectors a lane at 1024 lanes (n <= 32768 16-bit, 16384 float32)
//   GN_ROWS_ELEM  otherwise p1, p2 hold single values (m = n), up to 16384 (float32 8192)
// Several rows a block occur only for rows of at most 2048 elements, whose LDS stays below it too.
enum GnRowsMode { GN_CHUNKS = 0, GN_ROWS_ELEM = 1, GN_ROWS_VEC = 2 };
int64_t gn_rows_max(rmsnorm_dtype d) { return d == RMSNORM_DTYPE_F32 ? 8192 : 16384; }
constexpr int64_t kGnRowsLdsFloats = 36864;  // 144 KiB of a compute unit's 160 KiB
GnRowsMode gn_rows_mode(int64_t n, int64_t S, int64_t Cg, rmsnorm_dtype d, bool wide) {
  if (S > gn_chunk_elems(d)) return GN_CHUNKS;
  const int V = vec_elems(d);
  if (wide && S % V == 0 && n <= 2 * gn_rows_max(d) && 2 * (n / V + Cg) + 128 <= kGnRowsLdsFloats)
    return GN_ROWS_VEC;
  if (n <= gn_rows_max(d) && 2 * (n + Cg) + 128 <= kGnRowsLdsFloats) return GN_ROWS_ELEM;
  return GN_CHUNKS;
}

// Row-kernel shape: one value a lane while 1024 threads can cover the row, else a power of two up
// to 4 16-byte vectors or 16 single elements a lane (many threads per row hide more latency than
// few threads with more values: bf16 (32, 256, 14 x 14), 32 groups, forward 7.1 -> 5.4 us and
// backward 11.0 -> 10.0 us against up to 4 vectors a lane); threads per row and rows per block
// (blocks of at least 256 threads). With 16-byte vectors, when all rows' threads would exceed one
// full round of the device (256 compute units x 2048 threads), a row takes half the threads and
// twice the vectors a lane (up to 4), so the whole grid is resident at once: bf16
// (32, 256, 32 x 32), 32 groups, forward 12.6 -> 9.9 us and backward 17.1 -> 14.3 us; rows that
// already fit keep one vector a lane ((16, 512, 16 x 16): four a lane measured 4.9 -> 5.9 us and
// 9.2 -> 11.0 us).
constexpr int64_t kGnRoundThreads = 256 * 2048;
struct GnRowShape {
  int iters, tpr, rows;
  bool wide, vseg;
};
GnRowShape gn_row_shape(int64_t n, GnRowsMode mode, bool wide, rmsnorm_dtype d, int64_t nrows) {
  const int64_t nv = wide ? ceil_div(n, vec_elems(d)) : n;
  GnRowShape sh;
  sh.wide = wide;
  sh.vseg = mode == GN_ROWS_VEC;
  sh.tpr = (int)clamp64(pow2_ceil(nv), 64, 1024);
  sh.iters = (int)pow2_ceil(ceil_div(nv, sh.tpr));
  while (wide && sh.tpr > 64 && sh.iters < 4 && nrows * sh.tpr > kGnRoundThreads) {
    sh.tpr /= 2;
    sh.iters = (int)pow2_ceil(ceil_div(nv, sh.tpr));
  }
  sh.rows = sh.tpr >= 256 ? 1 : 256 / sh.tpr;
  return sh;
}

template <DT D, bool WIDE, bool HAS_B>
rmsnorm_status gn_rows_fwd_launch(const GnRowShape& sh, GnArgs a, hipStream_t s) {
  a.tpr = sh.tpr;
  a.rows = sh.rows;
  const int64_t grid = ceil_div(a.B * a.G, sh.rows);
  const size_t lds = sizeof(float) * 2 * (size_t)sh.rows * (sh.tpr / 64);
  const int block = sh.rows * sh.tpr;
#define RMSN_GNRF(IT) launch(gn_rows_fwd_kernel<D, WIDE, IT, HAS_B>, grid, block, lds, s, a)
  switch (sh.iters) {
    case 1: return RMSN_GNRF(1);
    case 2: return RMSN_GNRF(2);
    case 4: return RMSN_GNRF(4);
    default: break;
  }
  if constexpr (!WIDE) {  // single elements: up to 16 a lane
    switch (sh.iters) {
      case 8: return RMSN_GNRF(8);
      case 16: return RMSN_GNRF(16);
      default: break;
    }
  }
#undef RMSN_GNRF
  return RMSNORM_ERR_UNSUPPORTED;
}

template <DT D, bool WIDE>
rmsnorm_status gn_rows_bwd_launch(const GnRowShape& sh, GnArgs a, hipStream_t s) {
  a.tpr = sh.tpr;
  a.rows = sh.rows;
  const int64_t grid = ceil_div(a.B * a.G, sh.rows);
  const int n = a.Cg * (int)a.S;
  const int m = sh.vseg ? n / Elem<D>::VEC : n;
  const size_t lds =
      sizeof(float) * (size_t)sh.rows * gn_rows_bwd_lds_floats(sh.tpr / 64, a.Cg, m);
  if (lds > sizeof(float) * (size_t)kGnRowsLdsFloats) return RMSNORM_ERR_UNSUPPORTED;
  const int block = sh.rows * sh.tpr;
  rmsnorm_status st = RMSNORM_ERR_UNSUPPORTED;
#define RMSN_GNRB(IT, VS) launch(gn_rows_bwd_kernel<D, WIDE, IT, VS>, grid, block, lds, s, a)
  if constexpr (WIDE) {  // 16-byte vectors: up to 4 a lane, vector or single-value pairs
    if (sh.vseg) {
      if (sh.iters == 1) st = RMSN_GNRB(1, true);
      else if (sh.iters == 2) st = RMSN_GNRB(2, true);
      else if (sh.iters == 4) st = RMSN_GNRB(4, true);
    } else {
      if (sh.iters == 1) st = RMSN_GNRB(1, false);
      else if (sh.iters == 2) st = RMSN_GNRB(2, false);
    }
  } else {  // single elements: up to 16 a lane
    if (sh.iters == 1) st = RMSN_GNRB(1, false);
    else if (sh.iters == 2) st = RMSN_GNRB(2, false);
    else if (sh.iters == 4) st = RMSN_GNRB(4, false);
    else if (sh.iters == 8) st = RMSN_GNRB(8, false);
    else if (sh.iters == 16) st = RMSN_GNRB(16, false);
  }
#undef RMSN_GNRB
  if (st != RMSNORM_OK) return st;
  return launch(gn_params_kernel, ceil_div(a.C, 4), 256, 0, s, a);
}

template <bool FWD>
rmsnorm_status gn_rows_by_dtype(rmsnorm_dtype dtype, const GnRowShape& sh, const GnArgs& a,
                                hipStream_t s) {
#define RMSN_GNR(D)                                                                          \
  (FWD ? (sh.wide ? (a.b ? gn_rows_fwd_launch<D, true, true>(sh, a, s)                       \
                         : gn_rows_fwd_launch<D, true, false>(sh, a, s))                     \
                  : (a.b ? gn_rows_fwd_launch<D, false, true>(sh, a, s)                      \
                         : gn_rows_fwd_launch<D, false, false>(sh, a, s)))                   \
       : (sh.wide ? gn_rows_bwd_launch<D, true>(sh, a, s) : gn_rows_bwd_launch<D, false>(sh, a, s)))
  switch (dtype) {
    case RMSNORM_DTYPE_F32: return RMSN_GNR(DT::F32);
    case RMSNORM_DTYPE_F16: return RMSN_GNR(DT::F16);
    case RMSNORM_DTYPE_BF16: return RMSN_GNR(DT::BF16);
  }
#undef RMSN_GNR
  return RMSNORM_ERR_INVALID_ARG;
}

rmsnorm_status gn_fwd_impl(const void* x, const void* w, const void* b, void* y, float* mean,
                           float* rstd, void* workspace, size_t wsb, int64_t B, int64_t C,
                           int64_t S, int64_t G, rmsnorm_dtype dtype, float eps, void* stream) {
  if (!std::isfinite(eps) || eps < 0.f) return RMSNORM_ERR_INVALID_ARG;
  int64_t K = 0, chunks = 0;
  rmsnorm_status st = gn_common(x, w, y, mean, rstd, workspace, wsb, B, C, S, G, dtype, &K, &chunks);
  if (st != RMSNORM_OK) return st;
  const int eb = elem_bytes(dtype);
  if (!aligned(b, (uintptr_t)eb)) return RMSNORM_ERR_MISALIGNED;
  if (B == 0) return RMSNORM_OK;
  GnArgs a = gn_args(B, C, S, G, K, workspace);
  a.x = x; a.w = w; a.b = b; a.out = y; a.mean = mean; a.rstd = rstd; a.eps = eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n = (C / G) * S;
  const bool rwide = aligned(x, 16) && aligned(y, 16) && (n * eb) % 16 == 0;
  const GnRowsMode mode = gn_rows_mode(n, S, C / G, dtype, rwide);
  if (mode != GN_CHUNKS)
    return gn_rows_by_dtype<true>(dtype, gn_row_shape(n, mode, rwide, dtype, B * G), a, s);
  const bool wide = gn_wide(x, S, eb) && gn_wide(y, S, eb);
  return wide ? gn_by_dtype<true, true>(dtype, a, chunks, s)
              : gn_by_dtype<true, false>(dtype, a, chunks, s);
}

rmsnorm_status gn_bwd_impl(const void* dy, const void* x, const void* w, const float* mean,
                           const float* rstd, void* dx, float* dw, float* db, void* workspace,
                           size_t wsb, int64_t B, int64_t C, int64_t S, int64_t G,
                           rmsnorm_dtype dtype, void* stream) {
  int64_t K = 0, chunks = 0;
  rmsnorm_status st = gn_common(x, w, dx, mean, rstd, workspace, wsb, B, C, S, G, dtype, &K,
                                &chunks);
  if (st != RMSNORM_OK) return st;
  if (dw == nullptr || (B > 0 && (dy == nullptr || mean == nullptr || rstd == nullptr)))
    return RMSNORM_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  if (!aligned(dy, (uintptr_t)eb) || !aligned(dw, 4) || !aligned(db, 4))
    return RMSNORM_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(C, 256)), dim3(256), 0, s, dw,
                       (int)C);
    if (db)
      hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(C, 256)), dim3(256), 0, s, db,
                         (int)C);
    return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
  }
  GnArgs a = gn_args(B, C, S, G, K, workspace);
  a.x = x; a.dy = dy; a.w = w; a.out = dx; a.dw = dw; a.db = db;
  a.mean = const_cast<float*>(mean); a.rstd = const_cast<float*>(rstd);
  const int64_t n = (C / G) * S;
  const bool rwide = aligned(x, 16) && aligned(dy, 16) && aligned(dx, 16) && (n * eb) % 16 == 0;
  const GnRowsMode mode = gn_rows_mode(n, S, C / G, dtype, rwide);
  if (mode != GN_CHUNKS)  // one chunk per segment (K = 1): the pairs' layout is shared
    return gn_rows_by_dtype<false>(dtype, gn_row_shape(n, mode, rwide, dtype, B * G), a, s);
  const bool wide = gn_wide(x, S, eb) && gn_wide(dy, S, eb) && gn_wide(dx, S, eb);
  return wide ? gn_by_dtype<false, true>(dtype, a, chunks, s)
              : gn_by_dtype<false, false>(dtype, a, chunks, s);
}

}  // namespace

// ---- exported C interface -------------------------------------------------------------------------
extern "C" {

__attribute__((visibility("default"))) rmsnorm_status layernorm_fwd(
    const void* x, int64_t ldx, const void* w, const void* b, void* y, int64_t ldy, float* mean,
    float* rstd, int64_t M, int64_t N, rmsnorm_dtype dtype, float eps, rmsnorm_variant variant,
    void* stream) {
  return ln_fwd_impl(x, ldx, w, b, y, ldy, mean, rstd, M, N, dtype, eps, variant, stream);
}

__attribute__((visibility("default"))) size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N,
                                                                            rmsnorm_dtype dtype) {
  if (!dtype_ok(dtype) || M <= 0 || N < 1 || N > RMSNORM_MAX_N) return 0;
  return ln_workspace_bytes(M, N);
}

__attribute__((visibility("default"))) rmsnorm_status layernorm_bwd(
    const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, const float* mean,
    const float* rstd, void* dx, int64_t lddx, float* dw, float* db, void* workspace,
    size_t workspace_bytes, int64_t M, int64_t N, rmsnorm_dtype dtype, rmsnorm_variant variant,
    void* stream) {
  return ln_bwd_impl(dy, lddy, x, ldx, w, mean, rstd, dx, lddx, dw, db, workspace,
                     workspace_bytes, M, N, dtype, variant, stream);
}

__attribute__((visibility("default"))) size_t groupnorm_workspace_bytes(int64_t B, int64_t C,
                                                                        int64_t S, int64_t G,
                                                                        rmsnorm_dtype dtype) {
  int64_t K = 0, chunks = 0;
  if (gn_shape(B, C, S, G, dtype, &K, &chunks) != RMSNORM_OK) return 0;
  return (size_t)chunks * sizeof(float2);
}

__attribute__((visibility("default"))) rmsnorm_status groupnorm_fwd(
    const void* x, const void* w, const void* b, void* y, float* mean, float* rstd,
    void* workspace, size_t workspace_bytes, int64_t B, int64_t C, int64_t S, int64_t G,
    rmsnorm_dtype dtype, float eps, void* stream) {
  return gn_fwd_impl(x, w, b, y, mean, rstd, workspace, workspace_bytes, B, C, S, G, dtype, eps,
                     stream);
}

__attribute__((visibility("default"))) rmsnorm_status groupnorm_bwd(
    const void* dy, const void* x, const void* w, const float* mean, const float* rstd, void* dx,
    float* dw, float* db, void* workspace, size_t workspace_bytes, int64_t B, int64_t C, int64_t S,
    int64_t G, rmsnorm_dtype dtype, void* stream) {
  return gn_bwd_impl(dy, x, w, mean, rstd, dx, dw, db, workspace, workspace_bytes, B, C, S, G,
                     dtype, stream);
}

}  // extern "C"
