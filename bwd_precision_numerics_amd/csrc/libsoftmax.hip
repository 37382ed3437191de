// Softmax (include/libsoftmax.h) and float64 RMSNorm (the _f64 entry points of
// include/librmsnorm.h): argument validation, kernel selection and launches. Every argument check
// runs before the first HIP call; nothing is allocated.
#include "../../include/libsoftmax.h"
#include "host_common.hpp"
#include "rmsnorm_bwd.hpp"
#include "softmax.hpp"

using namespace rmsn;

namespace {

// 16-byte vectors per thread in the register kernels' row shapes: at most 4 in the backward (it
// keeps y and dy) while 1024 threads can share a row, 8 in the forward (one float per element; a
// 4096-wide 16-bit row is one wavefront with no LDS round). The forward's partial vector is handled
// in the last iteration only, which keeps its 8-vector instantiation at 112 registers (bf16 1024 x
// 50264: 70 -> 55 us against the streaming kernel).
constexpr int kSmMaxIters = 4;
// The backward's rows wider than 4 vectors a thread at 1024 threads keep y and dy in registers up
// to 8 vectors a thread (64 registers of raw data) rather than reading them twice; float16 up to 6
// (its 7- and 8-vector instantiations spill 14 to 64 registers).
int sm_bwd_reg_max_iters(rmsnorm_dtype d) { return d == RMSNORM_DTYPE_F16 ? 6 : 8; }
// Float64 streaming backward with its dw sums in registers: up to 8 vectors (16 values) per thread.
constexpr int kF64StreamRegVectors = 8;
constexpr int kSmFwdFullMaxIters = 8;
// Threads per block: the forward's row groups share a block's barriers, so it stays small; the
// backward was measured faster with 1024.
constexpr int kSmFwdBlockThreads = 256;
constexpr int kSmBwdBlockThreads = 1024;

bool sm_dtype_ok(int d) { return dtype_ok(d) || d == RMSNORM_DTYPE_F64; }

// Threads per row for a row of nv vectors (or elements): at most max_iters per thread.
void sm_shape(int64_t nv, int max_iters, int* tpr, int* iters) {
  *tpr = (int)clamp64(pow2_ceil(ceil_div(nv, max_iters)), 64, 1024);
  *iters = (int)ceil_div(nv, *tpr);
}

// Shape of a forward or backward row. Both kernel families of one direction take the same shape
// for the same N and dtype, so with 16-byte vectors they map elements to threads identically.
// peel: rows not 16-byte aligned, every matrix's rows at one offset from a 16-byte boundary; the
// kernels take 16-byte vectors between a head and a tail of single elements, and the mapping is
// sized for floor(N / V) vectors (the most a row holds).
rmsnorm_status plan_sm(int64_t M, int64_t N, rmsnorm_dtype dtype, bool wide_ok, bool peel,
                       rmsnorm_variant req, size_t acc_bytes, int slots, bool fwd, Plan* p) {
  const int64_t nv_wide = peel ? N / vec_elems(dtype) : ceil_div(N, vec_elems(dtype));
  wide_ok = wide_ok || peel;
  p->peel = peel;
  int tpr, iters, max_iters = kSmMaxIters;
  if (fwd) max_iters = kSmFwdFullMaxIters;
  sm_shape(nv_wide, max_iters, &tpr, &iters);
  const bool reg_ok = wide_ok && iters <= (fwd ? max_iters : sm_bwd_reg_max_iters(dtype));
  rmsnorm_variant v = req;
  if (v == RMSNORM_VARIANT_AUTO) v = reg_ok ? RMSNORM_VARIANT_REGISTERS : RMSNORM_VARIANT_STREAMING;
  if (v == RMSNORM_VARIANT_LDS || (v == RMSNORM_VARIANT_REGISTERS && !reg_ok))
    return RMSNORM_ERR_UNSUPPORTED;
  p->variant = v;
  p->wide = v == RMSNORM_VARIANT_REGISTERS || wide_ok;
  if (v == RMSNORM_VARIANT_STREAMING) {
    sm_shape(wide_ok ? nv_wide : N, max_iters, &tpr, &iters);
    iters = 0;
  } else if (!peel && dtype != RMSNORM_DTYPE_F64 && (p->sub = narrow_lanes(nv_wide)) > 0) {
    tpr = p->sub;  // narrow rows: segments of lanes, 64 / sub rows per wavefront
  }
  p->tpr = tpr;
  p->iters = iters;
  const int bt = fwd ? kSmFwdBlockThreads : kSmBwdBlockThreads;
  p->groups = tpr >= bt ? 1 : bt / tpr;
  p->lds = round16(acc_bytes * slots * (size_t)p->groups * (tpr / 64));
  p->grid = ceil_div(M, p->groups);
  if (p->grid > INT32_MAX) return RMSNORM_ERR_UNSUPPORTED;
  return RMSNORM_OK;
}

// The backward's instantiations the plan can select (float16 stops at 6 vectors a thread).
template <DT D, int IT, bool PEEL>
rmsnorm_status sm_bwd_launch(const Plan& p, const SmArgs& a, hipStream_t s, int block) {
  if constexpr (D == DT::F16 && IT > 6) return RMSNORM_ERR_UNSUPPORTED;
  else return launch(softmax_bwd_kernel<D, true, IT, PEEL>, p.grid, block, p.lds, s, a);
}

// 16-byte-vector kernels: streaming (iters 0) or registers, whole rows or peeled (PEEL).
template <DT D, bool FWD, bool PEEL>
rmsnorm_status sm_dispatch_iters(const Plan& p, const SmArgs& a, hipStream_t s) {
  const int block = p.groups * p.tpr;
#define RMSN_SM(IT)                                                                       \
  (FWD ? launch(softmax_fwd_kernel<D, true, IT, false, PEEL>, p.grid, block, p.lds, s, a) \
       : sm_bwd_launch<D, IT, PEEL>(p, a, s, block))
  const int iters = p.variant == RMSNORM_VARIANT_STREAMING ? 0 : p.iters;
  switch (iters) {
    case 0: return RMSN_SM(0);
    case 1: return RMSN_SM(1);
    case 2: return RMSN_SM(2);
    case 3: return RMSN_SM(3);
    case 4: return RMSN_SM(4);
    case 5: return RMSN_SM(5);
    case 6: return RMSN_SM(6);
    case 7: return RMSN_SM(7);
    case 8: return RMSN_SM(8);
    default: break;
  }
#undef RMSN_SM
  return RMSNORM_ERR_UNSUPPORTED;
}

// Narrow rows on segments of p.sub lanes (float32 compute), one 16-byte vector a lane.
template <DT D, bool FWD, int SB>
rmsnorm_status sm_sub_launch(const Plan& p, const SmArgs& a, hipStream_t s, int block, bool full) {
  if constexpr (!FWD)
    return launch(softmax_bwd_kernel<D, true, 1, false, SB>, p.grid, block, p.lds, s, a);
  else if (full)
    return launch(softmax_fwd_kernel<D, true, 1, true, false, SB>, p.grid, block, p.lds, s, a);
  else
    return launch(softmax_fwd_kernel<D, true, 1, false, false, SB>, p.grid, block, p.lds, s, a);
}

template <DT D, bool FWD>
rmsnorm_status sm_dispatch(const Plan& p, const SmArgs& a, hipStream_t s) {
  const int block = p.groups * p.tpr;
  if constexpr (D != DT::F64) {
    if (p.sub > 0) {
      const bool full = (int64_t)p.sub * Elem<D>::VEC == a.N;
      switch (p.sub) {
        case 4: return sm_sub_launch<D, FWD, 4>(p, a, s, block, full);
        case 8: return sm_sub_launch<D, FWD, 8>(p, a, s, block, full);
        case 16: return sm_sub_launch<D, FWD, 16>(p, a, s, block, full);
        case 32: return sm_sub_launch<D, FWD, 32>(p, a, s, block, full);
        default: return RMSNORM_ERR_UNSUPPORTED;
      }
    }
  }
  if constexpr (FWD) {
    constexpr int V = 16 / (int)sizeof(typename Elem<D>::S);
    if (p.variant != RMSNORM_VARIANT_STREAMING && !p.peel && (int64_t)p.iters * p.tpr * V == a.N) {
#define RMSN_SMF(IT) launch(softmax_fwd_kernel<D, true, IT, true>, p.grid, block, p.lds, s, a)
      switch (p.iters) {
        case 1: return RMSN_SMF(1);
        case 2: return RMSN_SMF(2);
        case 3: return RMSN_SMF(3);
        case 4: return RMSN_SMF(4);
        case 5: return RMSN_SMF(5);
        case 6: return RMSN_SMF(6);
        case 7: return RMSN_SMF(7);
        case 8: return RMSN_SMF(8);
        default: return RMSNORM_ERR_UNSUPPORTED;
      }
#undef RMSN_SMF
    }
  }
  if (p.peel) return sm_dispatch_iters<D, FWD, true>(p, a, s);
  if (p.variant == RMSNORM_VARIANT_STREAMING && !p.wide)
    return FWD ? launch(softmax_fwd_kernel<D, false, 0>, p.grid, block, p.lds, s, a)
               : launch(softmax_bwd_kernel<D, false, 0>, p.grid, block, p.lds, s, a);
  return sm_dispatch_iters<D, FWD, false>(p, a, s);
}

template <bool FWD>
rmsnorm_status sm_impl(const void* a_in, int64_t lda, const void* dy, int64_t lddy, void* out,
                       int64_t ldo, int64_t M, int64_t N, rmsnorm_dtype dtype,
                       rmsnorm_variant variant, void* stream) {
  if (!sm_dtype_ok(dtype) || !variant_ok(variant)) return RMSNORM_ERR_INVALID_ARG;
  if (M < 0 || N < 1) return RMSNORM_ERR_INVALID_ARG;
  if (N > RMSNORM_MAX_N) return RMSNORM_ERR_UNSUPPORTED;
  const int eb = elem_bytes(dtype);
  rmsnorm_status st;
  if ((st = check_matrix(a_in, lda, M, N, eb)) != RMSNORM_OK) return st;
  if (!FWD && (st = check_matrix(dy, lddy, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(out, ldo, M, N, eb)) != RMSNORM_OK) return st;
  const bool wide = wide_fits(a_in, lda, eb) && wide_fits(out, ldo, eb) &&
                    (FWD || wide_fits(dy, lddy, eb));
  // Rows not 16-byte aligned but all at one offset from a boundary (contiguous rows of an odd
  // width, say): whole vectors between a head and a tail of single elements.
  const bool peel = !wide && N >= 2 * vec_elems(dtype) && same_row_phase(a_in, lda, out, ldo, eb) &&
                    (FWD || same_row_phase(a_in, lda, dy, lddy, eb));
  const size_t acc = dtype == RMSNORM_DTYPE_F64 ? 8 : 4;
  Plan p;
  if ((st = plan_sm(M, N, dtype, wide, peel, variant, acc, FWD ? 3 : 1, FWD, &p)) != RMSNORM_OK)
    return st;
  if (M == 0) return RMSNORM_OK;
  SmArgs a;
  a.x = a_in; a.dy = dy; a.out = out;
  a.ldx = lda; a.lddy = lddy; a.ldo = ldo; a.M = M; a.N = (int)N;
  a.tpr = p.tpr; a.groups = p.groups;
  a.comp = p.variant == RMSNORM_VARIANT_STREAMING && long_chain(N, dtype, p.wide, p.tpr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case RMSNORM_DTYPE_F32: return sm_dispatch<DT::F32, FWD>(p, a, s);
    case RMSNORM_DTYPE_F16: return sm_dispatch<DT::F16, FWD>(p, a, s);
    case RMSNORM_DTYPE_BF16: return sm_dispatch<DT::BF16, FWD>(p, a, s);
    case RMSNORM_DTYPE_F64: return sm_dispatch<DT::F64, FWD>(p, a, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

// ---- float64 RMSNorm ------------------------------------------------------------------------------
size_t f64_workspace_bytes(int64_t M, int64_t N) {
  return (size_t)num_partials(M) * (size_t)N * sizeof(double);
}

rmsnorm_status f64_fwd_impl(const double* x, int64_t ldx, const double* w, double* y, int64_t ldy,
                            double* rstd, int64_t M, int64_t N, double eps, double offset,
                            void* stream) {
  if (M < 0 || N < 1 || !std::isfinite(eps) || eps < 0.0 || !std::isfinite(offset))
    return RMSNORM_ERR_INVALID_ARG;
  if (N > RMSNORM_MAX_N) return RMSNORM_ERR_UNSUPPORTED;
  rmsnorm_status st;
  if ((st = check_matrix(x, ldx, M, N, 8)) != RMSNORM_OK) return st;
  if ((st = check_matrix(y, ldy, M, N, 8)) != RMSNORM_OK) return st;
  if (M > 0 && w == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(w, 8) || !aligned(rstd, 8)) return RMSNORM_ERR_MISALIGNED;
  const bool wide = wide_fits(x, ldx, 8) && wide_fits(y, ldy, 8) && aligned(w, 16);
  int tpr, iters;
  sm_shape(wide ? ceil_div(N, 2) : N, kSmMaxIters, &tpr, &iters);
  const bool regs = wide && iters <= kSmMaxIters;
  const int groups = tpr >= kFwdBlockThreads ? 1 : kFwdBlockThreads / tpr;
  const int64_t grid = ceil_div(M, groups);
  if (grid > INT32_MAX) return RMSNORM_ERR_UNSUPPORTED;
  if (M == 0) return RMSNORM_OK;
  F64Args a = {};
  a.x = x; a.w = w; a.out = y; a.rstd = rstd;
  a.ldx = ldx; a.ldo = ldy; a.M = M; a.N = (int)N; a.tpr = tpr; a.groups = groups;
  a.eps = eps; a.offset = offset;
  const size_t lds = round16(sizeof(double) * (size_t)groups * (tpr / 64));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int block = groups * tpr;
  if (!regs)
    return wide ? launch(rms_f64_fwd_kernel<true>, grid, block, lds, s, a)
                : launch(rms_f64_fwd_kernel<false>, grid, block, lds, s, a);
  switch (iters) {
    case 1: return launch(rms_f64_fwd_rows_kernel<1>, grid, block, lds, s, a);
    case 2: return launch(rms_f64_fwd_rows_kernel<2>, grid, block, lds, s, a);
    case 3: return launch(rms_f64_fwd_rows_kernel<3>, grid, block, lds, s, a);
    case 4: return launch(rms_f64_fwd_rows_kernel<4>, grid, block, lds, s, a);
    default: return RMSNORM_ERR_UNSUPPORTED;
  }
}

rmsnorm_status f64_bwd_impl(const double* dy, int64_t lddy, const double* x, int64_t ldx,
                            const double* w, const double* rstd, double* dx, int64_t lddx,
                            double* dw, void* workspace, size_t wsb, int64_t M, int64_t N,
                            double offset, void* stream) {
  if (M < 0 || N < 1 || !std::isfinite(offset)) return RMSNORM_ERR_INVALID_ARG;
  if (N > RMSNORM_MAX_N) return RMSNORM_ERR_UNSUPPORTED;
  rmsnorm_status st;
  if ((st = check_matrix(dy, lddy, M, N, 8)) != RMSNORM_OK) return st;
  if ((st = check_matrix(x, ldx, M, N, 8)) != RMSNORM_OK) return st;
  if ((st = check_matrix(dx, lddx, M, N, 8)) != RMSNORM_OK) return st;
  if (dw == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (M > 0 && (w == nullptr || rstd == nullptr || workspace == nullptr))
    return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(w, 8) || !aligned(rstd, 8) || !aligned(dw, 8) || !aligned(workspace, 16))
    return RMSNORM_ERR_MISALIGNED;
  if (wsb < f64_workspace_bytes(M, N)) return RMSNORM_ERR_WORKSPACE;
  const bool wide = wide_fits(dy, lddy, 8) && wide_fits(x, ldx, 8) && wide_fits(dx, lddx, 8) &&
                    aligned(w, 16);
  F64Args a = {};
  a.x = x; a.dy = dy; a.w = w; a.rstd = const_cast<double*>(rstd); a.out = dx;
  a.part = static_cast<double*>(workspace); a.dw = dw;
  a.ldx = ldx; a.lddy = lddy; a.ldo = lddx; a.M = M; a.N = (int)N;
  a.P = (int)num_partials(M); a.offset = offset;
  int iters;
  bwd_shape(wide ? ceil_div(N, 2) : N, &a.tpr, &iters);
  a.groups = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {
    hipLaunchKernelGGL(fill_zero_f64_kernel, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s, dw,
                       (int)N);
    return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
  }
  const size_t lds = round16(sizeof(double) * 2 * (a.tpr / 64));
  if (wide && iters == 1) st = launch(rms_f64_bwd_rows_kernel<1>, a.P, a.tpr, lds, s, a);
  else if (wide && iters == 2) st = launch(rms_f64_bwd_rows_kernel<2>, a.P, a.tpr, lds, s, a);
  else if (wide && iters <= kF64StreamRegVectors)  // dw sums in registers
    st = launch(rms_f64_bwd_kernel<true, kF64StreamRegVectors>, a.P, a.tpr, lds, s, a);
  else
    st = wide ? launch(rms_f64_bwd_kernel<true>, a.P, a.tpr, lds, s, a)
              : launch(rms_f64_bwd_kernel<false>, a.P, a.tpr, lds, s, a);
  if (st != RMSNORM_OK) return st;
  hipLaunchKernelGGL(dw_reduce_kernel<double>, dim3((unsigned)ceil_div(N, 16)), dim3(256), 0, s,
                     a.part, N, a.P, (int)N, dw, nullptr, (int64_t)0);
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}

}  // namespace

// ---- exported C interface -------------------------------------------------------------------------
extern "C" {

__attribute__((visibility("default"))) rmsnorm_status softmax_fwd(
    const void* x, int64_t ldx, void* y, int64_t ldy, int64_t M, int64_t N, rmsnorm_dtype dtype,
    rmsnorm_variant variant, void* stream) {
  return sm_impl<true>(x, ldx, nullptr, 0, y, ldy, M, N, dtype, variant, stream);
}

__attribute__((visibility("default"))) rmsnorm_status softmax_bwd(
    const void* dy, int64_t lddy, const void* y, int64_t ldy, void* dx, int64_t lddx, int64_t M,
    int64_t N, rmsnorm_dtype dtype, rmsnorm_variant variant, void* stream) {
  return sm_impl<false>(y, ldy, dy, lddy, dx, lddx, M, N, dtype, variant, stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_fwd_f64(
    const double* x, int64_t ldx, const double* w, double* y, int64_t ldy, double* rstd,
    int64_t M, int64_t N, double eps, double offset, void* stream) {
  return f64_fwd_impl(x, ldx, w, y, ldy, rstd, M, N, eps, offset, stream);
}

__attribute__((visibility("default"))) size_t rmsnorm_bwd_f64_workspace_bytes(int64_t M,
                                                                              int64_t N) {
  if (M <= 0 || N < 1 || N > RMSNORM_MAX_N) return 0;
  return f64_workspace_bytes(M, N);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bwd_f64(
    const double* dy, int64_t lddy, const double* x, int64_t ldx, const double* w,
    const double* rstd, double* dx, int64_t lddx, double* dw, void* workspace,
    size_t workspace_bytes, int64_t M, int64_t N, double offset, void* stream) {
  return f64_bwd_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, workspace, workspace_bytes, M, N,
                      offset, stream);
}

}  // extern "C"
