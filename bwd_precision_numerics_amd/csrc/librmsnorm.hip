// librmsnorm: C interface, argument validation, kernel selection and launches.
//
// Every argument check runs before the first HIP call, so a rejected call launches nothing and
// touches no device state. The library keeps no state apart from a per-device cache of the LDS
// limit, filled on first use (a relaxed atomic per device: racing threads store the same value).
#include <mutex>

#include "host_common.hpp"
#include "rmsnorm_bwd.hpp"
#include "rmsnorm_fwd.hpp"

using namespace rmsn;

// Scratch of rmsnorm_bwd_noalloc: the dw partial rows in a file-scope device array, one copy per
// device, held until the process ends. Host code never passes `scratch` itself to a kernel (on the
// host the name stands for a host-side shadow, not a device address): each device's address comes
// from hipGetSymbolAddress on that device's first call, and only that address is used.
static __device__ __align__(256) float scratch[RMSNORM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kBwdBlockThreads = 1024;  // backward: 16 wavefronts per persistent block
constexpr int kBwdRegMaxIters = 2;      // backward register kernel (rows + prefetch in registers)
// LDS-staged backward: rows past the register kernel's reach (2048 to 4096 vectors) take one row
// per 1024-thread block, 3 or 4 vectors per thread; the stage holds the row's x and dy
// (2 * 4096 * 16 bytes = 128 KiB at most) while registers carry the next row's loads.
constexpr int kBwdLdsMaxIters = 4;
// Streaming backward with its dw sums in registers: up to 8 vectors per thread (8192 vectors a row
// at 1024 threads, e.g. N = 65536 in 16-bit types).
// Register backward pipeline: rows per barrier (batch) and batches in flight ahead of the current
// one, and whether pass 2 reuses xhat and g*dy from pass 1. With the ring's loads issued as
// straight-line code, one batch ahead measured fastest at every depth tried (bf16 4096 x 4096 rows
// kernel: depth 1 19.5 us, 2 20.3, 3 20.8, 5 23.0; no prefetch 21.7): more rows in flight per compute
// unit lower the DRAM efficiency more than they hide latency. Two rows per barrier measured slower
// (24.2 against 22.6 us with the dw reduction).
template <int ITERS> struct BwdPipe;
template <> struct BwdPipe<1> {
  static constexpr int RB = 1, DEPTH = 1;
  static constexpr bool KEEP = true;
};
template <> struct BwdPipe<2> {
  static constexpr int RB = 1, DEPTH = 1;
  static constexpr bool KEEP = false;
};
int bwd_batch(int iters) { return iters == 1 ? BwdPipe<1>::RB : BwdPipe<2>::RB; }

// Automatic selection prefers the register kernel, then the LDS-staged one, then the streaming
// one. Measured (bf16, M = 4096, rows kernel): autograd casts at N = 16384, registers 79 us against
// 123 streaming; whole-vector rows N = 30000, LDS-staged 159 us against 190; rows with a partial
// last vector through a padded stride (N = 24577, 30001, 32767), LDS-staged 137, 171, 193 us
// against 176, 235, 282. The families give bit-identical results, so the choice changes only speed.
// peel_ok: rows not 16-byte aligned whose x and dy rows sit at one offset from a 16-byte boundary
// (streaming kernel, dw sums in LDS); peel_regs_ok: the same with w 16-byte aligned, where at most
// one whole vector per lane (floor(N / V) <= 1024) takes the register kernel for such rows.
rmsnorm_status plan_bwd(int64_t M, int64_t N, rmsnorm_dtype dtype, bool wide_ok, bool ag,
                        rmsnorm_variant req, Plan* p, bool peel_ok = false,
                        bool peel_regs_ok = false, bool narrow_ok = false) {
  const int64_t nv_wide = ceil_div(N, vec_elems(dtype));
  int tpr, iters;
  bwd_shape(nv_wide, &tpr, &iters);
  const int64_t nv_peel = N / vec_elems(dtype);
  const bool peel_regs = !wide_ok && peel_ok && peel_regs_ok && nv_peel <= kBwdBlockThreads;
  const bool reg_ok = (wide_ok && iters <= kBwdRegMaxIters) || peel_regs;
  const bool lds_ok = wide_ok && iters <= kBwdLdsMaxIters;
  rmsnorm_variant v = req;
  if (v == RMSNORM_VARIANT_AUTO) {
    if (reg_ok)
      v = RMSNORM_VARIANT_REGISTERS;
    else if (lds_ok)
      v = RMSNORM_VARIANT_LDS;
    else
      v = RMSNORM_VARIANT_STREAMING;
  }
  if (v == RMSNORM_VARIANT_REGISTERS && !reg_ok) return RMSNORM_ERR_UNSUPPORTED;
  if (v == RMSNORM_VARIANT_LDS && !lds_ok) return RMSNORM_ERR_UNSUPPORTED;
  p->variant = v;
  p->grid = num_partials(M);
  if (v == RMSNORM_VARIANT_STREAMING) {
    p->wide = wide_ok;
    p->peel = !wide_ok && peel_ok;
    const int64_t nv = wide_ok || p->peel ? nv_wide : N;
    bwd_shape(nv, &tpr, &iters);
    p->tpr = tpr;
    p->iters = 0;
    p->groups = 1;
    p->lds = round16(sizeof(float) * 2 * (tpr / 64));
    if (p->peel) p->lds = 128 + sizeof(float) * (size_t)peel_sum_floats(partial_ld(N));
    return RMSNORM_OK;
  }
  if (!wide_ok) {  // registers on peeled rows: one vector per lane, dw sums of each group in LDS
    p->peel = true;
    p->wide = true;
    p->tpr = (int)clamp64(pow2_ceil(nv_peel), 64, kBwdBlockThreads);
    p->iters = 1;
    p->groups = kBwdBlockThreads / p->tpr;
    p->lds = round16(sizeof(float) * 2 * (size_t)p->groups * (p->tpr / 64)) +
             sizeof(float) * (size_t)p->groups * (size_t)peel_sum_floats(partial_ld(N));
    return RMSNORM_OK;
  }
  p->wide = true;
  const int V = vec_elems(dtype);
  if (v == RMSNORM_VARIANT_REGISTERS && narrow_ok && N % V == 0 &&
      (p->sub = narrow_lanes(nv_wide)) > 0) {
    // Narrow rows of whole vectors: 1024 / sub row groups of sub lanes; LDS only for the
    // column combine of the groups' dw sums.
    p->tpr = p->sub;
    p->iters = 1;
    p->groups = kBwdBlockThreads / p->sub;
    p->lds = sizeof(float) * (size_t)combine_columns_floats(V);
    return RMSNORM_OK;
  }
  p->tpr = tpr;
  p->iters = iters;
  p->groups = kBwdBlockThreads / tpr;
  const int wpr = tpr / 64;
  size_t main_bytes;
  if (v == RMSNORM_VARIANT_LDS) {
    main_bytes = round16(sizeof(float) * 2 * (size_t)p->groups * wpr) +
                 (size_t)p->groups * 2 * iters * tpr * 16;
  } else {
    main_bytes = round16(sizeof(float) * 2 * (size_t)p->groups * wpr * bwd_batch(iters));
  }
  // The groups' dw sums: the pairwise tree's slices, or with one vector a lane and four or more
  // groups the column combine's array (combine_block).
  const size_t combine_bytes =
      iters == 1 && p->groups >= 4
          ? sizeof(float) * (size_t)combine_columns_floats(V)
          : sizeof(float) * (size_t)(p->groups / 2) * tpr * iters * V;
  p->lds = main_bytes > combine_bytes ? main_bytes : combine_bytes;
  return RMSNORM_OK;
}


// Register kernels on rows that their threads' vectors tile exactly (N = iters * tpr * V) take the
// FULL instantiation, which has no partial-vector code; the arithmetic is the same.
bool tiles_row(const Plan& p, int64_t N, int V) { return (int64_t)p.iters * p.tpr * V == N; }

template <DT D, Out O>
rmsnorm_status fwd_dispatch(const Plan& p, const FwdArgs& a, hipStream_t s) {
  const int block = p.groups * p.tpr;
  if (p.variant == RMSNORM_VARIANT_STREAMING) {
    if (p.peel) return launch(fwd_peel_kernel<D, O>, p.grid, block, p.lds, s, a);
    return p.wide ? launch(fwd_stream_kernel<D, true, O>, p.grid, block, p.lds, s, a)
                  : launch(fwd_stream_kernel<D, false, O>, p.grid, block, p.lds, s, a);
  }
  const bool lds = p.variant == RMSNORM_VARIANT_LDS;
  const bool full = tiles_row(p, a.N, Elem<D>::VEC);
  if (p.sub > 0) {  // narrow rows: one vector per lane, row groups of p.sub lanes
#define RMSN_FWD_SUB(SB)                                                                        \
  (full ? launch(fwd_rows_kernel<D, 1, O, false, true, SB>, p.grid, block, p.lds, s, a)         \
        : launch(fwd_rows_kernel<D, 1, O, false, false, SB>, p.grid, block, p.lds, s, a))
    switch (p.sub) {
      case 4: return RMSN_FWD_SUB(4);
      case 8: return RMSN_FWD_SUB(8);
      case 16: return RMSN_FWD_SUB(16);
      case 32: return RMSN_FWD_SUB(32);
      default: return RMSNORM_ERR_UNSUPPORTED;
    }
#undef RMSN_FWD_SUB
  }
#define RMSN_FWD_CASE(IT)                                                                   \
  case IT:                                                                                  \
    return lds    ? launch(fwd_rows_kernel<D, IT, O, true>, p.grid, block, p.lds, s, a)     \
           : full ? launch(fwd_rows_kernel<D, IT, O, false, true>, p.grid, block, p.lds, s, a) \
                  : launch(fwd_rows_kernel<D, IT, O, false>, p.grid, block, p.lds, s, a);
  switch (p.iters) {
    RMSN_FWD_CASE(1)
    RMSN_FWD_CASE(2)
    RMSN_FWD_CASE(3)
    RMSN_FWD_CASE(4)
    RMSN_FWD_CASE(5)
    RMSN_FWD_CASE(6)
    RMSN_FWD_CASE(7)
    RMSN_FWD_CASE(8)
    default:
      return RMSNORM_ERR_UNSUPPORTED;
  }
#undef RMSN_FWD_CASE
}

template <DT D, bool AG>
rmsnorm_status bwd_dispatch(const Plan& p, const BwdArgs& a, hipStream_t s) {
  const int block = p.groups * p.tpr;
  if (p.variant == RMSNORM_VARIANT_STREAMING) {
    if (p.peel) return launch(bwd_peel_kernel<D, AG>, p.grid, block, p.lds, s, a);
    // 16-byte rows of at most 8 vectors per thread keep their dw sums in registers. Up to 7 take
    // the 7-vector instantiation (no spill); 8 take the 8-vector one, which spills 5 or 6 registers
    // yet runs 2.5 times faster than sums kept in the workspace (bf16 4096 x 65536: 442 against
    // 1116 us; at 7 vectors, 4096 x 57344, the 7-vector kernel takes 370 us, the 8-vector 389).
    const int64_t per_thread = ceil_div(ceil_div(a.N, Elem<D>::VEC), p.tpr);
    if (p.wide && per_thread <= 7)
      return launch(bwd_stream_kernel<D, true, AG, 7>, p.grid, block, p.lds, s, a);
    if (p.wide && per_thread == 8)
      return launch(bwd_stream_kernel<D, true, AG, 8>, p.grid, block, p.lds, s, a);
    // Other rows (unaligned, or wider) keep the sums in LDS when the row fits there (bf16 4096 x
    // 30001, rows not 16-byte aligned: 564 us with the sums in the workspace).
    if (partial_ld(a.N) <= kStreamLdsAccFloats) {
      const size_t lds = 128 + sizeof(float) * (size_t)partial_ld(a.N);
      return p.wide ? launch(bwd_stream_kernel<D, true, AG, 0, true>, p.grid, block, lds, s, a)
                    : launch(bwd_stream_kernel<D, false, AG, 0, true>, p.grid, block, lds, s, a);
    }
    return p.wide ? launch(bwd_stream_kernel<D, true, AG>, p.grid, block, p.lds, s, a)
                  : launch(bwd_stream_kernel<D, false, AG>, p.grid, block, p.lds, s, a);
  }
  if (p.peel) return launch(bwd_peel_rows_kernel<D, AG>, p.grid, block, p.lds, s, a);
  const bool full = tiles_row(p, a.N, Elem<D>::VEC);
  if (p.variant == RMSNORM_VARIANT_LDS) {
    // Rows of 3 or 4 vectors per thread have 1024 threads (one row group) per block: the kernel
    // takes that as a compile-time constant.
    const Tail ltail = full ? Tail::FULL : (a.N % Elem<D>::VEC == 0 ? Tail::WHOLE : Tail::RAGGED);
#define RMSN_BWD_LDS(IT, TPRC)                                                                     \
  (ltail == Tail::FULL ? launch(bwd_lds_kernel<D, IT, AG, Tail::FULL, TPRC>, p.grid, block, p.lds, \
                                s, a)                                                               \
   : ltail == Tail::WHOLE                                                                           \
       ? launch(bwd_lds_kernel<D, IT, AG, Tail::WHOLE, TPRC>, p.grid, block, p.lds, s, a)         \
       : launch(bwd_lds_kernel<D, IT, AG, Tail::RAGGED, TPRC>, p.grid, block, p.lds, s, a))
    switch (p.iters) {
      case 1: return RMSN_BWD_LDS(1, 0);
      case 2: return RMSN_BWD_LDS(2, 0);
      case 3: return RMSN_BWD_LDS(3, kBwdBlockThreads);
      case 4: return RMSN_BWD_LDS(4, kBwdBlockThreads);
      default: return RMSNORM_ERR_UNSUPPORTED;
    }
#undef RMSN_BWD_LDS
  }
  // Whole 16-byte vectors on every lane (FULL), on the leading lanes (WHOLE), or a partial last
  // vector (RAGGED, rows with a padded stride). FULL and WHOLE rows fix the row group's wave count
  // at compile time (one of 1, 2, 4, 8, 16); RAGGED rows take it from the arguments.
  const Tail tail = full ? Tail::FULL : (a.N % Elem<D>::VEC == 0 ? Tail::WHOLE : Tail::RAGGED);
  const int wpr = p.tpr / 64;
#define RMSN_BWD_ROWS(IT, T, W)                                                            \
  launch(bwd_rows_kernel<D, IT, BwdPipe<IT>::DEPTH, BwdPipe<IT>::RB, AG, BwdPipe<IT>::KEEP, T, \
                         W>,                                                                \
         p.grid, block, p.lds, s, a)
#define RMSN_BWD_WPR(IT, T)                                            \
  (wpr == 1   ? RMSN_BWD_ROWS(IT, T, 1)                                 \
   : wpr == 2 ? RMSN_BWD_ROWS(IT, T, 2)                                 \
   : wpr == 4 ? RMSN_BWD_ROWS(IT, T, 4)                                 \
   : wpr == 8 ? RMSN_BWD_ROWS(IT, T, 8)                                 \
              : RMSN_BWD_ROWS(IT, T, 16))
  if (p.groups * p.tpr != kBwdBlockThreads) return RMSNORM_ERR_UNSUPPORTED;
  if (p.sub > 0) {  // narrow rows of whole vectors, one per lane
#define RMSN_BWD_SUB(T, SB)                                                                  \
  launch(bwd_rows_kernel<D, 1, BwdPipe<1>::DEPTH, BwdPipe<1>::RB, AG, BwdPipe<1>::KEEP, T, 0, \
                         SB>,                                                                 \
         p.grid, block, p.lds, s, a)
#define RMSN_BWD_SUBT(SB) \
  (tail == Tail::FULL ? RMSN_BWD_SUB(Tail::FULL, SB) : RMSN_BWD_SUB(Tail::WHOLE, SB))
    if (tail == Tail::RAGGED) return RMSNORM_ERR_UNSUPPORTED;
    switch (p.sub) {
      case 4: return RMSN_BWD_SUBT(4);
      case 8: return RMSN_BWD_SUBT(8);
      case 16: return RMSN_BWD_SUBT(16);
      case 32: return RMSN_BWD_SUBT(32);
      default: return RMSNORM_ERR_UNSUPPORTED;
    }
#undef RMSN_BWD_SUBT
#undef RMSN_BWD_SUB
  }
  switch (p.iters) {
    case 1:
      return tail == Tail::FULL    ? RMSN_BWD_WPR(1, Tail::FULL)
             : tail == Tail::WHOLE ? RMSN_BWD_WPR(1, Tail::WHOLE)
                                   : RMSN_BWD_ROWS(1, Tail::RAGGED, 0);
    case 2:  // two vectors per thread: row groups of 1024 threads
      return tail == Tail::FULL    ? RMSN_BWD_ROWS(2, Tail::FULL, 16)
             : tail == Tail::WHOLE ? RMSN_BWD_ROWS(2, Tail::WHOLE, 16)
                                   : RMSN_BWD_ROWS(2, Tail::RAGGED, 0);
    default: return RMSNORM_ERR_UNSUPPORTED;
  }
#undef RMSN_BWD_WPR
#undef RMSN_BWD_ROWS
}


template <Out O>
rmsnorm_status fwd_by_dtype(rmsnorm_dtype dtype, const Plan& p, const FwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case RMSNORM_DTYPE_F32:  // the two conventions coincide for float32 I/O
      return fwd_dispatch<DT::F32, O == Out::TWICE ? Out::ONCE : O>(p, a, s);
    case RMSNORM_DTYPE_F16:
      return fwd_dispatch<DT::F16, O>(p, a, s);
    case RMSNORM_DTYPE_BF16:
      return fwd_dispatch<DT::BF16, O>(p, a, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

// Shared by the T-output and 8-bit-output forwards: y holds `yb` bytes per element; its 16-byte
// input vectors map to V * yb output bytes, which the vector store needs aligned. The kernel and
// its summation order depend on x and w alone: a y that does not allow vector stores is written
// one element at a time by the same kernel, so rstd does not depend on where y lives.
rmsnorm_status fwd_impl(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                        float* rstd, int64_t M, int64_t N, rmsnorm_dtype dtype, float eps,
                        float offset, float scale, Out out, rmsnorm_variant variant,
                        void* stream) {
  rmsnorm_status st = check_common(M, N, dtype, eps, offset);
  if (st != RMSNORM_OK) return st;
  if (!variant_ok(variant) || !std::isfinite(scale)) return RMSNORM_ERR_INVALID_ARG;
  const int eb = elem_bytes(dtype);
  const int yb = is_f8(out) ? 1 : eb;
  if ((st = check_matrix(x, ldx, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(y, ldy, M, N, yb)) != RMSNORM_OK) return st;
  if (M > 0 && w == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(w, (uintptr_t)eb) || !aligned(rstd, 4)) return RMSNORM_ERR_MISALIGNED;
  const int yvec = vec_elems(dtype) * yb;  // output bytes per 16-byte input vector
  const bool wide = wide_fits(x, ldx, eb) && aligned(w, 16);
  // Rows that are not 16-byte aligned (or a w that is not) move whole vectors between an
  // element-wise head and tail when a row holds at least two vectors.
  const bool peel_ok = N >= 2 * vec_elems(dtype);
  Plan p;
  if ((st = plan_fwd(M, N, dtype, wide, variant, &p, peel_ok)) != RMSNORM_OK) return st;
  if (M == 0) return RMSNORM_OK;

  FwdArgs a;
  a.x = x; a.w = w; a.y = y; a.rstd = rstd;
  a.ldx = ldx; a.ldy = ldy; a.M = M; a.N = (int)N;
  a.tpr = p.tpr; a.groups = p.groups; a.eps = eps; a.offset = offset; a.scale = scale;
  a.yvec = p.peel ? !is_f8(out) && same_row_phase(x, ldx, y, ldy, eb)
                  : aligned(y, (uintptr_t)yvec) && (ldy * yb) % yvec == 0;
  a.comp = p.variant == RMSNORM_VARIANT_STREAMING &&
           long_chain(N, dtype, p.wide || p.peel, p.tpr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (out) {
    case Out::ONCE: return fwd_by_dtype<Out::ONCE>(dtype, p, a, s);
    case Out::TWICE: return fwd_by_dtype<Out::TWICE>(dtype, p, a, s);
    case Out::E4M3: return fwd_by_dtype<Out::E4M3>(dtype, p, a, s);
    case Out::E5M2: return fwd_by_dtype<Out::E5M2>(dtype, p, a, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

rmsnorm_status fwd_t(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy, float* rstd,
                     int64_t M, int64_t N, rmsnorm_dtype dtype, float eps, float offset,
                     rmsnorm_rounding rounding, rmsnorm_variant variant, void* stream) {
  if (!rounding_ok(rounding)) return RMSNORM_ERR_INVALID_ARG;
  const Out out = rounding == RMSNORM_ROUND_TWICE ? Out::TWICE : Out::ONCE;
  return fwd_impl(x, ldx, w, y, ldy, rstd, M, N, dtype, eps, offset, 1.0f, out, variant, stream);
}

size_t workspace_bytes(int64_t M, int64_t N) {
  return (size_t)num_partials(M) * (size_t)partial_ld(N) * sizeof(float);
}

rmsnorm_status check_bwd_rows(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                              const void* w, const float* rstd, void* dx, int64_t lddx,
                              void* workspace, size_t workspace_bytes_given, int64_t M, int64_t N,
                              int dtype, float offset, int rounding, int variant) {
  rmsnorm_status st = check_common(M, N, dtype, 0.f, offset);
  if (st != RMSNORM_OK) return st;
  if (!variant_ok(variant) || !bwd_rounding_ok(rounding)) return RMSNORM_ERR_INVALID_ARG;
  const int eb = elem_bytes((rmsnorm_dtype)dtype);
  if ((st = check_matrix(dy, lddy, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(x, ldx, M, N, eb)) != RMSNORM_OK) return st;
  if ((st = check_matrix(dx, lddx, M, N, eb)) != RMSNORM_OK) return st;
  if (M > 0 && (w == nullptr || rstd == nullptr || workspace == nullptr))
    return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(w, (uintptr_t)eb) || !aligned(rstd, 4) || !aligned(workspace, 16))
    return RMSNORM_ERR_MISALIGNED;
  if (workspace_bytes_given < workspace_bytes(M, N)) return RMSNORM_ERR_WORKSPACE;
  return RMSNORM_OK;
}

rmsnorm_status bwd_rows_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                             const void* w, const float* rstd, void* dx, int64_t lddx,
                             void* workspace, size_t workspace_bytes_given, int64_t M, int64_t N,
                             rmsnorm_dtype dtype, float offset, int rounding,
                             rmsnorm_variant variant, void* stream) {
  rmsnorm_status st = check_bwd_rows(dy, lddy, x, ldx, w, rstd, dx, lddx, workspace,
                                     workspace_bytes_given, M, N, dtype, offset, rounding, variant);
  if (st != RMSNORM_OK) return st;
  const int eb = elem_bytes(dtype);
  const bool wide = wide_fits(dy, lddy, eb) && wide_fits(x, ldx, eb) && wide_fits(dx, lddx, eb) &&
                    aligned(w, 16);
  // Otherwise x and dy rows at equal offsets from a 16-byte boundary move whole vectors between an
  // element-wise head and tail, with the dw sums in LDS (rows up to kStreamLdsAccFloats wide).
  const bool peel_ok = same_row_phase(x, ldx, dy, lddy, eb) && N >= 2 * vec_elems(dtype) &&
                       peel_sum_floats(partial_ld(N)) <= kStreamLdsAccFloats;
  const bool ag = autograd_casts(rounding, dtype);
  // Narrow rows: the register kernel addresses a wavefront's rows, up to 15 workspace-row counts
  // (num_partials) of strides apart, as 32-bit byte offsets from the first.
  const int64_t ld_max = ldx > lddy ? (ldx > lddx ? ldx : lddx) : (lddy > lddx ? lddy : lddx);
  const bool narrow_ok =
      ((int64_t)(64 / 4 - 1) * num_partials(M) * ld_max + N) * eb <= (int64_t)INT32_MAX;
  Plan p;
  if ((st = plan_bwd(M, N, dtype, wide, ag, variant, &p, peel_ok, aligned(w, 16), narrow_ok)) !=
      RMSNORM_OK)
    return st;
  if (M == 0) return RMSNORM_OK;

  BwdArgs a;
  a.dy = dy; a.x = x; a.w = w; a.rstd = rstd; a.dx = dx;
  a.part = static_cast<float*>(workspace);
  a.lddy = lddy; a.ldx = ldx; a.lddx = lddx; a.M = M;
  a.N = (int)N; a.ldp = (int)partial_ld(N); a.P = (int)num_partials(M);
  a.tpr = p.tpr; a.groups = p.groups; a.offset = offset;
  a.comp = p.variant == RMSNORM_VARIANT_STREAMING &&
           long_chain(N, dtype, p.wide || p.peel, p.tpr);
  a.dxvec = p.peel && same_row_phase(x, ldx, dx, lddx, eb);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case RMSNORM_DTYPE_F32:
      return bwd_dispatch<DT::F32, false>(p, a, s);
    case RMSNORM_DTYPE_F16:
      return ag ? bwd_dispatch<DT::F16, true>(p, a, s) : bwd_dispatch<DT::F16, false>(p, a, s);
    case RMSNORM_DTYPE_BF16:
      return ag ? bwd_dispatch<DT::BF16, true>(p, a, s) : bwd_dispatch<DT::BF16, false>(p, a, s);
  }
  return RMSNORM_ERR_INVALID_ARG;
}

rmsnorm_status dw_reduce_impl(const void* workspace, size_t workspace_bytes_given, float* dw,
                              int64_t M, int64_t N, rmsnorm_dtype dtype, void* stream) {
  rmsnorm_status st = check_common(M, N, dtype, 0.f, 0.f);
  if (st != RMSNORM_OK) return st;
  if (dw == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (M > 0 && workspace == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(dw, 4) || !aligned(workspace, 16)) return RMSNORM_ERR_MISALIGNED;
  if (workspace_bytes_given < workspace_bytes(M, N)) return RMSNORM_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, s, dw,
                       (int)N);
    return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
  }
  launch_dw_reduce(static_cast<const float*>(workspace), partial_ld(N), (int)num_partials(M),
                   (int)N, dw, nullptr, (int64_t)0, 1u, s);
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}

rmsnorm_status bwd_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w,
                        const float* rstd, void* dx, int64_t lddx, float* dw, void* workspace,
                        size_t workspace_bytes_given, int64_t M, int64_t N, rmsnorm_dtype dtype,
                        float eps, float offset, int rounding, rmsnorm_variant variant,
                        void* stream) {
  // Validate everything (both stages) before enqueuing anything.
  rmsnorm_status st = check_common(M, N, dtype, eps, offset);
  if (st != RMSNORM_OK) return st;
  if ((st = check_bwd_rows(dy, lddy, x, ldx, w, rstd, dx, lddx, workspace, workspace_bytes_given,
                           M, N, dtype, offset, rounding, variant)) != RMSNORM_OK)
    return st;
  if (dw == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(dw, 4)) return RMSNORM_ERR_MISALIGNED;

  st = bwd_rows_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, workspace, workspace_bytes_given, M, N,
                     dtype, offset, rounding, variant, stream);
  if (st != RMSNORM_OK) return st;
  return dw_reduce_impl(workspace, workspace_bytes_given, dw, M, N, dtype, stream);
}

// The device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

rmsnorm_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RMSNORM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RMSNORM_ERR_UNSUPPORTED;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr) return RMSNORM_ERR_HIP;
  *out = slot.ptr;
  return RMSNORM_OK;
}

rmsnorm_status bwd_noalloc_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                                const void* w, const float* rstd, void* dx, int64_t lddx,
                                float* dw, int64_t M, int64_t N, rmsnorm_dtype dtype, float eps,
                                float offset, int rounding, void* stream) {
  // Every check before any HIP call: the shape must fit the scratch array, and the arguments
  // pass rmsnorm_bwd's checks with a stand-in workspace of the array's size (any aligned
  // non-null address: nothing is launched on this pass).
  rmsnorm_status st = check_common(M, N, dtype, eps, offset);
  if (st != RMSNORM_OK) return st;
  if (workspace_bytes(M, N) > RMSNORM_NOALLOC_SCRATCH_BYTES) return RMSNORM_ERR_WORKSPACE;
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(256));
  if ((st = check_bwd_rows(dy, lddy, x, ldx, w, rstd, dx, lddx, stand_in,
                           RMSNORM_NOALLOC_SCRATCH_BYTES, M, N, dtype, offset, rounding,
                           RMSNORM_VARIANT_AUTO)) != RMSNORM_OK)
    return st;
  if (dw == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(dw, 4)) return RMSNORM_ERR_MISALIGNED;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != RMSNORM_OK) return st;
  return bwd_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, ws, RMSNORM_NOALLOC_SCRATCH_BYTES, M,
                  N, dtype, eps, offset, rounding, RMSNORM_VARIANT_AUTO, stream);
}

}  // namespace

// ---- exported C interface -------------------------------------------------------------------------
extern "C" {

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_fwd(
    const void* x, int64_t ldx, const void* w, void* y, int64_t ldy, float* rstd, int64_t M,
    int64_t N, rmsnorm_dtype dtype, float eps, float offset, rmsnorm_rounding rounding,
    void* stream) {
  return fwd_t(x, ldx, w, y, ldy, rstd, M, N, dtype, eps, offset, rounding, RMSNORM_VARIANT_AUTO,
               stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_fwd_variant(
    const void* x, int64_t ldx, const void* w, void* y, int64_t ldy, float* rstd, int64_t M,
    int64_t N, rmsnorm_dtype dtype, float eps, float offset, rmsnorm_rounding rounding,
    rmsnorm_variant variant, void* stream) {
  return fwd_t(x, ldx, w, y, ldy, rstd, M, N, dtype, eps, offset, rounding, variant, stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_fwd_fp8(
    const void* x, int64_t ldx, const void* w, void* y, int64_t ldy, float* rstd, int64_t M,
    int64_t N, rmsnorm_dtype dtype, float eps, float offset, float scale,
    rmsnorm_fp8_format format, rmsnorm_variant variant, void* stream) {
  if (format != RMSNORM_FP8_E4M3 && format != RMSNORM_FP8_E5M2) return RMSNORM_ERR_INVALID_ARG;
  const Out out = format == RMSNORM_FP8_E4M3 ? Out::E4M3 : Out::E5M2;
  return fwd_impl(x, ldx, w, y, ldy, rstd, M, N, dtype, eps, offset, scale, out, variant, stream);
}

__attribute__((visibility("default"))) size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N,
                                                                          rmsnorm_dtype dtype) {
  if (!dtype_ok(dtype) || M <= 0 || N < 1 || N > RMSNORM_MAX_N) return 0;
  return workspace_bytes(M, N);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bwd(
    const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, const float* rstd,
    void* dx, int64_t lddx, float* dw, void* workspace, size_t workspace_bytes_given, int64_t M,
    int64_t N, rmsnorm_dtype dtype, float eps, float offset, int rounding, void* stream) {
  return bwd_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, workspace, workspace_bytes_given, M, N,
                  dtype, eps, offset, rounding, RMSNORM_VARIANT_AUTO, stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bwd_variant(
    const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, const float* rstd,
    void* dx, int64_t lddx, float* dw, void* workspace, size_t workspace_bytes_given, int64_t M,
    int64_t N, rmsnorm_dtype dtype, float eps, float offset, int rounding, rmsnorm_variant variant,
    void* stream) {
  return bwd_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, workspace, workspace_bytes_given, M, N,
                  dtype, eps, offset, rounding, variant, stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bwd_noalloc(
    const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, const float* rstd,
    void* dx, int64_t lddx, float* dw, int64_t M, int64_t N, rmsnorm_dtype dtype, float eps,
    float offset, int rounding, void* stream) {
  return bwd_noalloc_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, dw, M, N, dtype, eps, offset,
                          rounding, stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bwd_rows(
    const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* w, const float* rstd,
    void* dx, int64_t lddx, void* workspace, size_t workspace_bytes_given, int64_t M, int64_t N,
    rmsnorm_dtype dtype, float offset, int rounding, rmsnorm_variant variant, void* stream) {
  return bwd_rows_impl(dy, lddy, x, ldx, w, rstd, dx, lddx, workspace, workspace_bytes_given, M, N,
                       dtype, offset, rounding, variant, stream);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bwd_dw_reduce(
    const void* workspace, size_t workspace_bytes_given, float* dw, int64_t M, int64_t N,
    rmsnorm_dtype dtype, void* stream) {
  return dw_reduce_impl(workspace, workspace_bytes_given, dw, M, N, dtype, stream);
}

__attribute__((visibility("default"))) const char* rmsnorm_status_string(rmsnorm_status s) {
  switch (s) {
    case RMSNORM_OK: return "ok";
    case RMSNORM_ERR_INVALID_ARG: return "invalid argument";
    case RMSNORM_ERR_UNSUPPORTED: return "unsupported size or variant";
    case RMSNORM_ERR_MISALIGNED: return "misaligned pointer";
    case RMSNORM_ERR_WORKSPACE: return "workspace too small";
    case RMSNORM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

__attribute__((visibility("default"))) int rmsnorm_abi_version(void) {
  return LIBRMSNORM_ABI_VERSION;
}

}  // extern "C"
