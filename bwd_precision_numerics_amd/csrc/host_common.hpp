// Host-side helpers shared by the library's translation units: argument checks, kernel-shape
// plans, the per-device LDS limit and the launch wrapper. Everything here has internal linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/librmsnorm.h"
#include "rmsnorm_common.hpp"

namespace {

constexpr int kFwdBlockThreads = 256;   // forward rows per block = 256 / threads-per-row
constexpr int kFwdMaxIters = 8;         // 16-byte vectors per thread, forward register kernels

int elem_bytes(rmsnorm_dtype d) {
  return d == RMSNORM_DTYPE_F32 ? 4 : (d == RMSNORM_DTYPE_F64 ? 8 : 2);
}
int vec_elems(rmsnorm_dtype d) { return 16 / elem_bytes(d); }
bool dtype_ok(int d) { return d == RMSNORM_DTYPE_F32 || d == RMSNORM_DTYPE_F16 || d == RMSNORM_DTYPE_BF16; }
bool rounding_ok(int r) { return r == RMSNORM_ROUND_ONCE || r == RMSNORM_ROUND_TWICE; }
// The backward's rounding argument may carry RMSNORM_BWD_AUTOGRAD_CASTS.
bool bwd_rounding_ok(int r) { return rounding_ok(r & ~RMSNORM_BWD_AUTOGRAD_CASTS); }
// The autograd casts only differ from the float32 backward for round twice in a 16-bit type.
bool autograd_casts(int r, int dtype) {
  return (r & RMSNORM_BWD_AUTOGRAD_CASTS) != 0 &&
         (r & ~RMSNORM_BWD_AUTOGRAD_CASTS) == RMSNORM_ROUND_TWICE && dtype != RMSNORM_DTYPE_F32;
}
bool variant_ok(int v) { return v >= RMSNORM_VARIANT_AUTO && v <= RMSNORM_VARIANT_STREAMING; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t pow2_ceil(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}
int64_t clamp64(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The largest element offset a row-strided [M, N] access touches must fit in int64.
bool extent_ok(int64_t M, int64_t N, int64_t ld) {
  if (M <= 1) return true;
  return (M - 1) <= (INT64_MAX - N) / ld;
}

// ---- device LDS limit (queried once per device) ---------------------------------------------------
std::atomic<int> g_lds_limit[64];

rmsnorm_status lds_limit(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RMSNORM_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int cached = g_lds_limit[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return RMSNORM_OK;
    }
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return RMSNORM_ERR_HIP;
  if (dev >= 0 && dev < 64) g_lds_limit[dev].store(v, std::memory_order_relaxed);
  *out = v;
  return RMSNORM_OK;
}

// ---- kernel plans ---------------------------------------------------------------------------------
struct Plan {
  rmsnorm_variant variant;  // resolved (never AUTO)
  bool wide;                // 16-byte vectors
  bool peel = false;        // streaming: rows not 16-byte aligned, whole vectors between an
                            // element-wise head and tail
  int tpr, iters, groups;
  int sub = 0;              // register kernels on narrow rows: row groups of `sub` lanes (4 to 32)
  size_t lds;               // dynamic LDS bytes
  int64_t grid;
};

size_t round16(size_t b) { return (b + 15) & ~size_t(15); }

// Forward: a wavefront per row up to 512 vectors (4096 16-bit elements), wider rows spread over
// more wavefronts with at most 8 vectors per thread.
void fwd_shape(int64_t nv, int* tpr, int* iters) {
  if (nv <= 64 * kFwdMaxIters) {
    *tpr = 64;
  } else {
    *tpr = (int)clamp64(pow2_ceil(ceil_div(nv, kFwdMaxIters)), 64, 1024);
  }
  *iters = (int)ceil_div(nv, *tpr);
}

// Compensated row sums in a streaming kernel: when a thread adds more than kPlainChainVectors
// vectors (or elements) of a row. `wide` says whether the kernel moves 16-byte vectors.
bool long_chain(int64_t N, rmsnorm_dtype dtype, bool wide, int tpr) {
  const int64_t nv = wide ? ceil_div(N, vec_elems(dtype)) : N;
  return ceil_div(nv, tpr) > rmsn::kPlainChainVectors;
}

// Backward: one 16-byte vector per thread up to 1024 vectors a row (8192 16-bit elements); wider
// rows give each thread more vectors (or take a streaming kernel).
void bwd_shape(int64_t nv, int* tpr, int* iters) {
  *tpr = (int)clamp64(pow2_ceil(nv), 64, 1024);
  *iters = (int)ceil_div(nv, *tpr);
}

// Register kernels on rows of at most 32 vectors: row groups of the next power of two (at least
// 4) lanes instead of a whole wavefront, so a wavefront holds 64 / sub rows (bf16 65536 x 128
// forward: one row per wavefront leaves 48 of its 64 lanes idle). 0: a wavefront or more per row.
constexpr int kMaxSubLanes = 32;
int narrow_lanes(int64_t nv) {
  return nv <= kMaxSubLanes ? (int)clamp64(pow2_ceil(nv), 4, kMaxSubLanes) : 0;
}

rmsnorm_status plan_fwd(int64_t M, int64_t N, rmsnorm_dtype dtype, bool wide_ok,
                        rmsnorm_variant req, Plan* p, bool peel_ok = false) {
  const int64_t nv_wide = ceil_div(N, vec_elems(dtype));
  int tpr, iters;
  fwd_shape(nv_wide, &tpr, &iters);
  const bool reg_ok = wide_ok && iters <= kFwdMaxIters;
  rmsnorm_variant v = req;
  if (v == RMSNORM_VARIANT_AUTO) v = reg_ok ? RMSNORM_VARIANT_REGISTERS : RMSNORM_VARIANT_STREAMING;
  if ((v == RMSNORM_VARIANT_REGISTERS || v == RMSNORM_VARIANT_LDS) && !reg_ok)
    return RMSNORM_ERR_UNSUPPORTED;
  p->variant = v;
  if (v == RMSNORM_VARIANT_STREAMING) {
    p->wide = wide_ok;
    p->peel = !wide_ok && peel_ok;
    const int64_t nv = wide_ok || p->peel ? nv_wide : N;
    fwd_shape(nv, &tpr, &iters);
    iters = 0;
  } else {
    p->wide = true;
    if (v == RMSNORM_VARIANT_REGISTERS && (p->sub = narrow_lanes(nv_wide)) > 0) tpr = p->sub;
  }
  p->tpr = tpr;
  p->iters = iters;
  p->groups = tpr >= kFwdBlockThreads ? 1 : kFwdBlockThreads / tpr;
  const int wpr = tpr / 64;
  size_t lds = round16(sizeof(float) * (size_t)p->groups * wpr);
  if (v == RMSNORM_VARIANT_LDS) lds += (size_t)p->groups * iters * tpr * 16;
  p->lds = lds;
  p->grid = ceil_div(M, p->groups);
  if (p->grid > INT32_MAX) return RMSNORM_ERR_UNSUPPORTED;
  return RMSNORM_OK;
}

// ---- launch helpers -------------------------------------------------------------------------------
template <typename Kernel, typename Args>
rmsnorm_status launch(Kernel k, int64_t grid, int block, size_t lds, hipStream_t stream,
                      const Args& args) {
  if (lds > 65536) {
    int limit = 0;
    const rmsnorm_status st = lds_limit(&limit);
    if (st != RMSNORM_OK) return st;
    if (lds > (size_t)limit) return RMSNORM_ERR_UNSUPPORTED;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return RMSNORM_ERR_HIP;
  }
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3((unsigned)block), lds, stream, args);
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}

// ---- validation -----------------------------------------------------------------------------------
rmsnorm_status check_common(int64_t M, int64_t N, int dtype, float eps, float offset) {
  if (!dtype_ok(dtype)) return RMSNORM_ERR_INVALID_ARG;
  if (M < 0 || N < 1) return RMSNORM_ERR_INVALID_ARG;
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(offset)) return RMSNORM_ERR_INVALID_ARG;
  if (N > RMSNORM_MAX_N) return RMSNORM_ERR_UNSUPPORTED;
  return RMSNORM_OK;
}

rmsnorm_status check_matrix(const void* p, int64_t ld, int64_t M, int64_t N, int eb) {
  if (ld < N) return RMSNORM_ERR_INVALID_ARG;
  if (!extent_ok(M, N, ld)) return RMSNORM_ERR_INVALID_ARG;
  if (M > 0 && p == nullptr) return RMSNORM_ERR_INVALID_ARG;
  if (!aligned(p, (uintptr_t)eb)) return RMSNORM_ERR_MISALIGNED;
  return RMSNORM_OK;
}

bool wide_fits(const void* p, int64_t ld, int eb) {
  return aligned(p, 16) && ((ld * eb) % 16 == 0);
}

// Row r of a matrix starts (base + r * ld * eb) bytes in; two matrices have every row at the same
// offset from a 16-byte boundary when their bases and their row strides agree modulo 16 bytes.
bool same_row_phase(const void* a, int64_t lda, const void* b, int64_t ldb, int eb) {
  return ((uintptr_t)a & 15u) == ((uintptr_t)b & 15u) &&
         (((uint64_t)lda * (uint64_t)eb) & 15u) == (((uint64_t)ldb * (uint64_t)eb) & 15u);
}

}  // namespace
