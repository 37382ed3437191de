/*
 * libsoftmax — softmax over the last dimension, forward and backward, for AMD Instinct MI355X
 * (gfx950), in the same shared library as librmsnorm.h and with its types and conventions (device
 * pointers owned by the caller, nothing allocated or retained, work enqueued on the caller's HIP
 * stream, all argument checks before any HIP call, rmsnorm_status results).
 *
 * Candle pull request 4059, "Add backward passes to the fused rms_norm, layer_norm and
 * softmax_last_dim ops": the forward computes in float32 for bfloat16 / float16 (and float32) and
 * rounds once at the store; float64 computes in float64. The backward is
 *
 *     dx = T( y * (dy - s) ),   s = sum_j dy_j * y_j
 *
 * from the forward's output y, with s in float32 for the 16-bit types and float32, float64 for
 * float64. The forward, per row: m = max_j x_j, e_j = exp(x_j - m), r = 1 / sum_k e_k,
 * y_j = T(e_j * r) (exp, the one division per row and every product in the compute type; sums in
 * an order of the library's choosing), within a few ulps of the compute type of the exact
 * e_j / sum before the cast.
 *
 * Layout: row-major [M, N], unit column stride, row strides in elements (>= N); dtype is one of
 * RMSNORM_DTYPE_F32, _F16, _BF16, _F64 for all tensors of a call. variant: AUTO, REGISTERS (the
 * row stays in registers; rows up to 8 sixteen-byte vectors per thread (float16 backward: 6)
 * of a 1024-thread group) or STREAMING (any N and alignment); LDS returns RMSNORM_ERR_UNSUPPORTED.
 * Rows take 16-byte accesses when every tensor is 16-byte aligned with row strides a multiple of
 * 16 bytes, or when N >= 2 * (16 / sizeof(T)) and every tensor's rows sit at one offset from a
 * 16-byte boundary (contiguous rows of an odd width, say: whole vectors between a head and a tail
 * of single elements); REGISTERS needs one of the two. Other layouts take element-wise kernels.
 */
#ifndef LIBSOFTMAX_H
#define LIBSOFTMAX_H

#include "librmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* y = softmax(x) over each row. M = 0 is a no-op. */
rmsnorm_status softmax_fwd(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t M, int64_t N,
                           rmsnorm_dtype dtype, rmsnorm_variant variant, void* stream);

/* dx = y * (dy - sum(dy * y)) over each row, from the forward's output y. M = 0 is a no-op. */
rmsnorm_status softmax_bwd(const void* dy, int64_t lddy, const void* y, int64_t ldy, void* dx,
                           int64_t lddx, int64_t M, int64_t N, rmsnorm_dtype dtype,
                           rmsnorm_variant variant, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSOFTMAX_H */
