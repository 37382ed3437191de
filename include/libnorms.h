/*
 * libnorms — LayerNorm and GroupNorm forward and backward for AMD Instinct MI355X (gfx950), built
 * into the same shared library as librmsnorm.h and sharing its types (rmsnorm_dtype,
 * rmsnorm_variant, rmsnorm_status) and conventions: every pointer is a device pointer owned by the
 * caller, nothing is allocated or retained, work is enqueued on the caller's HIP stream (`stream`
 * is a hipStream_t, NULL for the null stream), every argument check runs before any HIP call, and
 * failures come back as rmsnorm_status with nothing launched.
 *
 * Statistics are float32 for every I/O type and cached in float32 for the backward (Liger-Kernel
 * pull request 1608, "fix(group_norm): keep the backward statistics and reductions in fp32":
 * Mean and RSTD stored in float32 as layer_norm already did; the backward upcasts W, X and the
 * upstream gradient on load and reduces in float32). The backward is the derivative of the
 * composed formula with float32 statistics (candle pull request 4059, "Add backward passes to the
 * fused rms_norm, layer_norm and softmax_last_dim ops").
 *
 * LayerNorm, for each row r of an [M, N] matrix (each step one float32 operation, T(.) the
 * round-to-nearest-even cast to the I/O type at the store):
 *
 *     mean = (sum_j x_j) / N                 var = (sum_j (x_j - mean)^2) / N   (about the mean)
 *     rstd = 1 / sqrt(var + eps)             y   = T( ((x - mean) * rstd) * w + b )
 *
 * Backward, from the cached float32 mean and rstd:
 *
 *     xhat = (x - mean) * rstd     gdy = w * dy     c1 = (sum_j gdy_j) / N
 *     c2   = (sum_j gdy_j * xhat_j) / N             dx = T( rstd * ((gdy - c1) - xhat * c2) )
 *     dw_j = sum_r dy_rj * xhat_rj                  db_j = sum_r dy_rj          (float32)
 *
 * Row sums are float32 in an order of the library's choosing; dw and db are summed without atomics
 * in a fixed order (per-block partial rows in the workspace, then a fixed-order reduction), so
 * results are bit-reproducible and independent of the device.
 *
 * Layout as in librmsnorm.h: x, y, dy, dx row-major [M, N] with unit column stride and row strides
 * ld* in elements; w and b are [N] in the I/O dtype; mean, rstd are float32 [M]; dw, db float32
 * [N]. Outputs must not overlap inputs.
 */
#ifndef LIBNORMS_H
#define LIBNORMS_H

#include "librmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* LayerNorm forward. Computes y [M, N] and, when not NULL, the float32 mean [M] and rstd [M].
 *   x, ldx      input rows, row stride in elements (>= N)
 *   w           weight [N], same dtype as x (required)
 *   b           bias [N], same dtype as x, or NULL for no bias
 *   y, ldy      output rows
 *   mean, rstd  float32 [M] caches for the backward, each may be NULL to skip writing it
 *   eps         >= 0 and finite; added to the variance under the root
 *   variant     AUTO, REGISTERS or STREAMING (LDS returns RMSNORM_ERR_UNSUPPORTED)
 * M = 0 is a no-op. 16-byte accesses need x, w and b 16-byte aligned and ldx * sizeof(T) a
 * multiple of 16; otherwise, for N >= 2 * (16 / sizeof(T)), whole 16-byte vectors of x between a
 * head and a tail of single elements (y as vectors when its rows sit at x's offsets from a 16-byte
 * boundary), else an element-wise kernel. */
rmsnorm_status layernorm_fwd(const void* x, int64_t ldx, const void* w, const void* b, void* y,
                             int64_t ldy, float* mean, float* rstd, int64_t M, int64_t N,
                             rmsnorm_dtype dtype, float eps, rmsnorm_variant variant,
                             void* stream);

/* Bytes of device workspace layernorm_bwd needs: two float32 partial rows (dw, db) per block of
 * rows. A pure function of (M, N, dtype); 0 for M = 0 and for invalid sizes. */
size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype dtype);

/* LayerNorm backward. Computes dx [M, N] (dtype), dw [N] (float32) and, when db is not NULL,
 * db [N] (float32); dw and db are fully overwritten (zeros for M = 0).
 *   dy, lddy     upstream gradient rows
 *   x, ldx       the forward's input rows
 *   w            weight [N]
 *   mean, rstd   float32 [M] written by layernorm_fwd for the same x and eps (required)
 *   dx, lddx     input-gradient rows
 *   dw           float32 [N] weight gradient (required)
 *   db           float32 [N] bias gradient, or NULL to skip it
 *   workspace    at least layernorm_bwd_workspace_bytes(M, N, dtype) bytes, 16-byte aligned;
 *                contents on entry do not matter and are clobbered
 *   variant      AUTO, REGISTERS or STREAMING (LDS returns RMSNORM_ERR_UNSUPPORTED)
 * 16-byte accesses need dy, x and dx 16-byte aligned with row strides a multiple of 16 bytes and w
 * 16-byte aligned; rows that are not but whose x and dy rows sit at one offset from a 16-byte
 * boundary, with w 16-byte aligned and N / (16 / sizeof(T)) <= 1024, take whole vectors between a
 * head and a tail of single elements (REGISTERS); anything else the element-wise kernel. */
rmsnorm_status layernorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                             const void* w, const float* mean, const float* rstd, void* dx,
                             int64_t lddx, float* dw, float* db, void* workspace,
                             size_t workspace_bytes, int64_t M, int64_t N, rmsnorm_dtype dtype,
                             rmsnorm_variant variant, void* stream);

/* ---- GroupNorm ----------------------------------------------------------------------------------
 * x is [B, C, S] contiguous (S the flattened spatial size, row-major: element (b, c, s) at
 * (b * C + c) * S + s); C is split into G groups of Cg = C / G adjacent channels, and each
 * (batch, group) row of Cg * S elements is normalized with its own float32 mean and rstd; the
 * weight w [C] and bias b [C] (I/O dtype) are per channel:
 *
 *     y    = T( ((x - mean) * rstd) * w_c + b_c )
 *     dx   = T( rstd * ((w_c * dy - c1) - xhat * c2) ),  c1 = sum(w_c dy) / n, c2 = sum(w_c dy xhat) / n
 *     dW_c = sum over batch and space of dy * xhat,      dB_c = sum over batch and space of dy
 *
 * sums over the n = Cg * S elements of a row, in float32 (Liger-Kernel pull request 1608). The
 * work is split into chunks of one (batch, channel) segment (at most 8192 elements for 16-bit types,
 * 4096 for float32); per-chunk statistics and sums go to a caller-provided float32 workspace and are
 * combined in a fixed order, so results are bit-reproducible and no atomics are used. Rows whose S
 * fits one chunk are instead held whole by one group of threads (statistics from one read of x; in
 * the backward each segment's sums go to the same workspace pairs, one per segment) when they have
 * at most 32768 elements (16384 for float32) with 16-byte accesses and S a multiple of the
 * 16-byte vector, else at most 16384 (8192), and the backward's 2 * (m + Cg) + 128 floats of LDS
 * (m = n / vector or n staged values) fit 144 KiB. Group sizes up to RMSNORM_MAX_N elements are
 * supported. S * sizeof(T) (rows held whole: Cg * S * sizeof(T)) a multiple of 16 with
 * 16-byte-aligned tensors gives 16-byte accesses; anything else takes element-wise kernels. mean
 * and rstd are float32 [B, G]. */

/* Bytes of workspace groupnorm_fwd and groupnorm_bwd need (the same for both): 8 bytes per chunk.
 * A pure function of the shape and dtype; 0 for invalid shapes. */
size_t groupnorm_workspace_bytes(int64_t B, int64_t C, int64_t S, int64_t G, rmsnorm_dtype dtype);

/* GroupNorm forward. y [B, C, S]; mean, rstd [B, G] written when not NULL (the backward needs
 * them). w [C] required, b [C] or NULL for no bias. eps >= 0 and finite. B = 0 is a no-op.
 * C % G != 0, or a non-positive C, S or G, returns RMSNORM_ERR_INVALID_ARG. */
rmsnorm_status groupnorm_fwd(const void* x, const void* w, const void* b, void* y, float* mean,
                             float* rstd, void* workspace, size_t workspace_bytes, int64_t B,
                             int64_t C, int64_t S, int64_t G, rmsnorm_dtype dtype, float eps,
                             void* stream);

/* GroupNorm backward from the forward's mean and rstd. dx [B, C, S] (dtype); dw [C] float32
 * (required), db [C] float32 or NULL; both fully overwritten (zeros for B = 0). The workspace
 * contents on entry do not matter and are clobbered. */
rmsnorm_status groupnorm_bwd(const void* dy, const void* x, const void* w, const float* mean,
                             const float* rstd, void* dx, float* dw, float* db, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t C, int64_t S, int64_t G,
                             rmsnorm_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBNORMS_H */
