/*
 * librmsnorm — row-wise RMSNorm forward and backward for AMD Instinct MI355X (gfx950).
 *
 * C interface. Every pointer argument is a device pointer owned by the caller; the library
 * allocates nothing, keeps no state between calls and never synchronizes: work is enqueued on the
 * caller's HIP stream and its results are valid once that stream reaches this point. No C++
 * exception crosses this interface and nothing aborts; failures come back as rmsnorm_status.
 *
 * The operation (blog post "Den dolda avrundningen i RMSNorm", precisit.com, section
 * "En välbekant operation"): for each row r of an [M, N] matrix x,
 *
 *     rstd_r = 1 / sqrt( (1/N) * sum_j x_rj^2 + eps )      epsilon under the root
 *     xhat   = x * rstd                                     formed first, in float32
 *     g_j    = offset + w_j                                 offset 0: Llama gain, 1: Gemma gain
 *
 * and the output y is rounded to the I/O type T in one of two ways (same post, section
 * "Två ställen att avrunda"; section "Vilken konvention hör till modellen?" ties the first to
 * Llama and the second to Gemma):
 *
 *     RMSNORM_ROUND_TWICE:  y = T( float(T(xhat)) * g )     the normalized value is cast first
 *     RMSNORM_ROUND_ONCE:   y = T( xhat * g )               one cast, at the store
 *
 * where every product is one float32 multiply and T(.) is round-to-nearest-even. For T = float32
 * the two conventions coincide. Statistics are float32 (sums of float32 values in an order of the
 * library's choosing); the per-row rstd is cached in float32 for the backward, which reads it back
 * instead of recomputing it (Liger-Kernel pull request 92, "feat: correct casts in RMSNorm to match
 * references": the inverse RMS cache and the weight gradient are kept in float32).
 *
 * Backward (the derivative of the composed formula, as in candle pull request 4059, "Add backward
 * passes to the fused rms_norm, layer_norm and softmax_last_dim ops"; inputs upcast to float32 on
 * load and every reduction in float32, as in Liger-Kernel pull request 1608, "fix(group_norm): keep
 * the backward statistics and reductions in fp32"):
 *
 *     xhat = x * rstd,  gdy = g * dy,  c = (1/N) * sum_j gdy_j * xhat_j
 *     dx   = T( rstd * (gdy - xhat * c) )          each operation one float32 operation
 *     dw_j = sum_r dy_rj * xhat_rj                  float32, summed in a fixed order
 *
 * By default the backward is the same for both rounding conventions. With the flag
 * RMSNORM_BWD_AUTOGRAD_CASTS it instead makes the casts of differentiating the round-twice forward
 * computed in T (the Liger pull request says its backward reproduces the references' casts):
 *
 *     gdy  = T(g * dy)                              rounded to T before the reduction and dx
 *     dw_j = sum_r dy_rj * T(xhat_rj)
 *
 * (no effect with RMSNORM_ROUND_ONCE, whose forward works in float32 until the store, or with
 * float32 I/O). dw is produced as per-block float32
 * partial column sums in a caller-provided workspace followed by a second pass that adds the
 * partials in a fixed order: no floating-point atomics, so results are bit-reproducible run to run
 * and independent of the device's compute-unit count.
 *
 * Layout: x, y, dy and dx are row-major [M, N] with unit column stride and a row stride ld* (in
 * elements, ld* >= N; non-contiguous gradients are handled through the row stride). w is [N].
 * x, w, y, dy and dx share one dtype (the comparison in the blog post's footnote 6 assumes weights
 * stored in the input dtype). rstd is float32 [M]; dw is float32 [N]. Outputs must not overlap
 * inputs. The fast paths use 16-byte accesses on 16-byte aligned bases and row strides. Rows that
 * are not 16-byte aligned but sit at one offset from a 16-byte boundary in x and dy (contiguous rows
 * of an odd width, say; N >= 2 * (16 / sizeof(T))) move whole 16-byte vectors between a head and a
 * tail of single elements; any other layout still succeeds through an element-wise path.
 */
#ifndef LIBRMSNORM_H
#define LIBRMSNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIBRMSNORM_ABI_VERSION 4
/* Largest supported row width N. */
#define RMSNORM_MAX_N (1 << 24)

typedef enum rmsnorm_dtype {
  RMSNORM_DTYPE_F32 = 0,
  RMSNORM_DTYPE_F16 = 1,  /* IEEE binary16 */
  RMSNORM_DTYPE_BF16 = 2, /* bfloat16 */
  RMSNORM_DTYPE_F64 = 3   /* IEEE binary64: softmax_* only (the float64 RMSNorm has its own
                             entry points below); elsewhere RMSNORM_ERR_INVALID_ARG */
} rmsnorm_dtype;

typedef enum rmsnorm_rounding {
  RMSNORM_ROUND_ONCE = 0,  /* y = T(xhat * g)                (Gemma convention) */
  RMSNORM_ROUND_TWICE = 1  /* y = T(float(T(xhat)) * g)      (Llama convention) */
} rmsnorm_rounding;

/* Flag bit OR-ed into the backward's `rounding` argument (rmsnorm_bwd, rmsnorm_bwd_variant,
 * rmsnorm_bwd_rows): reproduce the casts of the autograd backward of the round-twice forward (see
 * above). The forward rejects it. */
#define RMSNORM_BWD_AUTOGRAD_CASTS 0x10

/* OCP 8-bit output formats of rmsnorm_fwd_fp8 (1 sign bit, then exponent and significand bits). */
typedef enum rmsnorm_fp8_format {
  RMSNORM_FP8_E4M3 = 0,  /* bias 7, largest finite 448, no infinities: overflow gives NaN */
  RMSNORM_FP8_E5M2 = 1   /* bias 15, largest finite 57344, IEEE-style: overflow gives +-inf */
} rmsnorm_fp8_format;

/* Kernel family. AUTO picks by dtype, N and the row layout, for speed; rstd, y and dx do not
 * depend on the family. The others force one family, for consistency
 * tests and measurements; a forced family that cannot serve the arguments returns
 * RMSNORM_ERR_UNSUPPORTED with nothing launched.
 *   REGISTERS  a row lives in registers between the reduction and the elementwise pass
 *   LDS        a row is staged in LDS between the two passes (same thread-to-element mapping and
 *              summation order as REGISTERS, so results are bit-identical to it)
 *   STREAMING  the elementwise pass reads the row again from memory; serves any N and any
 *              alignment (element-wise accesses when 16-byte accesses are not possible)   */
typedef enum rmsnorm_variant {
  RMSNORM_VARIANT_AUTO = 0,
  RMSNORM_VARIANT_REGISTERS = 1,
  RMSNORM_VARIANT_LDS = 2,
  RMSNORM_VARIANT_STREAMING = 3
} rmsnorm_variant;

typedef enum rmsnorm_status {
  RMSNORM_OK = 0,
  RMSNORM_ERR_INVALID_ARG = 1,  /* null pointer, negative size, ld < N, unknown enum, bad eps */
  RMSNORM_ERR_UNSUPPORTED = 2,  /* N > RMSNORM_MAX_N, or a forced variant that cannot serve */
  RMSNORM_ERR_MISALIGNED = 3,   /* a pointer not aligned to its element size (4 B for float32
                                   buffers, 2 B for 16-bit ones; 16 B for the workspace) */
  RMSNORM_ERR_WORKSPACE = 4,    /* workspace smaller than rmsnorm_bwd_workspace_bytes() */
  RMSNORM_ERR_HIP = 5           /* the HIP runtime reported an error at launch */
} rmsnorm_status;

/* Forward. Computes y [M, N] (dtype) and, when rstd is not NULL, the per-row float32 rstd [M].
 *   x, ldx     input rows, row stride in elements (>= N)
 *   w          gain weights [N], same dtype as x
 *   y, ldy     output rows, row stride in elements (>= N)
 *   rstd       float32 [M] cache for the backward, or NULL to skip writing it
 *   eps        >= 0 and finite; added to the mean of squares under the root
 *   offset     finite; the gain is offset + w (0: Llama, 1: Gemma)
 *   rounding   RMSNORM_ROUND_ONCE or RMSNORM_ROUND_TWICE (no effect for float32)
 *   stream     hipStream_t to enqueue on (NULL = the null stream)
 * M = 0 is a no-op. All argument checks run before any HIP call; on an error nothing is launched. */
rmsnorm_status rmsnorm_fwd(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                           float* rstd, int64_t M, int64_t N, rmsnorm_dtype dtype, float eps,
                           float offset, rmsnorm_rounding rounding, void* stream);

/* rmsnorm_fwd with an explicit kernel family (see rmsnorm_variant). */
rmsnorm_status rmsnorm_fwd_variant(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                                   float* rstd, int64_t M, int64_t N, rmsnorm_dtype dtype,
                                   float eps, float offset, rmsnorm_rounding rounding,
                                   rmsnorm_variant variant, void* stream);

/* Forward with an OCP 8-bit output (blog post "Den dolda avrundningen i RMSNorm", section
 * "Var implementationerna skiljer sig" and its footnote 3: a fused kernel that emits FP8 keeps the
 * normalization, the gain and the per-tensor scale in float32 and casts once at the store):
 *
 *     y8 = FP8( fl(xhat * g) * scale )      one float32 multiply each, then one cast
 *
 * FP8(.) rounds to nearest, ties to even, and does not saturate: a value beyond the format's
 * largest finite one becomes NaN (e4m3) or +-inf (e5m2), the behaviour of a plain conversion.
 * rstd is computed exactly as by rmsnorm_fwd (same summation order: bit-identical values) and is
 * written when not NULL.
 *   x, ldx, w, rstd, M, N, dtype, eps, offset, variant   as for rmsnorm_fwd_variant
 *   y, ldy     output rows, one byte per element; row stride in bytes (= elements), >= N
 *   scale      finite float32 per-tensor scale applied after the gain (1 for none)
 *   format     RMSNORM_FP8_E4M3 or RMSNORM_FP8_E5M2
 * The vector path needs y and ldy aligned to the bytes one 16-byte input vector maps to (8 for
 * 16-bit input, 4 for float32); otherwise the element-wise path serves the call. All argument
 * checks run before any HIP call. */
rmsnorm_status rmsnorm_fwd_fp8(const void* x, int64_t ldx, const void* w, void* y, int64_t ldy,
                               float* rstd, int64_t M, int64_t N, rmsnorm_dtype dtype, float eps,
                               float offset, float scale, rmsnorm_fp8_format format,
                               rmsnorm_variant variant, void* stream);

/* Bytes of device workspace rmsnorm_bwd needs for an [M, N] problem: the float32 partial column
 * sums of dw, one row per block of rows. A pure function of (M, N, dtype): it makes no HIP call
 * and does not depend on the device. Returns 0 for M = 0 and for invalid sizes. */
size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype dtype);

/* Backward. Computes dx [M, N] (dtype) and dw [N] (float32, fully overwritten).
 *   dy, lddy      upstream gradient rows
 *   x, ldx        the forward's input rows
 *   w             gain weights [N]
 *   rstd          float32 [M] written by rmsnorm_fwd for the same x and eps (required, not NULL)
 *   dx, lddx      input-gradient rows
 *   dw            float32 [N] weight gradient (d(offset + w)/dw = 1, so it does not depend on
 *                 offset)
 *   workspace     device buffer of at least rmsnorm_bwd_workspace_bytes(M, N, dtype) bytes,
 *                 16-byte aligned; its contents on entry do not matter and are clobbered
 *   eps           validated for symmetry with the forward; the backward reads rstd instead of
 *                 recomputing it
 *   rounding      RMSNORM_ROUND_ONCE or RMSNORM_ROUND_TWICE, optionally OR-ed with
 *                 RMSNORM_BWD_AUTOGRAD_CASTS; without the flag the result is the same for both
 * M = 0 writes dw = 0. All argument checks run before any HIP call. */
rmsnorm_status rmsnorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                           const void* w, const float* rstd, void* dx, int64_t lddx, float* dw,
                           void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                           rmsnorm_dtype dtype, float eps, float offset, int rounding,
                           void* stream);

/* rmsnorm_bwd with an explicit kernel family. */
rmsnorm_status rmsnorm_bwd_variant(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                                   const void* w, const float* rstd, void* dx, int64_t lddx,
                                   float* dw, void* workspace, size_t workspace_bytes, int64_t M,
                                   int64_t N, rmsnorm_dtype dtype, float eps, float offset,
                                   int rounding, rmsnorm_variant variant, void* stream);

/* The two stages of rmsnorm_bwd, exported so each kernel can be enqueued (and timed) on its own.
 * rmsnorm_bwd_rows writes dx and the per-block dw partials into the workspace;
 * rmsnorm_bwd_dw_reduce adds the partials of the same (M, N, dtype) into dw in a fixed order.
 * rmsnorm_bwd(...) == rmsnorm_bwd_rows(...) followed by rmsnorm_bwd_dw_reduce(...). */
rmsnorm_status rmsnorm_bwd_rows(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                                const void* w, const float* rstd, void* dx, int64_t lddx,
                                void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                                rmsnorm_dtype dtype, float offset, int rounding,
                                rmsnorm_variant variant, void* stream);
rmsnorm_status rmsnorm_bwd_dw_reduce(const void* workspace, size_t workspace_bytes, float* dw,
                                     int64_t M, int64_t N, rmsnorm_dtype dtype, void* stream);

/* rmsnorm_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same kernels and the same results
 * as rmsnorm_bwd (automatic kernel selection), with the dw partial rows in a scratch array the
 * library holds in each device's memory (RMSNORM_NOALLOC_SCRATCH_BYTES, kept until the process
 * ends) instead of a caller workspace. The call itself allocates nothing; its first call on a
 * device looks up that device's copy of the array.
 *   arguments    as for rmsnorm_bwd, without the workspace
 * Errors: RMSNORM_ERR_WORKSPACE (nothing launched) when rmsnorm_bwd_workspace_bytes(M, N, dtype)
 * exceeds RMSNORM_NOALLOC_SCRATCH_BYTES (N up to 8192 for M >= 256 rows); otherwise as for
 * rmsnorm_bwd. Every call on one device shares that device's array: calls that may overlap on one
 * device (different streams, or different host threads without ordering) race and give wrong dw;
 * calls ordered on one stream are safe. */
#define RMSNORM_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
rmsnorm_status rmsnorm_bwd_noalloc(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                                   const void* w, const float* rstd, void* dx, int64_t lddx,
                                   float* dw, int64_t M, int64_t N, rmsnorm_dtype dtype,
                                   float eps, float offset, int rounding, void* stream);

/* ---- float64 -------------------------------------------------------------------------------------
 * RMSNorm with float64 I/O and float64 arithmetic throughout, statistics included (candle pull
 * request 4059: float64 norm kernels take a float64 accumulator, so the forward's statistics equal
 * the ones the backward works with):
 *
 *     rstd = 1 / sqrt(sum_j x_j^2 / N + eps),   y = (x * rstd) * (offset + w)
 *     c = sum_j (offset + w_j) dy_j xhat_j / N,  dx = rstd * ((offset + w) * dy - xhat * c)
 *     dw_j = sum_r dy_rj * xhat_rj
 *
 * Same layout, ownership and error conventions as above; rstd is double [M], dw double [N], eps
 * and offset are doubles. dw is summed without atomics in a fixed order (float64 partial rows in
 * the workspace, then a fixed-order column sum). Rounding conventions do not apply (T = float64).
 * The 16-byte path needs 16-byte aligned bases and row strides; otherwise element-wise. */
rmsnorm_status rmsnorm_fwd_f64(const double* x, int64_t ldx, const double* w, double* y,
                               int64_t ldy, double* rstd, int64_t M, int64_t N, double eps,
                               double offset, void* stream);

/* Bytes of workspace rmsnorm_bwd_f64 needs (float64 partial rows); 0 for M = 0 or bad sizes. */
size_t rmsnorm_bwd_f64_workspace_bytes(int64_t M, int64_t N);

/* rstd (double [M], required) as written by rmsnorm_fwd_f64; dw double [N] fully overwritten
 * (zeros for M = 0); workspace 16-byte aligned, contents clobbered. */
rmsnorm_status rmsnorm_bwd_f64(const double* dy, int64_t lddy, const double* x, int64_t ldx,
                               const double* w, const double* rstd, double* dx, int64_t lddx,
                               double* dw, void* workspace, size_t workspace_bytes, int64_t M,
                               int64_t N, double offset, void* stream);

/* ---- measurement --------------------------------------------------------------------------------
 * HBM bandwidth reference kernels: plain 16-byte streaming patterns with the RMSNorm kernels'
 * non-temporal cache policy, the ceilings the benchmark reports the RMSNorm kernels against (the
 * algorithmic bytes of a pass are those of one of these patterns: the forward moves a copy's, the
 * backward rows a two-read-one-write's). `bytes` is the size of each stream, a multiple of 16;
 * all pointers are 16-byte aligned device memory owned by the caller; one kernel is enqueued on
 * `stream`, nothing is allocated.
 *   RMSNORM_PROBE_READ    reads a; writes rmsnorm_bandwidth_probe_out_bytes(bytes) bytes to c
 *                         (one word per block, so the loads are kept)
 *   RMSNORM_PROBE_WRITE   writes c
 *   RMSNORM_PROBE_COPY    c = a
 *   RMSNORM_PROBE_SUM2    c = a + b (32-bit integer lanes)
 *   RMSNORM_PROBE_LAUNCH  one empty 64-thread block (pointers and bytes ignored): the cost of a
 *                         launch
 * `kind` may be OR-ed with RMSNORM_PROBE_CACHED_STORES: plain stores instead of non-temporal ones.
 * Errors: RMSNORM_ERR_INVALID_ARG (unknown kind, a needed pointer NULL, bytes not a multiple of
 * 16), RMSNORM_ERR_MISALIGNED; all before any HIP call. */
enum {
  RMSNORM_PROBE_READ = 0,
  RMSNORM_PROBE_WRITE = 1,
  RMSNORM_PROBE_COPY = 2,
  RMSNORM_PROBE_SUM2 = 3,
  RMSNORM_PROBE_LAUNCH = 4,
  RMSNORM_PROBE_CACHED_STORES = 0x100
};

size_t rmsnorm_bandwidth_probe_out_bytes(size_t bytes);
rmsnorm_status rmsnorm_bandwidth_probe(int kind, const void* a, const void* b, void* c,
                                       size_t bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* rmsnorm_status_string(rmsnorm_status status);

/* LIBRMSNORM_ABI_VERSION of the built library. */
int rmsnorm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBRMSNORM_H */
