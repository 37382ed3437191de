// HBM bandwidth reference kernels: the ceilings the RMSNorm kernels are measured against.
//
// Four streaming patterns over 16-byte vectors, with the RMSNorm kernels' cache policy
// (non-temporal loads and stores) and nothing else: read only (each block XORs what it reads and
// writes one word, so the loads cannot be dropped), write only, copy (one read and one write
// stream: the forward's traffic) and a two-read-one-write sum (the backward's traffic); plus an
// empty one-block launch, the per-launch floor. Each block moves one tile of 512 threads x U
// vectors per stream, so the grid covers the buffers once. The tile shapes are the fastest of a
// sweep of block sizes, vectors per thread and load/store policies on gfx950: at 32 MiB per stream
// read 2, write 4, copy 4, sum 1 vectors per thread; from 128 MiB on one vector per thread. Plain
// (cached) stores instead of non-temporal ones are a flag: they measured faster on buffers of
// 1 GiB and slower at the RMSNorm sizes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/librmsnorm.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

constexpr int kThreads = 512;

template <int U>
__global__ void __launch_bounds__(kThreads) read_kernel(const u32x4* a, unsigned* out, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    v[u] = i < n ? ld_nt(a + i) : u32x4{0u, 0u, 0u, 0u};
  }
  unsigned x = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  // one word per block: the XOR of its lanes' words
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  __shared__ unsigned part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) x ^= part[w];
    out[blockIdx.x] = x;
  }
}

template <bool NTS>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NTS) st_nt(p, v);
  else *p = v;
}

template <int U, bool NTS>
__global__ void __launch_bounds__(kThreads) write_kernel(u32x4* c, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n) st<NTS>(c + i, u32x4{(unsigned)i, 0x3f800000u, 0u, 0u});
  }
}

__global__ void empty_kernel() {}

template <int U, bool NTS>
__global__ void __launch_bounds__(kThreads) copy_kernel(const u32x4* a, u32x4* c, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n) v[u] = ld_nt(a + i);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n) st<NTS>(c + i, v[u]);
  }
}

template <int U, bool NTS>
__global__ void __launch_bounds__(kThreads) sum2_kernel(const u32x4* a, const u32x4* b, u32x4* c,
                                                        int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * U + threadIdx.x;
  u32x4 va[U], vb[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n) {
      va[u] = ld_nt(a + i);
      vb[u] = ld_nt(b + i);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;
    if (i < n) st<NTS>(c + i, va[u] + vb[u]);
  }
}

// Vectors per thread of each pattern (tiles of 512 threads) below kLargeBytes per stream: read 2,
// write 4, copy 4, sum 1; one each from kLargeBytes on.
constexpr int kReadU = 2, kWriteU = 4, kCopyU = 4, kSumU = 1;
constexpr size_t kLargeBytes = (size_t)128 << 20;

int64_t tiles(int64_t n, int u) { return (n + (int64_t)kThreads * u - 1) / ((int64_t)kThreads * u); }

template <bool NTS>
rmsnorm_status probe_launch(int kind, const u32x4* pa, const u32x4* pb, u32x4* pc, int64_t n,
                            bool large, hipStream_t s) {
  switch (kind) {
    case RMSNORM_PROBE_WRITE:
      if (large) hipLaunchKernelGGL((write_kernel<1, NTS>), dim3((unsigned)tiles(n, 1)),
                                    dim3(kThreads), 0, s, pc, n);
      else hipLaunchKernelGGL((write_kernel<kWriteU, NTS>), dim3((unsigned)tiles(n, kWriteU)),
                              dim3(kThreads), 0, s, pc, n);
      break;
    case RMSNORM_PROBE_COPY:
      if (large) hipLaunchKernelGGL((copy_kernel<1, NTS>), dim3((unsigned)tiles(n, 1)),
                                    dim3(kThreads), 0, s, pa, pc, n);
      else hipLaunchKernelGGL((copy_kernel<kCopyU, NTS>), dim3((unsigned)tiles(n, kCopyU)),
                              dim3(kThreads), 0, s, pa, pc, n);
      break;
    case RMSNORM_PROBE_SUM2:
      hipLaunchKernelGGL((sum2_kernel<kSumU, NTS>), dim3((unsigned)tiles(n, kSumU)),
                         dim3(kThreads), 0, s, pa, pb, pc, n);
      break;
    default:
      return RMSNORM_ERR_INVALID_ARG;
  }
  return RMSNORM_OK;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) size_t rmsnorm_bandwidth_probe_out_bytes(size_t bytes) {
  const int u = bytes >= kLargeBytes ? 1 : kReadU;
  return (size_t)tiles((int64_t)(bytes / 16), u) * sizeof(unsigned);
}

__attribute__((visibility("default"))) rmsnorm_status rmsnorm_bandwidth_probe(
    int kind, const void* a, const void* b, void* c, size_t bytes, void* stream) {
  const bool cached = (kind & RMSNORM_PROBE_CACHED_STORES) != 0;
  kind &= ~RMSNORM_PROBE_CACHED_STORES;
  if (kind < RMSNORM_PROBE_READ || kind > RMSNORM_PROBE_LAUNCH) return RMSNORM_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == RMSNORM_PROBE_LAUNCH) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
    return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
  }
  if (bytes == 0) return RMSNORM_OK;
  if (bytes % 16 != 0) return RMSNORM_ERR_INVALID_ARG;
  const bool need_a = kind != RMSNORM_PROBE_WRITE, need_b = kind == RMSNORM_PROBE_SUM2;
  if ((need_a && !a) || (need_b && !b) || !c) return RMSNORM_ERR_INVALID_ARG;
  const uintptr_t mis = (reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                         reinterpret_cast<uintptr_t>(c)) & 15u;
  if (mis) return RMSNORM_ERR_MISALIGNED;
  const int64_t n = (int64_t)(bytes / 16);
  if (tiles(n, 1) > INT32_MAX) return RMSNORM_ERR_UNSUPPORTED;
  const bool large = bytes >= kLargeBytes;
  const u32x4* pa = static_cast<const u32x4*>(a);
  const u32x4* pb = static_cast<const u32x4*>(b);
  u32x4* pc = static_cast<u32x4*>(c);
  rmsnorm_status st = RMSNORM_OK;
  if (kind == RMSNORM_PROBE_READ) {
    if (large) hipLaunchKernelGGL(read_kernel<1>, dim3((unsigned)tiles(n, 1)), dim3(kThreads), 0,
                                  s, pa, static_cast<unsigned*>(c), n);
    else hipLaunchKernelGGL(read_kernel<kReadU>, dim3((unsigned)tiles(n, kReadU)),
                            dim3(kThreads), 0, s, pa, static_cast<unsigned*>(c), n);
  } else {
    st = cached ? probe_launch<false>(kind, pa, pb, pc, n, large, s)
                : probe_launch<true>(kind, pa, pb, pc, n, large, s);
    if (st != RMSNORM_OK) return st;
  }
  return hipGetLastError() == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_HIP;
}

}  // extern "C"
