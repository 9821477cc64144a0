// HBM reference kernels for the roofline: a pure read stream (the achievable
// read bandwidth the decode kernels are bounded by) and a plain copy of known
// size (to calibrate the memory-traffic counters).  Grid-stride loops with
// 16-byte vector loads, several in flight per lane.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "wg_stamps.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(kThreads) void read_stream(const u32x4 *__restrict__ src, size_t n,
                                                        uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // Keep the loads alive: one word per block, written only if a lane saw a
  // pattern that random data practically never produces.
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// The decode kernels' access pattern without their arithmetic: workgroup w
// reads the w-th contiguous share of the buffer front to back (16-byte
// non-temporal loads, kUnroll in flight per lane), and records its start and
// end clocks and XCD as the stamping build of the decode kernel does.
__global__ __launch_bounds__(kThreads) void read_share(const u32x4 *__restrict__ src, size_t n,
                                                       uint32_t *__restrict__ sink) {
  ATTN_WG_STAMP();
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n ? b0 + per : n;
  size_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * kThreads < b1; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += kThreads) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_stream(uint4 *__restrict__ dst,
                                                        const uint4 *__restrict__ src, size_t n) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from src; sink holds >= blocks words.
// nontemporal != 0 marks the loads as streaming (not kept in the caches).
__attribute__((visibility("default"))) int hbm_read_probe(const void *src, size_t bytes, void *sink, int blocks, int nontemporal,
                   void *stream) {
  if (!src || !sink || bytes % 16 || blocks < 1) return 1;
  if (nontemporal)
    hipLaunchKernelGGL(read_stream<true>, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)src, bytes / 16, (uint32_t *)sink);
  else
    hipLaunchKernelGGL(read_stream<false>, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)src, bytes / 16, (uint32_t *)sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Reads `bytes` (a multiple of 16) from src, one contiguous share per block
// (blocks <= 4096 for the stamps); sink holds >= blocks words.
__attribute__((visibility("default"))) int hbm_read_share_probe(const void *src, size_t bytes,
                                                                void *sink, int blocks,
                                                                void *stream) {
  if (!src || !sink || bytes % 16 || blocks < 1 || blocks > attn::probe::kMaxStampedWgs) return 1;
  hipLaunchKernelGGL(read_share, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4 *)src, bytes / 16, (uint32_t *)sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// Copies `bytes` (a multiple of 16) from src to dst.
__attribute__((visibility("default"))) int hbm_copy_probe(void *dst, const void *src, size_t bytes, int blocks, void *stream) {
  if (!src || !dst || bytes % 16 || blocks < 1) return 1;
  hipLaunchKernelGGL(copy_stream, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (uint4 *)dst, (const uint4 *)src, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
