// Bandwidth probes (blog post "warp decode", section "Hardware efficiency":
// the efficiency figure is a fraction of the peak that a copy kernel reaches
// on contiguous memory).  Grid-stride loops of 16-byte accesses; 512-thread
// workgroups, up to 65536 of them, was the fastest launch shape in a sweep of
// grid sizes, block sizes and unroll depths on MI355X.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kPeakThreads = 512;
constexpr int kPeakMaxBlocks = 65536;

__global__ __launch_bounds__(512) void copy_peak_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(512) void read_peak_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += a[u].v[0] ^ a[u].v[1] ^ a[u].v[2] ^ a[u].v[3];
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    acc += a.v[0] ^ a.v[1] ^ a.v[2] ^ a.v[3];
  }
  // a value no sum of real data is expected to produce keeps the loads alive
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace moe
