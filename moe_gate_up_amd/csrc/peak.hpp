// Bandwidth probes (blog post "warp decode", section "Hardware efficiency":
// the efficiency figure is a fraction of the peak that a copy kernel reaches
// on contiguous memory).  Grid-stride loops of 16-byte accesses, four in
// flight per lane per iteration.
#pragma once

#include "prims.hpp"

namespace moe {

__global__ __launch_bounds__(256) void copy_peak_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a; dst[i + stride] = b; dst[i + 2 * stride] = c; dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_peak_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc += a.v[t] ^ b.v[t] ^ c.v[t] ^ d.v[t];
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    acc += a.v[0] ^ a.v[1] ^ a.v[2] ^ a.v[3];
  }
  // a value no sum of real data is expected to produce keeps the loads alive
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace moe
