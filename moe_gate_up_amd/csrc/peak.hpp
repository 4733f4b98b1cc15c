// Bandwidth probes (blog post "warp decode", section "Hardware efficiency":
// the efficiency figure is a fraction of the peak that a copy kernel reaches
// on contiguous memory).  Grid-stride loops of 16-byte accesses; 512-thread
// workgroups, up to 65536 of them, was the fastest launch shape in a sweep of
// grid sizes, block sizes and unroll depths on MI355X.  Loads and stores
// carry the non-temporal bit, as the layer kernels' weight loads do: on
// MI355X the copy then moves 6.47 TB/s at its best size instead of 6.02, and
// the read probe holds 6.6 TB/s up to 4 GiB instead of falling to 6.2.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kPeakThreads = 512;
constexpr int kPeakMaxBlocks = 65536;

typedef uint32_t peak_v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void copy_peak_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const peak_v4u* s4 = reinterpret_cast<const peak_v4u*>(src);
  peak_v4u* d4 = reinterpret_cast<peak_v4u*>(dst);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s4 + i), d4 + i);
}

__global__ __launch_bounds__(512) void read_peak_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const peak_v4u t = __builtin_nontemporal_load(reinterpret_cast<const peak_v4u*>(src) + i + u * stride);
      a[u].v[0] = t[0]; a[u].v[1] = t[1]; a[u].v[2] = t[2]; a[u].v[3] = t[3];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += a[u].v[0] ^ a[u].v[1] ^ a[u].v[2] ^ a[u].v[3];
  }
  for (; i < n; i += stride) {
    const peak_v4u a = __builtin_nontemporal_load(reinterpret_cast<const peak_v4u*>(src) + i);
    acc += a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  // a value no sum of real data is expected to produce keeps the loads alive
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace moe
