// Host-side pieces shared by the library's translation units.
//
// The two down kernel families are compiled in translation units of their
// own (down_token.hip, down_mfma.hip) because they take different
// instruction-scheduling strategies (build.py): the per-token kernel is
// fastest when the scheduler keeps its loads together in long clauses, the
// matrix-core kernel when it maximises instruction-level parallelism, and
// every other kernel with the default.  Measured on MI355X, graph-timed, the
// down kernel alone: per-token H = 2048, 4 tokens 10.51 vs 10.99 us, H =
// 4096, 1 token 10.61 vs 11.28; matrix-core H = 2048, 32 tokens 32.98 vs
// 33.37, 64 tokens 43.42 vs 43.85.  Either strategy for the whole library
// slows other kernels (the vector-unit grouped gate/up at H = 4096 by 5-8 %).
// moe_decode.hip reaches these kernels only through the functions declared
// here, so each kernel is compiled in exactly one translation unit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#pragma GCC visibility push(hidden)
namespace moe_host {

constexpr int kWavesPerBlock = 4;   // 256 threads = 4 independent 64-lane wavefronts
constexpr int kMaxDownPasses = 16;  // k * I <= 16 passes of 1024 elements = 16384
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kMaxDevices = 64;

// Per-token down kernel, register budget per pass: R weight chunks (4 VGPRs)
// + R scales + h (8 VGPRs).
constexpr bool down_fits(int np, int r) { return np * (5 * r + 8) <= 224; }

// Runs f() once per device, on the first call made with that device current,
// and returns its result on every call.
struct PerDeviceOnce {
  std::once_flag flag[kMaxDevices];
  hipError_t rc[kMaxDevices];
  template <class F>
  hipError_t operator()(F f) {
    int dev = 0;
    hipError_t r = hipGetDevice(&dev);
    if (r != hipSuccess) return r;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(flag[dev], [&] { rc[dev] = f(); });
    return rc[dev];
  }
};

// A down launcher returns its number of workgroups and launches only when
// `go` is set (the plan query calls it with go = false).
using DownLaunch = long long (*)(bool go, hipStream_t, const void* h, const int32_t* ids, const float* tw,
                                 const uint8_t* wd, const uint8_t* sd, void* y, int B, int H, int I, int E, int k);

// down_token.hip: the per-token kernel with np passes over k*I and r output
// dimensions per wavefront; nullptr beyond the register budget.
DownLaunch pick_down(int np, int r);

// down_mfma.hip: the matrix-core grouped kernel for I (<= 2048), and its
// one-time per-device set-up (maximum dynamic LDS of every instantiation).
DownLaunch pick_down_mfma(int I);
hipError_t down_mfma_setup_current_device();

}  // namespace moe_host
#pragma GCC visibility pop
