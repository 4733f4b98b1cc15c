// Launchers and one-time set-up of the matrix-core grouped down kernel
// (down_grouped_mfma.hpp), compiled on their own with the scheduling strategy
// that maximises instruction-level parallelism (host.hpp, build.py).
#include <utility>

#include "down_grouped_mfma.hpp"
#include "host.hpp"

namespace moe_host {
namespace {

// Largest dynamic LDS of the matrix-core down kernel with NR rounds.
template <int NR>
constexpr int down_mfma_max_lds() { return moe::down_mfma_lds_bytes(NR, moe::kSortMaxExperts, moe::kSortMaxSlots); }
template <int... NRs>
constexpr bool down_mfma_lds_fits(std::integer_sequence<int, NRs...>) {
  return ((down_mfma_max_lds<NRs + 1>() <= kLdsPerCu) && ...);
}
static_assert(down_mfma_lds_fits(std::make_integer_sequence<int, moe::kDownMfmaMaxRounds>{}),
              "the matrix-core down kernel's largest LDS must fit one CU");

// Each instantiation's maximum dynamic LDS is set once per device (the
// largest its limits allow), like the matrix-core gate/up kernel's.
template <int... NRs>
hipError_t down_mfma_set_lds(std::integer_sequence<int, NRs...>) {
  hipError_t rc = hipSuccess;
  ((rc = rc != hipSuccess ? rc
                          : hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::moe_down_grouped_mfma_w64<NRs + 1>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                down_mfma_max_lds<NRs + 1>())),
   ...);
  return rc;
}

PerDeviceOnce g_down_mfma_setup;

// One workgroup per 8 output dimensions; rounds of 256 elements over I (I <= 2048).
template <int NR>
long long launch_down_mfma_t(bool go, hipStream_t st, const void* h, const int32_t* ids, const float* tw,
                             const uint8_t* wd, const uint8_t* sd, void* y, int B, int H, int I, int E, int k) {
  const long long blocks = H / moe::kDownMfmaRows;   // H is a multiple of 32
  if (!go) return blocks;
  hipLaunchKernelGGL((moe::moe_down_grouped_mfma_w64<NR>), dim3((unsigned)blocks), dim3(64 * moe::down_mfma_waves(NR)),
                     (unsigned)moe::down_mfma_lds_bytes(NR, E, B * k), st, static_cast<const uint16_t*>(h), ids, tw, wd, sd,
                     static_cast<uint16_t*>(y), B, H, I, E, k);
  return blocks;
}

template <int... NRs>
DownLaunch pick_down_mfma_nr(int nr, std::integer_sequence<int, NRs...>) {
  DownLaunch fn = nullptr;
  ((nr == NRs + 1 ? (fn = launch_down_mfma_t<NRs + 1>, 0) : 0), ...);
  return fn;
}

}  // namespace

hipError_t down_mfma_setup_current_device() {
  return g_down_mfma_setup(
      [] { return down_mfma_set_lds(std::make_integer_sequence<int, moe::kDownMfmaMaxRounds>{}); });
}

DownLaunch pick_down_mfma(int I) {
  return pick_down_mfma_nr((I + 255) / 256, std::make_integer_sequence<int, moe::kDownMfmaMaxRounds>{});
}

}  // namespace moe_host
