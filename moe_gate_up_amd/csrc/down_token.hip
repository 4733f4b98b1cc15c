// Launchers of the per-token down kernel (down.hpp), compiled on their own
// with the scheduling strategy that keeps loads in long clauses (host.hpp,
// build.py).
#include <utility>

#include "down.hpp"
#include "host.hpp"

namespace moe_host {
namespace {

// Per-token grid: one wavefront per (tile of R outputs, token), 4 tiles of one
// token per workgroup; dynamic LDS: h[b] of the workgroup's token, 2*k*I <= 32 KB.
template <int NP, int R>
long long launch_down_t(bool go, hipStream_t st, const void* h, const int32_t* ids, const float* tw,
                        const uint8_t* wd, const uint8_t* sd, void* y, int B, int H, int I, int E, int k) {
  const int tiles = (H + R - 1) / R;
  const long long blocks = ((long long)tiles * B + kWavesPerBlock - 1) / kWavesPerBlock;
  if (!go) return blocks;
  hipLaunchKernelGGL((moe::moe_down_3d_batched_w64<NP, R>), dim3((unsigned)blocks), dim3(64 * kWavesPerBlock),
                     (unsigned)(2 * k * I), st, static_cast<const uint16_t*>(h), ids, tw, wd, sd,
                     static_cast<uint16_t*>(y), B, H, I, E, k, tiles);
  return blocks;
}

template <int NP, int R>
DownLaunch down_fn() {
  if constexpr (down_fits(NP, R)) return launch_down_t<NP, R>;
  else return nullptr;
}

template <int NP>
DownLaunch pick_down_r(int r) {
  switch (r) {
    case 1: return down_fn<NP, 1>();
    case 2: return down_fn<NP, 2>();
    case 4: return down_fn<NP, 4>();
    case 8: return down_fn<NP, 8>();
  }
  return nullptr;
}

template <int... NPs>
DownLaunch pick_down_np(int np, int r, std::integer_sequence<int, NPs...>) {
  DownLaunch fn = nullptr;
  ((np == NPs + 1 ? (fn = pick_down_r<NPs + 1>(r), 0) : 0), ...);
  return fn;
}

}  // namespace

DownLaunch pick_down(int np, int r) {
  return pick_down_np(np, r, std::make_integer_sequence<int, kMaxDownPasses>{});
}

}  // namespace moe_host
