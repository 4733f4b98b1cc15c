// Gate/up kernel (blog post "warp decode", section "How the two kernels work",
// first two paragraphs): every (token b, routed slot j, neuron n) is one
// independent output; its gate and up rows of expert ids[b,j] are streamed
// once, converted from MXFP8 on the fly, dotted with x[b] in FP32, and
// SiLU(gate) * up is written once as bf16.
//
// MI355X mapping.  One 64-lane wavefront owns R consecutive neurons of one
// (b, j) slot.  Lane l owns the 32-element MX blocks l, l+64, ... of a row, so
// each lane needs exactly one E8M0 scale byte per row and block, and the 64
// lanes together cover 2048 contiguous bytes per row (two 16-byte loads per
// lane per block).  The lane's slice of x[b] is loaded once and reused for the
// R gate rows and R up rows.  All 4*R*NBL weight loads are issued before any
// arithmetic so each wave keeps R*4 KB in flight.  Per-lane partial sums are
// reduced across the wave with DPP row operations, not LDS.
//
// Grid order: wave id = tile * (B*k) + slot, tile (neuron group) slowest, so
// all tokens that share an expert read that expert's rows close together in
// time and the repeats are served from L2 / MALL instead of HBM.
#pragma once

#include "prims.hpp"

namespace moe {

template <int NBL, int R>
__global__ __launch_bounds__(256) void moe_gate_up_3d_batched_w64(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint8_t* __restrict__ su,
    uint16_t* __restrict__ h, int B, int H, int I, int E, int k, int n_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int slots = B * k;
  if (wave >= n_tiles * slots) return;
  const int tile = wave / slots;
  const int s = wave - tile * slots;
  const int b = s / k;
  const int n0 = tile * R;
  const int nblk = H >> 5;
  const int e_raw = __builtin_amdgcn_readfirstlane(ids[s]);
  const bool bad = (unsigned)e_raw >= (unsigned)E;
  const int e = bad ? 0 : e_raw;

  // x[b] slice: block q = lane + 64c covers elements [32q, 32q+32)
  u32x4 xa[NBL][4];
#pragma unroll
  for (int c = 0; c < NBL; ++c) {
    const int q = lane + 64 * c;
    if (q < nblk) {
      const uint16_t* xp = x + (size_t)b * H + q * 32;
#pragma unroll
      for (int t = 0; t < 4; ++t) xa[c][t] = load16(xp + 8 * t);
    }
  }

  u32x4 gw[R][NBL][2], uw[R][NBL][2];
  uint32_t gsc[R][NBL], usc[R][NBL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(n0 + r, I - 1);   // clamp the ragged last tile; its result is not stored
    const size_t row = (size_t)e * I + n;
    const uint8_t* gp = wg + row * H;
    const uint8_t* up = wu + row * H;
    const uint8_t* gs = sg + row * nblk;
    const uint8_t* us = su + row * nblk;
#pragma unroll
    for (int c = 0; c < NBL; ++c) {
      const int q = lane + 64 * c;
      if (q < nblk) {
        gw[r][c][0] = load16(gp + q * 32);
        gw[r][c][1] = load16(gp + q * 32 + 16);
        uw[r][c][0] = load16(up + q * 32);
        uw[r][c][1] = load16(up + q * 32 + 16);
        gsc[r][c] = gs[q];
        usc[r][c] = us[q];
      }
    }
  }

  float g[R], u[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    g[r] = 0.0f;
    u[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < NBL; ++c) {
      const int q = lane + 64 * c;
      if (q < nblk) {
        const float pg = block_dot(gw[r][c][0], gw[r][c][1], xa[c], 0.0f);
        const float pu = block_dot(uw[r][c][0], uw[r][c][1], xa[c], 0.0f);
        g[r] = fmaf(pg, e8m0_to_f32(gsc[r][c]), g[r]);
        u[r] = fmaf(pu, e8m0_to_f32(usc[r][c]), u[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    g[r] = wave_sum_row3(g[r]);
    u[r] = wave_sum_row3(u[r]);
  }

  // lanes 48..63 hold the sums; lane 48 + r writes neuron n0 + r
  const int r_out = lane - kSumLane;
  float gv = g[0], uv = u[0];
#pragma unroll
  for (int r = 1; r < R; ++r) {
    gv = (r_out == r) ? g[r] : gv;
    uv = (r_out == r) ? u[r] : uv;
  }
  if (r_out >= 0 && r_out < R && n0 + r_out < I) {
    const float hv = bad ? qnan() : silu(gv) * uv;
    h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(hv);
  }
}

}  // namespace moe
