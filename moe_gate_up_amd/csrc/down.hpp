// Down kernel (blog post "warp decode", section "How the two kernels work",
// third and fourth paragraphs): every (token b, output dimension o) is one
// independent output; it walks the token's k routed experts' down rows against
// h[b,j,:], folds each router weight into one FP32 accumulator, and writes
// y[b,o] once, so the weighted top-k combine is part of the projection.
//
// MI355X mapping.  One 64-lane wavefront owns R consecutive output dimensions
// of one token.  The k down rows of one output are treated as one
// concatenated reduction of k*I elements (k*I/32 MX blocks): lane l owns
// blocks l, l+64, ..., each of which lies inside one expert's row, so a lane
// folds (router weight x block scale) into a single multiplier per block.  At
// I=768 a row is 24 blocks and the 192 blocks of 8 experts spread evenly over
// 64 lanes (3 each), which 16-byte loads per lane could not do for a single
// 768-byte row.  h[b] is loaded once per wave and reused for the R outputs.
// Grid order: wave id = tile * B + b (tile slowest) so tokens that share an
// expert read its rows close together in time.
#pragma once

#include "prims.hpp"

namespace moe {

template <int NBL, int R>
__global__ __launch_bounds__(256) void moe_down_3d_batched_w64(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ tw,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd,
    uint16_t* __restrict__ y, int B, int H, int I, int E, int k, int o_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= o_tiles * B) return;
  const int tile = wave / B;
  const int b = wave - tile * B;
  const int o0 = tile * R;
  const int nb_row = I >> 5;          // MX blocks per down row
  const int nb_tot = k * nb_row;      // blocks of the k concatenated rows

  const uint8_t* wrow[NBL];
  const uint8_t* srow[NBL];
  float fold[NBL];
  bool any_bad = false;
  u32x4 ha[NBL][4];
#pragma unroll
  for (int c = 0; c < NBL; ++c) {
    const int q = lane + 64 * c;
    fold[c] = 0.0f;
    wrow[c] = wd;
    srow[c] = sd;
    if (q < nb_tot) {
      const int j = q / nb_row;
      const int qb = q - j * nb_row;
      const int e_raw = ids[b * k + j];
      const bool bad = (unsigned)e_raw >= (unsigned)E;
      any_bad |= bad;
      const size_t row0 = (size_t)(bad ? 0 : e_raw) * H;   // row (e, o=0)
      wrow[c] = wd + row0 * I + qb * 32;
      srow[c] = sd + row0 * nb_row + qb;
      fold[c] = tw[b * k + j];
      const uint16_t* hp = h + (size_t)b * k * I + q * 32;   // h[b] is [k, I] contiguous
#pragma unroll
      for (int t = 0; t < 4; ++t) ha[c][t] = load16(hp + 8 * t);
    }
  }
  const bool bad_token = __builtin_amdgcn_ballot_w64(any_bad) != 0;

  u32x4 w[R][NBL][2];
  uint32_t sc[R][NBL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int o = min(o0 + r, H - 1);   // clamp the ragged last tile; its result is not stored
#pragma unroll
    for (int c = 0; c < NBL; ++c) {
      const int q = lane + 64 * c;
      if (q < nb_tot) {
        const uint8_t* p = wrow[c] + (size_t)o * I;
        w[r][c][0] = load16(p);
        w[r][c][1] = load16(p + 16);
        sc[r][c] = srow[c][(size_t)o * nb_row];
      }
    }
  }

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < NBL; ++c) {
      const int q = lane + 64 * c;
      if (q < nb_tot) {
        const float p = block_dot(w[r][c][0], w[r][c][1], ha[c], 0.0f);
        acc[r] = fmaf(p, fold[c] * e8m0_to_f32(sc[r][c]), acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = wave_sum_row3(acc[r]);

  // lanes 48..63 hold the sums; lane 48 + r writes output o0 + r
  const int r_out = lane - kSumLane;
  float v = acc[0];
#pragma unroll
  for (int r = 1; r < R; ++r) v = (r_out == r) ? acc[r] : v;
  if (r_out >= 0 && r_out < R && o0 + r_out < H)
    y[(size_t)b * H + o0 + r_out] = f32_to_bf16_rne(bad_token ? qnan() : v);
}

}  // namespace moe
