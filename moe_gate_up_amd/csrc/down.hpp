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
// Straight-line code with buffer loads (scalar base, 32-bit lane offset,
// scalar row offset); every load is issued before the first arithmetic.
// Grid order: wave id = tile * B + b (tile slowest), with workgroups remapped
// so that each XCD runs a contiguous range of tiles: tokens that share an
// expert read its rows at about the same time on the same XCD (L2 hits).
#pragma once

#include "prims.hpp"

namespace moe {

template <int NBL, int R>
__global__ __launch_bounds__(256) void moe_down_3d_batched_w64(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ tw,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd,
    uint16_t* __restrict__ y, int B, int H, int I, int E, int k, int o_tiles) {
  const int lane = threadIdx.x & 63;
  // wave-uniform: keep the index math in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(xcd_contiguous_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6));
  if (wave >= o_tiles * B) return;
  const int tile = __builtin_amdgcn_readfirstlane(wave / B);   // VALU division, uniform result
  const int b = wave - tile * B;
  const int o0 = tile * R;
  const int nb_row = I >> 5;          // MX blocks per down row
  const int nb_tot = k * nb_row;      // blocks of the k concatenated rows

  const uint32_t wbytes = (uint32_t)E * (uint32_t)H * (uint32_t)I;   // < 2^32, checked on the host
  const rsrc_t wr = make_rsrc(wd, wbytes), sr = make_rsrc(sd, wbytes / 32);
  const rsrc_t hr = make_rsrc(h, (uint64_t)B * k * I * 2);
  const rsrc_t idr = make_rsrc(ids, (uint64_t)B * k * 4), twr = make_rsrc(tw, (uint64_t)B * k * 4);

  // lane block q of the concatenated rows: slot j = q / nb_row, block qb within the row.
  // Lanes past the end re-read the last block and fold it with weight 0.
  uint32_t woff[NBL], soff[NBL], hoff[NBL];
  float fold[NBL];
  bool any_bad = false;
#pragma unroll
  for (int c = 0; c < NBL; ++c) {
    const int q_raw = lane + 64 * c;
    const int q = min(q_raw, nb_tot - 1);
    const int j = q / nb_row;
    const int qb = q - j * nb_row;
    const uint32_t slot = (uint32_t)(b * k + j);
    const int e_raw = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, slot * 4u, 0, 0));
    const bool bad = (unsigned)e_raw >= (unsigned)E;
    any_bad |= bad;
    const uint32_t row0 = (uint32_t)(bad ? 0 : e_raw) * (uint32_t)H;   // row (e, o=0)
    woff[c] = row0 * (uint32_t)I + (uint32_t)qb * 32u;
    soff[c] = row0 * (uint32_t)nb_row + (uint32_t)qb;
    hoff[c] = (uint32_t)q * 64u;   // h[b] is [k, I] contiguous: block q = bytes [64q, 64q+64)
    const float wj = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(twr, slot * 4u, 0, 0));
    fold[c] = q_raw < nb_tot ? wj : 0.0f;
  }
  const bool bad_token = __builtin_amdgcn_ballot_w64(any_bad) != 0;

  const uint32_t hbase = (uint32_t)b * (uint32_t)k * (uint32_t)I * 2u;
  u32x4 ha[NBL][4];
#pragma unroll
  for (int c = 0; c < NBL; ++c)
#pragma unroll
    for (int t = 0; t < 4; ++t) ha[c][t] = bload16(hr, hoff[c] + 16u * t, hbase);

  u32x4 w[R][NBL][2];
  uint32_t sc[R][NBL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t o = (uint32_t)min(o0 + r, H - 1);   // ragged last tile: clamp, not stored
    const uint32_t wo = o * (uint32_t)I, so = o * (uint32_t)nb_row;
#pragma unroll
    for (int c = 0; c < NBL; ++c) {
      w[r][c][0] = bload16(wr, woff[c], wo);
      w[r][c][1] = bload16(wr, woff[c] + 16u, wo);
      sc[r][c] = bload8(sr, soff[c], so);
    }
  }

  // keep every load above this point: all of the wave's memory traffic is in flight at once
  __builtin_amdgcn_sched_barrier(0);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0f;
#pragma unroll
    for (int c = 0; c < NBL; ++c) {
      const float p = block_dot(w[r][c][0], w[r][c][1], ha[c], 0.0f);
      acc[r] = fmaf(p, fold[c] * e8m0_to_f32(sc[r][c]), acc[r]);
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
