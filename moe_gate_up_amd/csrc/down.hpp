// Down kernel (blog post "warp decode", section "How the two kernels work",
// third and fourth paragraphs): every (token b, output dimension o) is one
// independent output; it walks the token's k routed experts' down rows against
// h[b,j,:], folds each router weight into one FP32 accumulator, and writes
// y[b,o] once, so the weighted top-k combine is part of the projection.
//
// MI355X mapping.  One 64-lane wavefront owns R consecutive output dimensions
// of one token.  The k down rows of one output are treated as one
// concatenated reduction of k*I elements, read in passes of 1024 elements:
// in pass c lane l takes the 16 elements at 1024c + 16l, which lie inside one
// expert's row (rows are multiples of 32 elements), so each lane folds
// (router weight x block scale) into a single multiplier per chunk, and each
// load instruction covers whole cache lines of at most two rows.  At I=768 a
// single row is too short for 64 lanes x 16 bytes; the 6144 concatenated
// elements of 8 experts are 6 passes.  The 4 wavefronts of a workgroup serve
// the same token, so h[b] (2*k*I bytes) is loaded once per workgroup into LDS,
// a quarter by each wavefront, and read back after one barrier; it is reused
// for the R outputs of every wavefront.  Straight-line code with buffer loads
// (scalar base, 32-bit lane offset, scalar row offset); every global load is
// issued before the first arithmetic.
//
// Grid order: tile-major in groups of 4 tiles (wave id = (group, b, tile in
// group)), with workgroups remapped so that each XCD runs a contiguous range
// of groups: tokens that share an expert read its rows at about the same time
// on the same XCD (L2 hits), and a workgroup reads 4*R consecutive rows of
// each of its token's experts.
#pragma once

#include "prims.hpp"

namespace moe {

template <int NP, int R>
__global__ __launch_bounds__(256) void moe_down_3d_batched_w64(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ tw,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd,
    uint16_t* __restrict__ y, int B, int H, int I, int E, int k, int o_tiles) {
  const int lane = threadIdx.x & 63;
  // wave-uniform: keep the index math in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(xcd_contiguous_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6));
  // o_tiles is a multiple of 4 and the grid is exact: no wave leaves before the barrier
  if (wave >= o_tiles * B) return;
  // (H/R is a multiple of 4 because H is a multiple of 32 and R <= 8)
  const int grp = __builtin_amdgcn_readfirstlane(wave / (4 * B));   // VALU division, uniform result
  const int rem = wave - grp * 4 * B;
  const int b = rem >> 2;
  const int tile = grp * 4 + (rem & 3);
  const int o0 = tile * R;
  const int nb_row = I >> 5;          // MX blocks per down row
  const int n_tot = k * I;            // elements of the k concatenated rows

  const uint32_t wbytes = (uint32_t)E * (uint32_t)H * (uint32_t)I;   // < 2^32, checked on the host
  const rsrc_t wr = make_rsrc(wd, wbytes), sr = make_rsrc(sd, wbytes / 32);
  const rsrc_t hr = make_rsrc(h, (uint64_t)B * k * I * 2);
  const rsrc_t idr = make_rsrc(ids, (uint64_t)B * k * 4), twr = make_rsrc(tw, (uint64_t)B * k * 4);

  // h[b] does not depend on the routing: issue its loads first, 16 bytes per
  // thread and piece, workgroup-wide
  constexpr int NLD = (NP + 1) / 2;   // 2*k*I <= NP * 2 KB = NLD pieces of 256 x 16 B
  const uint32_t hbase = (uint32_t)b * (uint32_t)n_tot * 2u;
  u32x4 hv[NLD];
  uint32_t hoff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    hoff[i] = (uint32_t)min(4096 * i + 16 * (int)threadIdx.x, 2 * n_tot - 16);   // clamped: duplicate, same value
    hv[i] = bload16(hr, hoff[i], hbase);
  }
  uint32_t off[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) off[c] = (uint32_t)min(1024 * c + 16 * lane, n_tot - 16);   // clamped duplicates fold with weight 0

  // slot j = off / I of each chunk: its expert, router weight and row offsets.
  // One division for pass 0; later passes step by 1024 = step_j * I + step_w.
  const int step_j = 1024 / I, step_w = 1024 - (1024 / I) * I;
  int j = (16 * lane) / I;
  int within = 16 * lane - j * I;
  uint32_t woff[NP], soff[NP];
  float fold[NP];
  int bias[NP];
  bool any_bad = false;
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    if (c > 0) {
      j += step_j;
      within += step_w;
      if (within >= I) {
        within -= I;
        j += 1;
      }
    }
    const bool live = (1024 * c + 16 * lane) < n_tot;
    if (!live) {   // clamped duplicate of the last chunk
      j = k - 1;
      within = I - 16;
    }
    const uint32_t slot = (uint32_t)(b * k + j);
    const int e_raw = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, slot * 4u, 0, 0));
    const bool bad = (unsigned)e_raw >= (unsigned)E;
    any_bad |= bad;
    const uint32_t row0 = (uint32_t)(bad ? 0 : e_raw) * (uint32_t)H;   // row (e, o=0)
    woff[c] = row0 * (uint32_t)I + (uint32_t)within;
    soff[c] = row0 * (uint32_t)nb_row + (uint32_t)(within >> 5);
    const float wj = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(twr, slot * 4u, 0, 0));
    fold[c] = wj;
    bias[c] = live ? kLiveChunk : kDeadChunk;   // zero the clamped duplicates
  }
  const bool bad_token = __builtin_amdgcn_ballot_w64(any_bad) != 0;

  u32x4 w[R][NP];
  uint32_t sc[R][NP];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t o = (uint32_t)min(o0 + r, H - 1);   // ragged last tile: clamp, not stored
    const uint32_t wo = o * (uint32_t)I, so = o * (uint32_t)nb_row;
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      w[r][c] = bload16<kStream>(wr, woff[c], wo);
      sc[r][c] = bload8<kStream>(sr, soff[c], so);
    }
  }

  // keep every load above this point: all of the wave's memory traffic is in flight at once
  __builtin_amdgcn_sched_barrier(0);
  extern __shared__ __attribute__((aligned(16))) uint8_t hs[];   // h[b], 2*k*I bytes
#pragma unroll
  for (int i = 0; i < NLD; ++i) *reinterpret_cast<u32x4*>(hs + hoff[i]) = hv[i];
  __syncthreads();

  float acc[R];
  uint64_t nan_lanes[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0f;
    nan_lanes[r] = 0;
  }
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const u32x4* hp = reinterpret_cast<const u32x4*>(hs + off[c] * 2u);
    const u32x4 ha[2] = {hp[0], hp[1]};   // this lane's 16 elements of h[b], shared by the R rows
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r] = fmaf(apply_e8m0(chunk_dot(w[r][c], ha, 0.0f), sc[r][c], bias[c]), fold[c], acc[r]);
      nan_lanes[r] |= nan_scale_lanes(sc[r][c]);
    }
  }
  uint64_t nan_rows = 0;   // bit r: an E8M0 NaN code among output r's rows
#pragma unroll
  for (int r = 0; r < R; ++r) nan_rows |= (uint64_t)(nan_lanes[r] != 0) << r;
  // one reduce-scatter of the R sums; output r is written by scatter_lane<R>(r)
  const float tot = wave_reduce_scatter<R>(acc, lane);
  int r_out = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) r_out = (lane == scatter_lane<R>(r)) ? r : r_out;
  if (r_out >= 0 && o0 + r_out < H) {
    const bool nan_out = bad_token || ((nan_rows >> r_out) & 1);
    y[(size_t)b * H + o0 + r_out] = f32_to_bf16_rne(nan_out ? qnan() : tot);
  }
}

}  // namespace moe
