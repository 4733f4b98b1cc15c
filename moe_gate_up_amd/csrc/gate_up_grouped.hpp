// Gate/up kernel, expert-grouped variant (blog post "warp decode", section
// "How the two kernels work" for the arithmetic; section "Warp decode and
// Composer training" for why grouping pays once several tokens share an
// expert).  Each output h[b,j,n] is still computed by one wavefront from the
// streamed gate and up rows, with no padding, gather buffer or combine: the
// only change is that one wavefront owns R neurons of one expert e for every
// slot routed to e, so the rows are read from memory and converted from MXFP8
// once, then dotted with each of those tokens' activations in turn.
//
// The wavefront first scans topk_ids (B*k <= 1024 entries, 64 per ballot) for
// the slots that use e and exits before loading anything if there are none.
// The R gate and R up rows are loaded with the same 1 KB-contiguous passes as
// the per-slot kernel and converted to bf16 pairs in registers.  Then, slot
// by slot, the lane's slice of x[b] is loaded, the 2R dot products are
// formed with v_dot2c_f32_bf16, each 16-element partial is scaled by its
// E8M0 scale (v_ldexp_f32), the 2R sums are reduced with DPP and lanes
// 48..48+R-1 write SiLU(g)*u.
//
// Measured on MI355X this variant is slower than the per-slot kernel at
// every batch size swept (B = 1..64, H = 2048 and 4096): each token adds a
// dependent activation load to the wavefront's critical path, x is re-read
// per (expert, tile, token), and holding converted rows limits occupancy,
// which outweighs converting each row once.  (Fetching four tokens'
// activations per round was slower still.)  It is kept as an opt-in variant.  The wavefront for expert 0 of each tile also
// writes NaN for slots whose id is outside [0, E), so every output is written
// exactly once.
//
// Grid order: wave id = tile * E + e (tile slowest), workgroups remapped so
// each XCD runs a contiguous range of tiles.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kGroupedMaxSlots = 1024;   // B*k limit of the expert-grouped variant

template <int NCH, int R>
__global__ __launch_bounds__(256) void moe_gate_up_expert_grouped_w64(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint8_t* __restrict__ su,
    uint16_t* __restrict__ h, int B, int H, int I, int E, int k, int n_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(xcd_contiguous_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6));
  if (wave >= n_tiles * E) return;
  const int tile = __builtin_amdgcn_readfirstlane(wave / E);   // VALU division, uniform result
  const int e = wave - tile * E;
  const int n0 = tile * R;
  const int slots = B * k;
  const int nq = (slots + 63) / 64;
  const int nblk = H >> 5;

  // ---- which slots use expert e (and, for e == 0, whether any id is invalid)
  const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);
  // expert id of slot 64q + lane; slots past B*k read as E (matches no expert);
  // an invalid id of a real slot reads as -1
  auto slot_id = [&](int q) {
    const int sl = 64 * q + lane;
    const int v = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)min(sl, slots - 1) * 4u, 0, 0));
    return sl < slots ? ((unsigned)v >= (unsigned)E ? -1 : v) : E;
  };
  int count = 0;
  bool any_bad = false;
  for (int q = 0; q < nq; ++q) {
    const int v = slot_id(q);
    count += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v == e));
    any_bad |= __builtin_amdgcn_ballot_w64(v == -1) != 0;
  }
  const bool nan_duty = e == 0 && any_bad;
  if (count == 0 && !nan_duty) return;

  // ---- load and convert the expert's R gate and R up rows
  uint32_t off[NCH];
  int bias[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int o = 1024 * c + 16 * lane;
    off[c] = (uint32_t)min(o, H - 16);
    bias[c] = o < H ? kLiveChunk : kDeadChunk;
  }
  const uint32_t wbytes = (uint32_t)E * (uint32_t)I * (uint32_t)H;   // < 2^32, checked on the host
  const rsrc_t xr = make_rsrc(x, (uint64_t)B * H * 2);
  const rsrc_t gr = make_rsrc(wg, wbytes), ur = make_rsrc(wu, wbytes);
  const rsrc_t gsr = make_rsrc(sg, wbytes / 32), usr = make_rsrc(su, wbytes / 32);

  u32x4 gw[R][NCH], uw[R][NCH];
  uint32_t gsc[R][NCH], usc[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)(e * I + min(n0 + r, I - 1));   // ragged last tile: clamp, not stored
    const uint32_t woff = row * (uint32_t)H, soff = row * (uint32_t)nblk;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      gw[r][c] = bload16(gr, off[c], woff);
      uw[r][c] = bload16(ur, off[c], woff);
      gsc[r][c] = bload8(gsr, off[c] >> 5, soff);
      usc[r][c] = bload8(usr, off[c] >> 5, soff);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // bf16 pairs of the rows: [r][c][8 dwords]
  uint32_t gb[R][NCH][8], ub[R][NCH][8];
  uint64_t nan_rows = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    uint64_t nan_lanes = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        gb[r][c][2 * d] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2(gw[r][c].v[d], false));
        gb[r][c][2 * d + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2(gw[r][c].v[d], true));
        ub[r][c][2 * d] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2(uw[r][c].v[d], false));
        ub[r][c][2 * d + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2(uw[r][c].v[d], true));
      }
      nan_lanes |= nan_scale_lanes(gsc[r][c]) | nan_scale_lanes(usc[r][c]);
    }
    nan_rows |= (uint64_t)(nan_lanes != 0) << r;
  }

  const int r_out = lane - kSumLane;
  const bool writer = r_out >= 0 && r_out < R && n0 + r_out < I;

  // ---- every slot routed to e, one at a time
  for (int q = 0; q < nq; ++q) {
    uint64_t m = __builtin_amdgcn_ballot_w64(slot_id(q) == e);
    while (m) {
      const int s = 64 * q + __builtin_ctzll(m);
      m &= m - 1;
      const int b = __builtin_amdgcn_readfirstlane(s / k);
      const uint32_t xoff = (uint32_t)b * (uint32_t)H * 2u;
      u32x4 xa[NCH][2];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        xa[c][0] = bload16(xr, off[c] * 2u, xoff);
        xa[c][1] = bload16(xr, off[c] * 2u + 16u, xoff);
      }
      float g[R], u[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        g[r] = 0.0f;
        u[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          float pg = 0.0f, pu = 0.0f;
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            const bf16x2_t xv = as_bf16x2(xa[c][d >> 2].v[d & 3]);
            pg = dot2(as_bf16x2(gb[r][c][d]), xv, pg);
            pu = dot2(as_bf16x2(ub[r][c][d]), xv, pu);
          }
          g[r] += apply_e8m0(pg, gsc[r][c], bias[c]);
          u[r] += apply_e8m0(pu, usc[r][c], bias[c]);
        }
        g[r] = wave_sum_row3(g[r]);
        u[r] = wave_sum_row3(u[r]);
      }
      float gv = g[0], uv = u[0];
#pragma unroll
      for (int r = 1; r < R; ++r) {
        gv = (r_out == r) ? g[r] : gv;
        uv = (r_out == r) ? u[r] : uv;
      }
      if (writer) {
        const bool nan_out = (nan_rows >> r_out) & 1;
        h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(nan_out ? qnan() : silu(gv) * uv);
      }
    }
  }

  // ---- slots with an invalid expert id: written as NaN by expert 0's wavefront
  if (nan_duty) {
    for (int q = 0; q < nq; ++q) {
      uint64_t m = __builtin_amdgcn_ballot_w64(slot_id(q) == -1);
      while (m) {
        const int bit = __builtin_ctzll(m);
        m &= m - 1;
        const int s = 64 * q + bit;
        if (writer) h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(qnan());
      }
    }
  }
}

}  // namespace moe
