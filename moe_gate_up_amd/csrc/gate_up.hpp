// Gate/up kernel (blog post "warp decode", section "How the two kernels work",
// first two paragraphs): every (token b, routed slot j, neuron n) is one
// independent output; its gate and up rows of expert ids[b,j] are streamed
// once, converted from MXFP8 on the fly, dotted with x[b] in FP32, and
// SiLU(gate) * up is written once as bf16.
//
// MI355X mapping.  One 64-lane wavefront owns R consecutive neurons of one
// (b, j) slot.  A row is read in passes of 1024 contiguous bytes: in pass c
// lane l loads the 16 bytes at 1024c + 16l, so every load instruction of the
// wave covers eight whole 128-byte cache lines (the contiguous access the
// pages' copy-kernel peak is measured with).  Two neighbouring lanes share
// the E8M0 scale of their 32-element block.  The lane's slice of x[b] is
// loaded once and reused for the R gate rows and R up rows.  When k is a
// multiple of 4 (XL), the 4 wavefronts of a workgroup are 4 slots of the same
// token: each loads a quarter of x[b] into LDS and all four read it back
// after one barrier, which takes 3/4 of the activation loads off the vector
// memory pipeline that the weight stream needs.  The code is
// straight-line: every load of the wave is issued before the first
// arithmetic, so each wave keeps R*4 KB in flight; lanes past the end of a
// row re-read its last chunk and contribute zero.  Loads are buffer loads:
// scalar base, 32-bit lane offset, scalar row offset.  The 2R per-lane
// partial sums are reduced in one reduce-scatter (permlane swaps across rows,
// DPP inside rows), not through LDS.
//
// Grid order: wave id = tile * (B*k) + slot, tile (neuron group) slowest, and
// workgroups are remapped so that each XCD runs a contiguous range of tiles.
// All tokens that share an expert then read that expert's rows at about the
// same time on the same XCD, and the repeats hit that XCD's L2.
//
// ROUTE (E <= 128): the router step is the kernel's prologue.  The
// workgroup reads its token's E logits instead of ids, selects the token's
// top k itself (the same selection as the router kernel: once per workgroup
// when its 4 wavefronts share the token, else once per wavefront) and takes
// selection j for slot j; the first neuron tile also stores the ids and the
// routing weights for the down kernel.  The x loads are issued before the
// selection, so they are in flight while it runs.
#pragma once

#include "prims.hpp"
#include "router.hpp"

namespace moe {

template <int NCH, int R, bool XL, bool ROUTE>
__global__ __launch_bounds__(256) void moe_gate_up_3d_batched_w64(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint8_t* __restrict__ su,
    uint16_t* __restrict__ h, int B, int H, int I, int E, int k, int n_tiles,
    const float* __restrict__ logits, int32_t* __restrict__ ids_out, float* __restrict__ tw_out) {
  const int lane = threadIdx.x & 63;
  // wave-uniform: keep the index math in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(xcd_contiguous_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6));
  const int slots = B * k;
  // With XL the grid is exact (B*k and so n_tiles*B*k are multiples of 4), so
  // no wave of a workgroup leaves before the barrier.
  if (wave >= n_tiles * slots) return;
  // integer division runs on the VALU; readfirstlane returns the (uniform) results to SGPRs
  const int tile = __builtin_amdgcn_readfirstlane(wave / slots);
  const int s = wave - tile * slots;
  const int b = __builtin_amdgcn_readfirstlane(s / k);
  const int n0 = tile * R;
  const int nblk = H >> 5;
  int e_raw = 0;
  if constexpr (!ROUTE) e_raw = __builtin_amdgcn_readfirstlane(ids[s]);

  // element offset of this lane's 16-element chunk in pass c, clamped to the
  // row; the scale bias zeroes the clamped duplicates
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

  const uint32_t xoff = (uint32_t)b * (uint32_t)H * 2u;
  u32x4 xa[NCH][2];
  constexpr int NX = (NCH + 1) / 2;   // XL: 16-byte pieces of x[b] per thread (256 threads x 16 B per piece)
  u32x4 xv[NX];
  uint32_t xo[NX];
  if constexpr (XL) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      xo[i] = (uint32_t)min(4096 * i + 16 * (int)threadIdx.x, 2 * H - 16);   // clamped: duplicate, same value
      xv[i] = bload16(xr, xo[i], xoff);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      xa[c][0] = bload16(xr, off[c] * 2u, xoff);
      xa[c][1] = bload16(xr, off[c] * 2u + 16u, xoff);
    }
  }

  if constexpr (ROUTE) {
    constexpr int NV = route_per_lane(kRouteFusedMaxExperts);
    const int w_in = threadIdx.x >> 6;
    // XL: the workgroup's 4 slots j0 .. j0+3 share the token; wavefront 0
    // selects once and hands the experts over through LDS.  Else every
    // wavefront selects for its own slot.
    const int s0 = XL ? s - w_in : s, nsl = XL ? 4 : 1;
    if (!XL || w_in == 0) {
      const int j0 = s0 - b * k;
      const RouteSel rs = wave_select<NV>(logits + (size_t)b * E, E, k, lane);
      if constexpr (XL) {
        extern __shared__ __attribute__((aligned(16))) uint8_t lds_x[];
        int* sel = reinterpret_cast<int*>(lds_x + 2 * H);
        for (int i = 0; i < 4; ++i) {
          const int ei = route_expert(rs, j0 + i);
          if (lane == 0) sel[i] = ei;
        }
      } else {
        e_raw = route_expert(rs, j0);
      }
      if (tile == 0) {   // the first neuron tile also stores ids and weights of its slots
        const float w = route_weight(rs, k, lane);
        if (lane >= j0 && lane < j0 + nsl) {
          ids_out[s0 + lane - j0] = rs.id;
          tw_out[s0 + lane - j0] = w;
        }
      }
    }
    if constexpr (XL) {
      extern __shared__ __attribute__((aligned(16))) uint8_t lds_x[];
      __syncthreads();
      e_raw = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(lds_x + 2 * H)[w_in]);
    }
  }
  const bool bad = (unsigned)e_raw >= (unsigned)E;
  const int e = bad ? 0 : e_raw;

  u32x4 gw[R][NCH], uw[R][NCH];
  uint32_t gsc[R][NCH], usc[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)(e * I + min(n0 + r, I - 1));   // ragged last tile: clamp, not stored
    const uint32_t woff = row * (uint32_t)H, soff = row * (uint32_t)nblk;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      gw[r][c] = bload16<kStream>(gr, off[c], woff);
      uw[r][c] = bload16<kStream>(ur, off[c], woff);
      gsc[r][c] = bload8<kStream>(gsr, off[c] >> 5, soff);
      usc[r][c] = bload8<kStream>(usr, off[c] >> 5, soff);
    }
  }

  // keep every load above this point: all of the wave's memory traffic is in flight at once
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XL) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // x[b], 2H bytes
#pragma unroll
    for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4*>(xs + xo[i]) = xv[i];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4* p = reinterpret_cast<const u32x4*>(xs + off[c] * 2u);
      xa[c][0] = p[0];
      xa[c][1] = p[1];
    }
  }

  float g[R], u[R];
  uint64_t nan_rows = 0;   // bit r: an E8M0 NaN code in row r
#pragma unroll
  for (int r = 0; r < R; ++r) {
    g[r] = 0.0f;
    u[r] = 0.0f;
    uint64_t nan_lanes = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      g[r] += apply_e8m0(chunk_dot(gw[r][c], xa[c], 0.0f), gsc[r][c], bias[c]);
      u[r] += apply_e8m0(chunk_dot(uw[r][c], xa[c], 0.0f), usc[r][c], bias[c]);
      nan_lanes |= nan_scale_lanes(gsc[r][c]) | nan_scale_lanes(usc[r][c]);
    }
    nan_rows |= (uint64_t)(nan_lanes != 0) << r;
  }
  // one reduce-scatter of the 2R sums: g[r] is index r, u[r] index R + r
  float v[2 * R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    v[r] = g[r];
    v[R + r] = u[r];
  }
  const float tot = wave_reduce_scatter<2 * R>(v, lane);
  // index R + r sits 32 lanes above index r: fetch it into the lower half
  float lo = tot, hi = tot;
  permlane32_swap(lo, hi);   // hi (lanes 0..31) = tot of lanes 32..63
  int r_out = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) r_out = (lane == scatter_lane<2 * R>(r)) ? r : r_out;
  if (r_out >= 0 && n0 + r_out < I) {
    const bool nan_out = bad || ((nan_rows >> r_out) & 1);
    const float hv = nan_out ? qnan() : silu(tot) * hi;
    h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(hv);
  }
}

}  // namespace moe
