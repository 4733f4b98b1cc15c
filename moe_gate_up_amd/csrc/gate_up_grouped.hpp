// Gate/up kernel, expert-grouped variant (blog post "warp decode", section
// "How the two kernels work" for the arithmetic; section "Warp decode and
// Composer training" for why grouping pays once several tokens share an
// expert).  Every output h[b,j,n] is still one neuron's SiLU(gate) * up,
// produced from streamed MXFP8 rows dotted with x[b] in FP32 and written
// once, with no padding, expert-major gather buffer or combine.  What changes
// is who reads the rows: a workgroup owns 4R consecutive neurons of one
// expert e (R per wavefront) for every slot routed to e, so each routed row is
// read from memory once per layer however many tokens share the expert.  The
// per-slot kernel reads it once per slot; at 32 tokens x 8 of 128 experts the
// average expert serves 2.3 slots, and those repeat reads (L2 hits) occupy
// the vector-memory pipeline that the weight stream needs.
//
// Steps of one workgroup:
//  1. the 4 wavefronts split topk_ids (B*k <= 1024: at most 4 dword loads per
//     lane) and count the slots routed to e with ballots; the counts meet in
//     LDS, and with none the whole workgroup leaves before any weight is read;
//  2. each wavefront issues its R gate and R up rows (1 KB-contiguous passes
//     as in the per-slot kernel) and their E8M0 scales, then writes its part
//     of the list of e's slots (slot index and token) to LDS;
//  3. per chunk of up to M slots, the 4 wavefronts copy those tokens' x rows
//     into LDS (direct global->LDS loads, 1 KB per wave instruction), one
//     barrier, then each
//     wavefront takes the chunk's slots in turn: it reads its lanes' slice of
//     x from LDS, converts its raw E4M3 rows to bf16 pairs and forms the 2R
//     dot products with v_dot2c_f32_bf16, scales each 16-element partial by
//     its E8M0 scale (v_ldexp_f32), reduces the 2R sums with one
//     reduce-scatter and writes R outputs.
// The workgroup for expert 0 also writes NaN for the slots whose id is
// outside [0, E), so every output is written exactly once.
//
// Grid: workgroup id = neuron group * E + e.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kGroupedMaxSlots = 1024;                   // B*k limit of the expert-grouped variant
constexpr int kGroupedIdLoads = kGroupedMaxSlots / 64;   // topk_ids dwords per lane
constexpr int kGroupedInfoBytes = kGroupedIdLoads * 4;   // LDS per-group counts
constexpr int kGroupedListBytes = kGroupedMaxSlots * 4;  // LDS slot list
constexpr int kGroupedXBytes = 32768;                    // LDS for staged activations

// slots per chunk: M x rows of 2*1024*NCH bytes fit in kGroupedXBytes
constexpr int grouped_chunk(int nch) { return 16 / nch < 1 ? 1 : (16 / nch > 8 ? 8 : 16 / nch); }
constexpr int grouped_lds_bytes(int nch, int H) {
  return kGroupedInfoBytes + kGroupedListBytes + grouped_chunk(nch) * (((2 * H + 1023) / 1024) * 1024);
}

template <int NCH, int R>
__global__ __launch_bounds__(256) void moe_gate_up_expert_grouped_w64(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint8_t* __restrict__ su,
    uint16_t* __restrict__ h, int B, int H, int I, int E, int k) {
  constexpr int M = grouped_chunk(NCH);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint32_t* qinfo = reinterpret_cast<uint32_t*>(lds);                  // per 64-slot group: count | invalid << 31
  uint32_t* list = reinterpret_cast<uint32_t*>(lds + kGroupedInfoBytes);   // e's slots
  uint8_t* xs = lds + kGroupedInfoBytes + kGroupedListBytes;           // M rows of x, 2H bytes each, 1 KB-padded

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, in an SGPR
  const int blk = blockIdx.x;
  const int grp = __builtin_amdgcn_readfirstlane(blk / E);   // VALU division, uniform result
  const int e = blk - grp * E;
  const int n0 = (grp * 4 + w) * R;   // this wavefront's first neuron (may be >= I: nothing stored)
  const int slots = B * k;
  const int nq = (slots + 63) >> 6;

  // ---- 1. which slots use e.  Wavefront w scans the 64-slot groups q = w,
  // w+4, w+8, w+12 (one dword load per lane each) and posts each group's
  // count of e's slots (and whether it holds an invalid id) to LDS.
  const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);
  constexpr int QW = kGroupedIdLoads / 4;   // groups per wavefront
  int idq[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int sl = 64 * (w + 4 * i) + lane;
    idq[i] = (int)__builtin_bit_cast(
        uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)min(sl, slots - 1) * 4u, 0, 0));
  }
  uint64_t mq[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const bool real = 64 * (w + 4 * i) + lane < slots;
    mq[i] = __builtin_amdgcn_ballot_w64(real && idq[i] == e);
    const bool bad = __builtin_amdgcn_ballot_w64(real && (unsigned)idq[i] >= (unsigned)E) != 0;
    if (lane == 0) qinfo[w + 4 * i] = (uint32_t)__builtin_popcountll(mq[i]) | ((uint32_t)bad << 31);
  }
  __syncthreads();
  const uint32_t qi = qinfo[lane & (kGroupedIdLoads - 1)];
  int count = 0, any_bad = 0;
  int qbase[kGroupedIdLoads];   // slots of e in groups before q (uniform)
#pragma unroll
  for (int q = 0; q < kGroupedIdLoads; ++q) {
    const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)qi, q);
    qbase[q] = count;
    count += (int)(v & 0x7FFFFFFFu);
    any_bad |= (int)(v >> 31);
  }
  const bool nan_duty = e == 0 && any_bad;
  if (count == 0 && !nan_duty) return;   // same decision in all 4 wavefronts: no barrier is left waiting

  // ---- 2. the wavefront's R gate and R up rows of expert e, raw
  uint32_t off[NCH];
  int bias[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int o = 1024 * c + 16 * lane;
    off[c] = (uint32_t)min(o, H - 16);
    bias[c] = o < H ? kLiveChunk : kDeadChunk;
  }
  const int nblk = H >> 5;
  const uint32_t wbytes = (uint32_t)E * (uint32_t)I * (uint32_t)H;   // < 2^32, checked on the host
  const rsrc_t xr = make_rsrc(x, (uint64_t)B * H * 2);
  const rsrc_t gr = make_rsrc(wg, wbytes), ur = make_rsrc(wu, wbytes);
  const rsrc_t gsr = make_rsrc(sg, wbytes / 32), usr = make_rsrc(su, wbytes / 32);
  u32x4 gw[R][NCH], uw[R][NCH];
  uint32_t gsc[R][NCH], usc[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)(e * I + min(n0 + r, I - 1));   // ragged: clamp, not stored
    const uint32_t woff = row * (uint32_t)H, soff = row * (uint32_t)nblk;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      gw[r][c] = bload16(gr, off[c], woff);
      uw[r][c] = bload16(ur, off[c], woff);
      gsc[r][c] = bload8(gsr, off[c] >> 5, soff);
      usc[r][c] = bload8(usr, off[c] >> 5, soff);
    }
  }

  // list of e's slots in slot order: slot | token << 16
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    if (mq[i] >> lane & 1) {
      const int pos = qbase[w + 4 * i] +
                      (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mq[i] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mq[i], 0u));
      const int sl = 64 * (w + 4 * i) + lane;
      list[pos] = (uint32_t)sl | ((uint32_t)(sl / k) << 16);
    }
  }
  __syncthreads();

  int r_out = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) r_out = (lane == scatter_lane<2 * R>(r)) ? r : r_out;
  const bool writer = r_out >= 0 && n0 + r_out < I;
  bool nan_out = false;

  // ---- 3. chunks of up to M slots.  x rows are copied global -> LDS without
  // passing through registers (buffer loads with the LDS bit: lane l's 16 bytes
  // land at the wave-uniform LDS base + 16 l); a row is cut into 1 KB pieces,
  // piece p by wavefront p % 4, and rows sit XS bytes apart in LDS.
  const int pieces = (2 * H + 1023) >> 10;
  const int XS = pieces << 10;
  auto stage = [&](int m0) {   // issue the copies of slots m0 .. m0 + M - 1
    const int nm = min(M, count - m0);
    for (int m = 0; m < nm; ++m) {
      const uint32_t xo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(list[m0 + m] >> 16)) * (uint32_t)H * 2u;
      // bytes past 2H land in the row's padding and are never read; the whole
      // offset is in the lane offset, so reads past the end of x are range-checked (zero)
      for (int p = w; p < pieces; p += 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xs + m * XS + 1024 * p), 16,
                                                 xo + 1024u * p + 16u * lane, 0, 0, 0);
    }
  };
  // the first chunk's copies go out before anything waits for the weights
  if (count > 0) stage(0);
  for (int m0 = 0; m0 < count; m0 += M) {
    if (m0 > 0) {
      __syncthreads();   // every wavefront is done with the previous chunk's x
      stage(m0);
    }
    const int nm = min(M, count - m0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wavefront's copies are in LDS
    __syncthreads();
    if (m0 == 0) {   // the scales have arrived by now
      uint64_t nan_rows = 0;   // bit r: an E8M0 NaN code in row r
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint64_t nan_lanes = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) nan_lanes |= nan_scale_lanes(gsc[r][c]) | nan_scale_lanes(usc[r][c]);
        nan_rows |= (uint64_t)(nan_lanes != 0) << r;
      }
      nan_out = writer && ((nan_rows >> r_out) & 1);
    }
    for (int m = 0; m < nm; ++m) {
      const int s = (int)(list[m0 + m] & 0xFFFFu);
      u32x4 xa[NCH][2];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const u32x4* p = reinterpret_cast<const u32x4*>(xs + m * XS + off[c] * 2u);
        xa[c][0] = p[0];
        xa[c][1] = p[1];
      }
      float v[2 * R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        v[r] = 0.0f;
        v[R + r] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          v[r] += apply_e8m0(chunk_dot(gw[r][c], xa[c], 0.0f), gsc[r][c], bias[c]);
          v[R + r] += apply_e8m0(chunk_dot(uw[r][c], xa[c], 0.0f), usc[r][c], bias[c]);
        }
      }
      const float tot = wave_reduce_scatter<2 * R>(v, lane);
      float lo = tot, hi = tot;
      permlane32_swap(lo, hi);   // hi (lanes 0..31) = the up sum, 32 lanes above the gate sum
      if (writer) h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(nan_out ? qnan() : silu(tot) * hi);
    }
  }

  // ---- slots with an invalid expert id: NaN, written by expert 0's workgroup
  if (nan_duty) {   // ids read again rather than kept live in 16 VGPRs
    for (int q = 0; q < nq; ++q) {
      {
        const int sl = 64 * q + lane;
        const int v = (int)__builtin_bit_cast(
            uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)min(sl, slots - 1) * 4u, 0, 0));
        uint64_t m = __builtin_amdgcn_ballot_w64(sl < slots && (unsigned)v >= (unsigned)E);
        while (m) {
          const int s = 64 * q + __builtin_ctzll(m);
          m &= m - 1;
          if (writer) h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(qnan());
        }
      }
    }
  }
}

}  // namespace moe
