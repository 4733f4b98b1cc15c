// Gate/up kernel, expert-grouped variant (blog post "warp decode", section
// "How the two kernels work" for the arithmetic; section "Warp decode and
// Composer training" for why grouping pays once several tokens share an
// expert).  Every output h[b,j,n] is still one neuron's SiLU(gate) * up,
// produced from streamed MXFP8 rows dotted with x[b] in FP32 and written
// once, with no padding, expert-major gather buffer or combine.  What changes
// is who reads the rows: a work item is 4R consecutive neurons of one routed
// expert e (R per wavefront) for every slot routed to e, so each routed row is
// read from memory once per layer however many tokens share the expert.  The
// per-slot kernel reads it once per slot; at 32 tokens x 8 of 128 experts the
// average routed expert serves 2.3 slots, and those repeat reads (L2 hits)
// occupy the vector-memory pipeline that the weight stream needs.
//
// The grid is persistent: at most 2048 workgroups (about two per slot the
// chip holds at once), each taking pairs of work items round-robin.  Every
// workgroup first indexes the B*k <= 1024 slots by expert in LDS
// (slot_index.hpp), which yields the routed experts and each one's slots, cut
// into work units of at most min(4M, 16) slots (four fillings of the 32 KB
// LDS staging area of M x rows), so that an expert shared by many tokens is
// spread over several workgroups while an expert with a handful of slots is
// one unit (its rows read once).  Since one expert's units go to different
// workgroups, every workgroup must cut them alike: the index puts the slots
// of such experts in slot order (STABLE).  Unrouted experts produce no
// work.  A work item is a work
// unit times a group of 4R neurons:
//  1. each wavefront issues its R gate and R up rows (1 KB-contiguous passes
//     as in the per-slot kernel) and their E8M0 scales;
//  2. per chunk of up to M slots, the 4 wavefronts copy those tokens' x rows
//     into LDS with direct global->LDS loads (1 KB per wave instruction, no
//     registers) unless the previous item's unit left them there, one
//     barrier, then each wavefront takes the chunk's slots in
//     turn: it reads its lanes' slice of x from LDS, forms the 2R dot products
//     from the bf16-converted rows with v_dot2c_f32_bf16, scales each
//     16-element partial by its E8M0 scale (v_ldexp_f32), reduces the 2R sums
//     with one reduce-scatter and writes R outputs.
// Slots whose id is outside [0, E) get NaN in every neuron, written by the
// workgroup blockIdx.x == slot mod gridDim.x, so every output is written
// exactly once.
#pragma once

#include "slot_index.hpp"

namespace moe {

constexpr int kGroupedMaxSlots = kSortMaxSlots;       // B*k limit of the expert-grouped variant
constexpr int kGroupedMaxExperts = kSortMaxExperts;   // E limit
constexpr int kGroupedXBytes = 32768;                 // LDS for staged activations
constexpr int kGroupedUnitChunks = 4;                 // staging rounds per work unit, up to
constexpr int kGroupedUnitMaxSlots = 16;              // slots per work unit

// bytes of one staged x row (1 KB-padded) and rows per chunk (at most 8)
constexpr int kGroupedMaxChunk = 8;
__host__ __device__ constexpr int grouped_xrow(int H) { return ((2 * H + 1023) / 1024) * 1024; }
__host__ __device__ constexpr int grouped_chunk(int H) {
  return kGroupedXBytes / grouped_xrow(H) < 1
             ? 1
             : (kGroupedXBytes / grouped_xrow(H) > kGroupedMaxChunk ? kGroupedMaxChunk : kGroupedXBytes / grouped_xrow(H));
}
// slots per work unit: four fillings of the staging area, at most 16 (a hot
// expert's slots are spread over several workgroups)
__host__ __device__ constexpr int grouped_unit_slots(int H) {
  return kGroupedUnitChunks * grouped_chunk(H) < kGroupedUnitMaxSlots ? kGroupedUnitChunks * grouped_chunk(H)
                                                                      : kGroupedUnitMaxSlots;
}
// LDS layout: slot index | staged x [M rows]
__host__ __device__ constexpr int grouped_lds_bytes(int E, int S, int H) {
  return slot_index_lds_bytes(E, S) + grouped_chunk(H) * grouped_xrow(H);
}

// Up to 4 rows x passes: at least 4 wavefronts per SIMD (<= 128 VGPRs), so
// that the persistent grid keeps 4 workgroups per CU in flight.
__host__ __device__ constexpr int grouped_min_waves(int nch, int r) { return nch * r <= 4 ? 4 : 1; }

template <int NCH, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(grouped_min_waves(NCH, R))))
void moe_gate_up_expert_grouped_w64(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint8_t* __restrict__ su,
    uint16_t* __restrict__ h, int B, int H, int I, int E, int k) {
  const int slots = B * k;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const SlotIndex si = build_slot_index<256, true>(lds, ids, slots, E, k, grouped_unit_slots(H));
  uint8_t* xs = lds + slot_index_lds_bytes(E, slots);   // M rows of x, 2H bytes each, 1 KB-padded
  const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);

  // ---- per-lane constants of the R-row passes
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
  int r_out = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) r_out = (lane == scatter_lane<2 * R>(r)) ? r : r_out;
  const int XS = grouped_xrow(H);
  const int pieces = XS >> 10;
  // x rows per chunk.  MCAP bounds it for this NCH (H > 1024 (NCH - 1), so a
  // staged row is more than 2 KB (NCH - 1)) and sizes the token registers.
  constexpr int MC = kGroupedXBytes / 2048 / (NCH > 1 ? NCH - 1 : 1);
  constexpr int MCAP = NCH == 1 || MC > kGroupedMaxChunk ? kGroupedMaxChunk : (MC > 0 ? MC : 1);
  const int M = min(grouped_chunk(H), MCAP);

  // ---- work items: (work unit = up to M slots of one routed expert, group of 4 tiles g)
  const int n_grp = (I + 4 * R - 1) / (4 * R);
  const int n_items = si.n_units * n_grp;
  u32x4 gw[R][NCH], uw[R][NCH];
  uint32_t gsc[R][NCH], usc[R][NCH];
  auto load_rows = [&](int e, int n0) {   // the wavefront's R gate and R up rows of expert e
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = (uint32_t)(e * I + min(n0 + r, I - 1));   // ragged: clamp, not stored
      const uint32_t woff = row * (uint32_t)H, soff = row * (uint32_t)nblk;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        gw[r][c] = bload16<kStream>(gr, off[c], woff);
        uw[r][c] = bload16<kStream>(ur, off[c], woff);
        gsc[r][c] = bload8<kStream>(gsr, off[c] >> 5, soff);
        usc[r][c] = bload8<kStream>(usr, off[c] >> 5, soff);
      }
    }
  };
  // the item's expert, its unit's slots (si.sorted[first .. first + count)) and the wavefront's first neuron
  auto item_unit = [&](int item, int& e, int& first, int& count, int& n0) {
    const int un = __builtin_amdgcn_readfirstlane(item / n_grp);   // VALU division, uniform result
    si.unit(un, e, first, count);
    n0 = ((item - un * n_grp) * 4 + w) * R;   // may be >= I: nothing stored
  };
  // Items go out round-robin in pairs: workgroup b takes items 2b, 2b + 1,
  // then 2(b + G), 2(b + G) + 1, ...  The two items of a pair are mostly
  // neighbouring neuron groups of one unit, so the second one finds the
  // unit's x rows still staged in LDS; the items that run at the same time
  // stay next to each other in the weight tensors.  (Pairs measured 1-3 %
  // faster than single items, quads slower at 32 tokens; contiguous
  // per-workgroup ranges were slower still.)
  constexpr int kPair = 2;
  int staged = -1;     // the unit whose x rows are all in LDS, or -1
  bool used = false;   // an earlier item of this workgroup used the staging area
  for (int t = 0;; ++t) {
    const int item = (blockIdx.x + (t / kPair) * gridDim.x) * kPair + t % kPair;
    if (item >= n_items) break;
    int e, first, count, n0;   // count: 1 .. 4M
    item_unit(item, e, first, count, n0);
    const int un = __builtin_amdgcn_readfirstlane(item / n_grp);
    load_rows(e, n0);
    const bool restage = staged != un || count > M;

    // x rows are copied global -> LDS without passing through registers
    // (buffer loads with the LDS bit: lane l's 16 bytes land at the
    // wave-uniform LDS base + 16 l); a row is cut into 1 KB pieces, piece p
    // by wavefront p % 4, and rows sit XS bytes apart in LDS.  Bytes past 2H
    // land in the row's padding and are never read; the whole offset is in
    // the lane offset, so reads past the end of x are range-checked (zero).
    auto stage = [&](int m0) {
      const int nm = min(M, count - m0);
      uint32_t tok[MCAP];   // the chunk's tokens: all LDS reads first, one round trip
#pragma unroll
      for (int m = 0; m < MCAP; ++m)
        tok[m] = m < nm ? si.sorted[first + m0 + m] >> 16 : 0u;
#pragma unroll
      for (int m = 0; m < MCAP; ++m) {
        if (m < nm) {
          const uint32_t xo = (uint32_t)__builtin_amdgcn_readfirstlane((int)tok[m]) * (uint32_t)H * 2u;
          for (int p = w; p < pieces; p += 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(xs + m * XS + 1024 * p),
                                                     16, xo + 1024u * p + 16u * lane, 0, 0, 0);
        }
      }
    };
    if (restage) {
      if (used) __syncthreads();   // every wavefront is done with the staged x
      stage(0);   // the first chunk's copies go out before anything waits for the weights
    }
    bool nan_out = false;
    for (int m0 = 0; m0 < count; m0 += M) {
      if (m0 > 0) {
        __syncthreads();   // every wavefront is done with the previous chunk's x
        stage(m0);
      }
      const int nm = min(M, count - m0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the rows, and this wavefront's copies in LDS
      if (restage || m0 > 0) __syncthreads();     // every wavefront's copies
      if (m0 == 0) {   // the scales have arrived by now
        uint64_t nan_rows = 0;   // bit r: an E8M0 NaN code in row r
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint64_t nan_lanes = 0;
#pragma unroll
          for (int c = 0; c < NCH; ++c) nan_lanes |= nan_scale_lanes(gsc[r][c]) | nan_scale_lanes(usc[r][c]);
          nan_rows |= (uint64_t)(nan_lanes != 0) << r;
        }
        nan_out = r_out >= 0 && ((nan_rows >> r_out) & 1);
      }
      for (int m = 0; m < nm; ++m) {
        const int s = (int)(si.sorted[first + m0 + m] & 0xFFFFu);
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
        if (r_out >= 0 && n0 + r_out < I) h[(size_t)s * I + n0 + r_out] = f32_to_bf16_rne(nan_out ? qnan() : silu(tot) * hi);
      }
    }
    staged = count > M ? -1 : un;   // a unit staged in several chunks leaves only its last chunk
    used = true;
  }

  // ---- slots with an invalid expert id: NaN in every neuron
  if (si.n_bad > 0) {
    for (int sl = blockIdx.x; sl < slots; sl += gridDim.x) {
      const int v = (int)__builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)sl * 4u, 0, 0));
      if ((unsigned)__builtin_amdgcn_readfirstlane(v) >= (unsigned)E)
        for (int n = tid; n < I; n += 256) h[(size_t)sl * I + n] = f32_to_bf16_rne(qnan());
    }
  }
}

}  // namespace moe
