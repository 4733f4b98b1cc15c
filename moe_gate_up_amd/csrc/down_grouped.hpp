// Down kernel, expert-grouped variant (blog post "warp decode", section "How
// the two kernels work", third and fourth paragraphs, for the arithmetic;
// section "Warp decode and Composer training" for the regime where several
// tokens share an expert).  Every output y[b,o] is still one FP32 sum over the
// token's k routed slots, each slot's dot product scaled by its router weight,
// written once as bf16, with no per-expert output buffer and no separate
// combine.  What changes is who reads the rows: a workgroup owns RO (8, or
// 4 for I > 1024) consecutive output dimensions for every token of the
// batch, so each routed expert's RO down rows are read once per layer however
// many tokens share it (the per-token kernel reads them once per token; at 32
// tokens x 8 of 128 experts, 2.3 times on average).
//
// Steps of one workgroup (NW wavefronts):
//  1. index the B*k slots by expert in LDS (slot_index.hpp);
//  2. the slots of each routed expert are cut into work units of at most 8
//     (so that an expert shared by many tokens is spread over wavefronts);
//     wavefront w starts with unit w and then takes the next unhanded unit
//     from an LDS counter whenever it comes free.  For each unit it loads
//     the expert's RO rows -- contiguous in memory, read as RO row passes
//     where lane l takes the 16 bytes at 16 l (+1024 per pass) -- and their
//     RO x I/32 E8M0 scales with one dword load per lane (moved to the
//     lanes that use them with ds_bpermute), then for every slot routed to
//     the expert loads that slot's h row, forms the RO dot products (E4M3 ->
//     bf16, v_dot2c_f32_bf16, v_ldexp_f32 per 16-element partial), sums them
//     across the wave with one reduce-scatter and stores router weight x sum
//     for each of the RO outputs as the slot's contribution in LDS;
//  3. thread (b, r) adds token b's k slot contributions in slot order and
//     writes y[b, o0 + r] once.
// The sum of every output runs in slot order whichever wavefront computed a
// slot's contribution: the result does not depend on timing.  Outputs of a
// token with an invalid id, or touching a row with a NaN scale code, are NaN.
#pragma once

#include "slot_index.hpp"

namespace moe {

constexpr int kDownGroupedMaxTokens = 64;  // one token per lane
constexpr int kDownGroupedSlotsPerRound = 2;
constexpr int kDownGroupedUnitSlots = 8;   // slots per work unit: a hot expert is spread over wavefronts

// Launch shape by passes of 1024 elements over I (graph-timed on MI355X):
// one pass (I <= 1024): 8 output dimensions per workgroup of 16 wavefronts;
// two passes: 4 output dimensions per workgroup of 8 wavefronts.
__host__ __device__ constexpr int down_grouped_rows(int np) { return np <= 1 ? 8 : 4; }
__host__ __device__ constexpr int down_grouped_waves(int np) { return np <= 1 ? 16 : 8; }
// LDS layout: slot index | per-slot contributions [S][RO] floats | per-slot
// NaN masks [S] | next-unit counter
__host__ __device__ constexpr int down_grouped_lds_bytes(int np, int E, int S) {
  return slot_index_lds_bytes(E, S) + S * (down_grouped_rows(np) + 1) * 4 + 16;
}

template <int NP>
__global__ __launch_bounds__(64 * down_grouped_waves(NP)) void moe_down_expert_grouped_w64(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ tw,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd,
    uint16_t* __restrict__ y, int B, int H, int I, int E, int k) {
  constexpr int NW = down_grouped_waves(NP);
  constexpr int NT = 64 * NW;
  constexpr int RO = down_grouped_rows(NP);
  constexpr int MS = kDownGroupedSlotsPerRound;
  const int slots = B * k;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int o0 = blockIdx.x * RO;
  float* contrib = reinterpret_cast<float*>(lds + slot_index_lds_bytes(E, slots));   // [S][RO]
  uint32_t* nanmask = reinterpret_cast<uint32_t*>(contrib + slots * RO);            // [S]
  int* next_unit = reinterpret_cast<int*>(nanmask + slots);
  // zero (a slot with an invalid id belongs to no unit) -- ordered before the
  // unit loop by the index build's barriers
  for (int i = tid; i < slots * (RO + 1); i += NT) contrib[i] = 0.0f;
  if (tid == 0) *next_unit = NW;   // units 0 .. NW-1 go to wavefronts 0 .. NW-1
  const SlotIndex si = build_slot_index<NT, false>(lds, ids, slots, E, k, kDownGroupedUnitSlots);

  const int nblk = I >> 5;
  uint32_t off[NP];
  int bias[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const int o = 1024 * c + 16 * lane;
    off[c] = (uint32_t)min(o, I - 16);
    bias[c] = o < I ? kLiveChunk : kDeadChunk;
  }
  const uint32_t wbytes = (uint32_t)E * (uint32_t)H * (uint32_t)I;   // < 2^32, checked on the host
  const rsrc_t wr = make_rsrc(wd, wbytes), sr = make_rsrc(sd, wbytes / 32);
  const rsrc_t hr = make_rsrc(h, (uint64_t)slots * I * 2), twr = make_rsrc(tw, (uint64_t)slots * 4);

  int r_lane = -1;   // the output row whose total this lane holds after the reduce-scatter
#pragma unroll
  for (int r = 0; r < RO; ++r) r_lane = (lane == scatter_lane<RO>(r)) ? r : r_lane;

  // the expert's RO rows and their scales (row0 * nblk is a multiple of 4: H
  // and o0 are multiples of 4); dword t of lane l holds scale bytes 256 t + 4 l ..
  u32x4 wv[RO][NP];
  uint32_t sw[NP];
  auto load_rows = [&](int e) {   // scales first: they are needed first
    const uint32_t row0 = (uint32_t)e * (uint32_t)H + (uint32_t)o0;
#pragma unroll
    for (int t = 0; t < NP; ++t)   // past the end of s_down: range-checked, reads zero
      sw[t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(sr, row0 * (uint32_t)nblk + 256u * t + 4u * lane, 0, kStream));
#pragma unroll
    for (int r = 0; r < RO; ++r)
#pragma unroll
      for (int c = 0; c < NP; ++c) wv[r][c] = bload16<kStream>(wr, off[c], (row0 + r) * (uint32_t)I);
  };
  // One work unit (up to 8 slots of one routed expert) with its expert's rows
  // already requested: its slots' h rows, dot products and accumulation.
  auto process = [&](int un) {
    int e, first, count;   // slots si.sorted[first .. first + count), count 1 .. kDownGroupedUnitSlots
    si.unit(un, e, first, count);

    // h rows and router weights of the first round of slots
    auto load_round = [&](int m0, u32x4 (&hv)[MS][NP][2], float (&ws)[MS]) {
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const uint32_t ent = si.sorted[first + min(m0 + m, count - 1)];   // past the end: repeat, unused
        const uint32_t sl = (uint32_t)__builtin_amdgcn_readfirstlane((int)(ent & 0xFFFFu));
#pragma unroll
        for (int c = 0; c < NP; ++c) {
          hv[m][c][0] = bload16(hr, off[c] * 2u, sl * (uint32_t)I * 2u);
          hv[m][c][1] = bload16(hr, off[c] * 2u + 16u, sl * (uint32_t)I * 2u);
        }
        ws[m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(twr, 0u, sl * 4u, 0));
      }
    };
    u32x4 hv[MS][NP][2];
    float ws[MS];
    load_round(0, hv, ws);
    __builtin_amdgcn_sched_barrier(0);

    // scale byte of (row r, pass c) for this lane, and the rows holding a NaN code
    uint32_t sc[RO][NP];
    uint32_t nan_rows = 0;
#pragma unroll
    for (int r = 0; r < RO; ++r) {
      uint64_t nl = 0;
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        const uint32_t q = (uint32_t)(r * nblk) + (off[c] >> 5);
        const int src = (int)(((q >> 2) & 63u) << 2);
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < NP; ++t) {
          const uint32_t vt = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sw[t]);
          v = ((q >> 8) == (uint32_t)t) ? vt : v;
        }
        sc[r][c] = (v >> ((q & 3u) * 8u)) & 0xFFu;
        nl |= nan_scale_lanes(sc[r][c]);
      }
      nan_rows |= (uint32_t)(nl != 0) << r;
    }

    for (int m0 = 0; m0 < count; m0 += MS) {
      if (m0 > 0) load_round(m0, hv, ws);
      const int nm = min(MS, count - m0);
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        if (m < nm) {
          // the rows stay E4M3 in registers and are converted per slot: keeping
          // them converted would double their registers past the 128 that a
          // 16-wavefront workgroup allows
#pragma unroll
          for (int r = 0; r < RO; ++r)
#pragma unroll
            for (int c = 0; c < NP; ++c) asm volatile("" : "+v"(wv[r][c].v[0]), "+v"(wv[r][c].v[1]), "+v"(wv[r][c].v[2]), "+v"(wv[r][c].v[3]));
          float p[RO];
#pragma unroll
          for (int r = 0; r < RO; ++r) {
            p[r] = 0.0f;
#pragma unroll
            for (int c = 0; c < NP; ++c) p[r] += apply_e8m0(chunk_dot(wv[r][c], hv[m][c], 0.0f), sc[r][c], bias[c]);
          }
          const float tot = wave_reduce_scatter<RO>(p, lane);
          const int sl = __builtin_amdgcn_readfirstlane((int)(si.sorted[first + m0 + m] & 0xFFFFu));
          const float wsm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, ws[m])));
          // the slot's weighted contribution to its token's RO outputs, kept
          // per slot: the final sum runs over slots in a fixed order, whichever
          // wavefront computed them
          if (r_lane >= 0) contrib[sl * RO + r_lane] = wsm * tot;
          if (lane == 0) nanmask[sl] = nan_rows;
        }
      }
      // An unconditional use of every load of the round, after all of its
      // consumers: it keeps the compiler from sinking a slot's loads into that
      // slot's branch (which put their latency behind the previous slot's
      // work); by now the values have arrived, so it costs no wait.
#pragma unroll
      for (int m = 0; m < MS; ++m) {
#pragma unroll
        for (int c = 0; c < NP; ++c) asm volatile("" ::"v"(hv[m][c][0].v[0]), "v"(hv[m][c][1].v[0]));
        asm volatile("" ::"v"(ws[m]));
      }
    }
    };

  // Units are handed out as wavefronts come free (an LDS counter): units
  // differ in slot count and in memory latency, and a fixed round-robin left
  // a workgroup's slowest wavefront finishing long after its fastest.  The
  // first unit is processed outside the loop and its rows are loaded
  // unconditionally (a wavefront without a unit reads rows it will not use),
  // so no row register is merged across a branch or carried around the loop:
  // either made the compiler wait for the loads right away.
  load_rows(si.n_units > 0 ? si.unit_expert(min(w, si.n_units - 1)) : 0);
  if (w < si.n_units) {
    process(w);
    for (;;) {
      int un = 0;
      if (lane == 0) un = atomicAdd(next_unit, 1);
      un = __builtin_amdgcn_readfirstlane(un);
      if (un >= si.n_units) break;
      load_rows(si.unit_expert(un));
      process(un);
    }
  }

  // ---- thread (b, r) adds its token's k slot contributions in slot order
  __syncthreads();
  for (int t = tid; t < B * RO; t += NT) {
    const int b = t / RO, r = t - b * RO;
    float sum = 0.0f;
    uint32_t nn = 0;
    for (int j = 0; j < k; ++j) {
      sum += contrib[(b * k + j) * RO + r];
      nn |= nanmask[b * k + j];
    }
    bool nan_out = (nn >> r) & 1u;
    if (si.n_bad > 0) {   // a token with an invalid id is NaN everywhere
      for (int j = 0; j < k; ++j) nan_out |= (unsigned)ids[b * k + j] >= (unsigned)E;
    }
    y[(size_t)b * H + o0 + r] = f32_to_bf16_rne(nan_out ? qnan() : sum);
  }
}

}  // namespace moe
