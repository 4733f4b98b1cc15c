// Down kernel, expert-grouped variant with the dot products on the matrix
// cores (blog post "warp decode", section "How the two kernels work", third
// and fourth paragraphs, for the arithmetic; section "Warp decode and
// Composer training" for the regime where several tokens share an expert).
// Every output y[b,o] is still one FP32 sum over the token's k routed slots,
// each slot's dot product scaled by its router weight, written once as bf16,
// with no per-expert output buffer and no separate combine.
//
// Organisation as in the vector-unit grouped down kernel: a workgroup owns 8
// consecutive output dimensions o0..o0+7 for every token; it indexes the
// B*k slots by expert in LDS, cuts each routed expert's slots into work
// units of at most 8, and its wavefronts take units as they come free (an
// LDS counter).  Each slot's weighted contribution to the 8 outputs goes to
// LDS, and at the end thread (b, r) adds token b's k contributions in slot
// order and writes y[b, o0 + r] once, so the result does not depend on which
// wavefront took which unit.
//
// What changes is the product.  For one unit the wavefront reads the expert's
// 8 rows once, converts each E4M3 value to bf16 once per group of 4 slots
// (exact: every E4M3 value is a bf16 value), and forms all 8 x (up to 4)
// dot products with v_mfma_f32_4x4x4_16b_bf16: 16 independent 4x4x4
// products per instruction.  Block b of the 16 takes the 16-element chunk b
// of a 256-element round of the reduction: lane 4b + j holds 16 bytes of row
// j of a row group of 4 (one contiguous 256-byte run per row and load) and
// lane 4b + i the 32 bytes of slot i's h over the same 16 elements; four
// instructions cover the chunk (4 elements each), and the result of block b
// lands in lane 4b + j, register i = slot i.  Each 16-element chunk lies in
// one 32-element MX block, so the lane that loaded the row's chunk scales
// the chunk's FP32 partial sums by the block's E8M0 scale with v_ldexp_f32
// (exact) and adds them up over the rounds; the 16 chunks are then summed
// across lanes (permlane swaps and DPP rotations, no LDS).  The NaN scale
// code 0xFF forces the affected outputs to NaN, as in the vector kernels;
// chunks past the end of a row re-read the row's last chunk and are scaled
// by 2^-512 (zero).
//
// The vector units only convert and scale: per unit and group of 4 slots, 48
// conversions, 48 scale-and-add steps and ~20 reduction steps per lane,
// against ~160 instructions per slot (conversion, dot2, ldexp, reduction) in
// the vector-unit grouped kernel.
#pragma once

#include "slot_index.hpp"

namespace moe {

constexpr int kDownMfmaRows = 8;        // output dimensions per workgroup: 2 row groups of 4
constexpr int kDownMfmaUnitSlots = 8;   // slots per work unit (2 groups of 4 MFMA columns)
constexpr int kDownMfmaMaxRounds = 8;   // I <= 8 rounds of 256 elements

// Launch shape by rounds of 256 elements over I (graph-timed on MI355X, H =
// 2048, I = 768, 32 tokens): 12 wavefronts per workgroup up to 3 rounds (34.4
// us against 35.6 with 16 and 35.2 with 8; more units in flight per CU only
// lengthen the queues), 8 up to 6 rounds, 6 beyond so that the stages fit LDS
// (160 KB per CU).
__host__ __device__ constexpr int down_mfma_waves(int nr) { return nr <= 3 ? 12 : (nr <= 6 ? 8 : 6); }
// Each wavefront stages its unit's 8 rows in LDS, each row padded to whole
// rounds of 256 bytes.
__host__ __device__ constexpr int down_mfma_stage_bytes(int nr) { return kDownMfmaRows * 256 * nr; }
// LDS layout: slot index | per-slot contributions [S][8] floats | per-slot
// NaN masks [S] | next-unit counter | one row stage per wavefront
__host__ __device__ constexpr int down_mfma_lds_bytes(int nr, int E, int S) {
  return a16(slot_index_lds_bytes(E, S) + S * (kDownMfmaRows + 1) * 4 + 16) +
         down_mfma_waves(nr) * down_mfma_stage_bytes(nr);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

// Four E4M3 codes (one dword, byte order) -> four bf16 values (exact).
__device__ __forceinline__ bf16x4_t e4m3x4_to_bf16x4(uint32_t word) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true);
  bf16x4_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
  return r;
}

__device__ __forceinline__ bf16x4_t as_bf16x4(uint32_t a, uint32_t b) {
  bf16x2_t x = as_bf16x2(a), y = as_bf16x2(b);
  bf16x4_t r;
  r[0] = x[0]; r[1] = x[1]; r[2] = y[0]; r[3] = y[1];
  return r;
}

template <int NR>
__global__ __launch_bounds__(64 * down_mfma_waves(NR)) void moe_down_grouped_mfma_w64(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ ids, const float* __restrict__ tw,
    const uint8_t* __restrict__ wd, const uint8_t* __restrict__ sd,
    uint16_t* __restrict__ y, int B, int H, int I, int E, int k) {
  constexpr int NW = down_mfma_waves(NR);
  constexpr int NT = 64 * NW;
  constexpr int RO = kDownMfmaRows;
  const int slots = B * k;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int o0 = blockIdx.x * RO;
  float* contrib = reinterpret_cast<float*>(lds + slot_index_lds_bytes(E, slots));   // [S][RO]
  uint32_t* nanmask = reinterpret_cast<uint32_t*>(contrib + slots * RO);            // [S]
  int* next_unit = reinterpret_cast<int*>(nanmask + slots);
  uint8_t* stage = lds + a16(slot_index_lds_bytes(E, slots) + slots * (RO + 1) * 4 + 16) +
                   w * down_mfma_stage_bytes(NR);   // this wavefront's rows
  // zero (a slot with an invalid id belongs to no unit) -- ordered before the
  // unit loop by the index build's barriers
  for (int i = tid; i < slots * (RO + 1); i += NT) contrib[i] = 0.0f;
  if (tid == 0) *next_unit = NW;   // units 0 .. NW-1 go to wavefronts 0 .. NW-1
  const SlotIndex si = build_slot_index<NT, false>(lds, ids, slots, E, k, kDownMfmaUnitSlots);

  // lane 4b + j: chunk b of every round; row j of a row group (weights) and
  // slot column j (h) of the matrix-core blocks
  const int lb = lane >> 2, lj = lane & 3;
  const int nblk = I >> 5;
  uint32_t koff[NR];   // the lane's element offset in round r (a chunk past the row's end re-reads the last one)
  int kbias[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int o = 256 * r + 16 * lb;
    koff[r] = (uint32_t)min(o, I - 16);
    kbias[r] = o < I ? kLiveChunk : kDeadChunk;
  }
  const uint32_t wbytes = (uint32_t)E * (uint32_t)H * (uint32_t)I;   // < 2^32, checked on the host
  const rsrc_t wr = make_rsrc(wd, wbytes), sr = make_rsrc(sd, wbytes / 32);
  const rsrc_t hr = make_rsrc(h, (uint64_t)slots * I * 2), twr = make_rsrc(tw, (uint64_t)slots * 4);

  // The unit's 8 rows are contiguous in memory (8 x I bytes); they are copied
  // into this wavefront's stage with buffer loads that write LDS directly,
  // 1 KB of consecutive bytes per instruction (lane l takes 16 bytes).  In the
  // stage a row occupies NR x 256 bytes, 16 NR pieces of 16 bytes; piece p of
  // row rho sits at position p ^ 4 (rho mod 4), so that the reads below -- 4
  // rows at the same position in each 16-lane group -- fall in distinct
  // banks.  Positions past a row's end hold a copy of its last piece (never
  // read).  Loading the rows straight into the product layout instead
  // (4 rows x 256 bytes per instruction) streamed ~8 % slower.
  //
  // Their 8 x I/32 scale codes are contiguous too: dword t of lane l holds
  // bytes 256 t + 4 l .. (one dword load per lane and 256 bytes; a byte load
  // per chunk instead cost ~5 us at 32 tokens, H = 2048, I = 768).
  constexpr int NSW = NR <= 4 ? 1 : 2;   // 8 x I/32 <= 512 bytes
  constexpr int PR = 16 * NR;            // stage pieces per row
  uint32_t sw[NSW];
  const int npr = I >> 4;                // real pieces per row
  auto load_rows = [&](int e) {
    typedef __attribute__((address_space(3))) void lds_void;
    const uint32_t row0 = (uint32_t)e * (uint32_t)H + (uint32_t)o0;   // wave-uniform
#pragma unroll
    for (int t = 0; t < NSW; ++t)   // past the end of s_down: range-checked, reads zero (the range
      // check covers the vector offset only, so the whole offset goes there)
      sw[t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(sr, row0 * (uint32_t)nblk + 256u * t + 4u * lane, 0, kStream));
#pragma unroll
    for (int t = 0; t < 2 * NR; ++t) {   // 8 rows x PR pieces = 2 NR instructions of 64 pieces
      const int P = 64 * t + lane;
      const int rho = P / PR, q = P - rho * PR;
      const int pc = min(q ^ (4 * (rho & 3)), npr - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(stage + 1024 * t), 16,
                                               (uint32_t)rho * (uint32_t)I + 16u * (uint32_t)pc,
                                               row0 * (uint32_t)I, 0, kStream);
    }
  };
  // the lane's 16 bytes of (row group g, round r) from the stage
  auto stage_read = [&](int g, int r) {
    const int p = (int)(koff[r] >> 4);
    return *reinterpret_cast<const u32x4*>(stage + (4 * g + lj) * (16 * PR) + 16 * (p ^ (4 * lj)));
  };
  // the scale code of (row group g, round r) for this lane's row and chunk,
  // moved from the lane that loaded it
  auto scale_codes = [&](uint32_t (&sc)[2][NR]) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t q = (uint32_t)((4 * g + lj) * nblk) + (koff[r] >> 5);
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < NSW; ++t) {
          const uint32_t vt = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((q >> 2) & 63u) << 2), (int)sw[t]);
          v = (q >> 8) == (uint32_t)t ? vt : v;
        }
        sc[g][r] = (v >> ((q & 3u) * 8u)) & 0xFFu;
      }
  };

  // One work unit (up to 8 slots of one routed expert) with its expert's rows
  // already requested.  Both groups' h (slots 0-3 and 4-7) are requested
  // before any product: requested after the first group's products, the
  // second group's waited a whole L2 round trip per unit (at 64 tokens, where
  // most units have more than 4 slots, the down kernel ran 44.2 us against
  // 37.6 with no h loads at all).
  static_assert(kDownMfmaUnitSlots == 8, "two groups of 4 slot columns per unit");
  // the lane's slot column of group m0 (past the unit's end: the last slot again, unused), its h and weight
  auto load_group = [&](int first, int count, int m0, uint32_t& sl, u32x4 (&hv)[NR][2], float& wsl) {
    sl = si.sorted[first + min(m0 + lj, count - 1)] & 0xFFFFu;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      hv[r][0] = bload16(hr, sl * (uint32_t)I * 2u + koff[r] * 2u, 0);
      hv[r][1] = bload16(hr, sl * (uint32_t)I * 2u + koff[r] * 2u + 16u, 0);
    }
    wsl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(twr, sl * 4u, 0, 0));
  };
  // the products of slot columns m0 .. m0 + 3 and their contributions
  auto group = [&](int first, int count, int m0, const uint32_t (&sc)[2][NR], uint32_t sl, const u32x4 (&hv)[NR][2],
                   float wsl) {
    // rows whose chunks hold the NaN scale code
    uint32_t nan_rows = 0;
    if (m0 == 0) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint64_t nl = 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) nl |= nan_scale_lanes(sc[g][r]);
#pragma unroll
        for (int j = 0; j < 4; ++j) nan_rows |= (uint32_t)((nl & (0x1111111111111111ull << j)) != 0) << (4 * g + j);
      }
    }

    float acc[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const u32x4 wv = stage_read(g, r);
        f32x4_v c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x4_t hb = as_bf16x4(hv[r][m >> 1].v[2 * (m & 1)], hv[r][m >> 1].v[2 * (m & 1) + 1]);
          c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(hb, e4m3x4_to_bf16x4(wv.v[m]), c, 0, 0, 0);
        }
        // lane 4b + j, register i: chunk b of row 4g + j against slot column i
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] += apply_e8m0(c[i], sc[g][r], kbias[r]);
      }
      // round by round: the compiler would otherwise convert every round's
      // rows first and hold them all (128 VGPRs at I = 768 instead of ~100)
      __builtin_amdgcn_sched_barrier(0);
    }
    // sum the 16 chunks: values v = (g, i); lanes 32..63 keep g = 1, then
    // odd rows keep i = 2, 3; the 4 lanes of each (g, i pair, j) hold the sum
    float v[8];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * g + i] = acc[g][i];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      permlane32_swap(v[t], v[t + 4]);
      v[t] += v[t + 4];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      permlane16_swap(v[t], v[t + 2]);
      v[t] += v[t + 2];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v[t] += dpp<0x128>(v[t]);   // row_ror:8: lane ^ 8 within the row
      v[t] += dpp<0x124>(v[t]);   // row_ror:4: with the above, the 4 lanes l, l+4, l+8, l+12 of the row
    }
    // slot ids and router weights of the 4 columns (lanes 0..3 hold them)
    uint32_t s_id[4];
    float s_w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_id[i] = (uint32_t)__builtin_amdgcn_readlane((int)sl, i);
      s_w[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wsl), i));
    }
    if ((lane & 12) == 0) {   // lane 32 g + 16 p + j writes rows 4 g + j of slot columns 2 p, 2 p + 1
      const int g = lane >> 5, p = (lane >> 4) & 1;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i = 2 * p + t;
        if (m0 + i < count) {
          const uint32_t s = i == 0 ? s_id[0] : (i == 1 ? s_id[1] : (i == 2 ? s_id[2] : s_id[3]));
          const float ww = i == 0 ? s_w[0] : (i == 1 ? s_w[1] : (i == 2 ? s_w[2] : s_w[3]));
          contrib[s * RO + 4 * g + lj] = ww * v[t];
        }
      }
    }
    // every slot of the unit carries the unit's NaN rows
    if (m0 == 0 && lane < count) nanmask[si.sorted[first + lane] & 0xFFFFu] = nan_rows;
  };
  auto process = [&](int un) {
    int e, first, count;   // slots si.sorted[first .. first + count), count 1 .. kDownMfmaUnitSlots
    si.unit(un, e, first, count);
    (void)e;
    uint32_t sl0 = 0, sl1 = 0;
    u32x4 hv0[NR][2], hv1[NR][2];
    float w0 = 0.0f, w1 = 0.0f;
    load_group(first, count, 0, sl0, hv0, w0);
    if (count > 4) load_group(first, count, 4, sl1, hv1, w1);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t sc[2][NR];
    scale_codes(sc);
    group(first, count, 0, sc, sl0, hv0, w0);
    if (count > 4) group(first, count, 4, sc, sl1, hv1, w1);
  };

  // Units are handed out as wavefronts come free.  The first unit is
  // processed outside the loop and its rows are loaded unconditionally (a
  // wavefront without a unit reads rows it will not use), so no row register
  // is merged across a branch or carried around the loop.
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
