// Device primitives for the gfx950 (CDNA4) warp-decode kernels.
//
// - MXFP8 decode: E4M3 pairs become bf16 pairs with gfx950's
//   v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value is a bf16 value); the
//   E8M0 block scale, a power of two, multiplies the block's FP32 partial sum
//   once, which is exact barring overflow/underflow.
// - Dot products: v_dot2c_f32_bf16 multiplies two bf16 pairs and accumulates
//   in FP32, so one instruction does two multiply-adds on raw bf16 activations
//   with no bf16->FP32 unpacking.
// - Cross-lane sums of the R (or 2R) outputs of a wave are one reduce-scatter:
//   permlane32/permlane16 swaps across rows, DPP exchanges inside rows.  No
//   LDS traffic, no barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct alignas(16) u32x4 {
  uint32_t v[4];
};

// Buffer resources: a tensor's base address and byte size live in scalar
// registers and every load is base + per-lane 32-bit offset + wave-uniform
// 32-bit offset, so no per-lane 64-bit address arithmetic is needed.  (The
// third dword selects a 32-bit data format, as raw buffer loads on gfx9-family
// chips require.)  Offsets must stay below 2^32; the host checks tensor sizes.
// The range check (a load past the size reads zero) covers the per-lane
// offset only, not the wave-uniform one: a load that relies on it puts its
// whole offset in the per-lane operand.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// Cache policy operand of the buffer loads.  kStream sets the non-temporal
// bit (nt) of gfx950's loads, which marks the lines as streaming data.  The
// weight rows and their scale codes are read once per decode step and are in
// no cache at the next step; loaded this way every layer kernel ran faster on
// MI355X (H = 2048, I = 768, 32 tokens: layer 97.7 -> 90.3 us), presumably
// because they no longer displace what many workgroups re-read from L2 (the
// activations, the intermediate, the ids).
constexpr int kCached = 0;
constexpr int kStream = 2;

// 16 bytes at base + voff + soff.
template <int CP = kCached>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP);
  u32x4 o;
  o.v[0] = t[0]; o.v[1] = t[1]; o.v[2] = t[2]; o.v[3] = t[3];
  return o;
}

// One byte at base + voff + soff, zero-extended.
template <int CP = kCached>
__device__ __forceinline__ uint32_t bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, CP);
}

// s_waitcnt immediate that waits until at most n (< 64) vector-memory
// operations of the wave are outstanding, leaving the other counters alone.
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

// E4M3 bytes 0,1 (hi=false) or 2,3 (hi=true) of `word` -> bf16 pair (exact).
__device__ __forceinline__ bf16x2_t e4m3x2_to_bf16x2(uint32_t word, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// acc + a.x*b.x + a.y*b.y, FP32 accumulate.
__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

// Apply an E8M0 block scale to an FP32 partial sum: p * 2^(s + bias), one
// v_ldexp_f32 (exact, subnormal results included).  bias is -127 for a real
// chunk and kDeadChunk for a clamped duplicate, which makes its contribution
// zero.  The NaN code 0xFF is not representable this way: callers collect
// the lanes holding it with nan_scale_lanes() and force the output to NaN.
constexpr int kLiveChunk = -127;
constexpr int kDeadChunk = -512;
__device__ __forceinline__ float apply_e8m0(float p, uint32_t s, int bias) {
  return __builtin_ldexpf(p, (int)s + bias);
}
__device__ __forceinline__ uint64_t nan_scale_lanes(uint32_t s) { return __builtin_amdgcn_ballot_w64(s == 255u); }

// Dot product of 16 E4M3 weights (w: 16 bytes) with 16 bf16 activations
// (xa: 2 x 16 bytes), returned unscaled in FP32.
__device__ __forceinline__ float chunk_dot(const u32x4& w, const u32x4* xa, float acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // weights 4d..4d+3; activations are dwords 2d and 2d+1 of the 8
    acc = dot2(e4m3x2_to_bf16x2(w.v[d], false), as_bf16x2(xa[d >> 1].v[(2 * d) & 3]), acc);
    acc = dot2(e4m3x2_to_bf16x2(w.v[d], true), as_bf16x2(xa[d >> 1].v[(2 * d + 1) & 3]), acc);
  }
  return acc;
}

// DPP move of v; lanes in rows outside ROW_MASK read 0 (the identity of +).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes (lane l gets the sum of lanes 0..l):
// row_shr steps inside each 16-lane row, then row_bcast:15 / row_bcast:31 carry
// the rows' totals forward.  No LDS.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dppi<0x111>(v);        // row_shr:1
  v += dppi<0x112>(v);        // row_shr:2
  v += dppi<0x114>(v);        // row_shr:4
  v += dppi<0x118>(v);        // row_shr:8
  v += dppi<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dppi<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the row sum.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp<0x141>(v);   // row_half_mirror: quads 0<->1, 2<->3 of each 8-lane half
  v += dpp<0x140>(v);   // row_mirror: halves of the 16-lane row
  return v;
}

// Sum over all 64 lanes.  The total lands in every lane of row 3 (lanes 48..63);
// other rows hold partial sums.  row_bcast:15 adds row 0's sum into row 1 and
// row 2's into row 3; row_bcast:31 then adds lane 31 (rows 0+1) into row 3.
constexpr int kSumLane = 48;
__device__ __forceinline__ float wave_sum_row3(float v) {
  v = row_sum16(v);
  v += dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// gfx950 cross-row swaps.  v_permlane32_swap exchanges lanes 32..63 of a with
// lanes 0..31 of b; v_permlane16_swap exchanges the odd 16-lane rows of a with
// the even rows of b.  Written as inline assembly because the compiler's
// builtins for these instructions returned the new value of the first operand
// for both results (checked with an on-device lane probe); the s_nop gives
// the two wait states a VALU write needs before a permlane reads it.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// One halving step of a reduce-scatter inside 16-lane rows: lanes whose
// `bit` is clear keep the low half of the values, the others the high half,
// and each adds its DPP partner's copy of the half it keeps.
template <int CTRL, int N>
__device__ __forceinline__ void row_exchange(float (&v)[N], bool bit) {
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const float keep = bit ? v[j + N / 2] : v[j];
    const float send = bit ? v[j] : v[j + N / 2];
    v[j] = keep + dpp<CTRL>(send);
  }
}

// Reduce-scatter of V = 2^m values (V <= 16) over the 64 lanes of a wave:
// afterwards every lane holds the wave total of one value index.  The index
// bits are taken from lane bits 5, 4, 3, 2 (most significant first): lanes
// 32..63 vs 0..31 (permlane32), odd vs even rows (permlane16), then inside a
// row lane^8 (row_ror:8) and lane^7 (row_half_mirror); the remaining lane
// bits are summed over.  About 1.2 adds per value instead of 6 per value for
// separate sums.  scatter_lane<V>(i) is the lowest lane holding index i.
template <int V>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 16 && (V & (V - 1)) == 0, "V must be a power of two <= 16");
  if constexpr (V >= 2) {
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      permlane32_swap(v[j], v[j + V / 2]);
      v[j] += v[j + V / 2];
    }
  } else {
    float a = v[0], b = v[0];
    permlane32_swap(a, b);
    v[0] = a + b;
  }
  constexpr int V2 = V >= 2 ? V / 2 : 1;
  if constexpr (V2 >= 2) {
#pragma unroll
    for (int j = 0; j < V2 / 2; ++j) {
      permlane16_swap(v[j], v[j + V2 / 2]);
      v[j] += v[j + V2 / 2];
    }
  } else {
    float a = v[0], b = v[0];
    permlane16_swap(a, b);
    v[0] = a + b;
  }
  constexpr int V3 = V2 >= 2 ? V2 / 2 : 1;
  float w[V3];
#pragma unroll
  for (int j = 0; j < V3; ++j) w[j] = v[j];
  if constexpr (V3 >= 2) {
    row_exchange<0x128>(w, (lane & 8) != 0);   // row_ror:8: partner lane ^ 8
  } else {
    w[0] += dpp<0x128>(w[0]);
  }
  constexpr int V4 = V3 >= 2 ? V3 / 2 : 1;
  if constexpr (V4 >= 2) {
    float x2[V4];
#pragma unroll
    for (int j = 0; j < V4; ++j) x2[j] = w[j];
    row_exchange<0x141>(x2, (lane & 4) != 0);   // row_half_mirror: partner lane ^ 7
    w[0] = x2[0];
  } else {
    w[0] += dpp<0x141>(w[0]);
  }
  w[0] += dpp<0x4E>(w[0]);   // quad_perm [2,3,0,1]: lane ^ 2
  w[0] += dpp<0xB1>(w[0]);   // quad_perm [1,0,3,2]: lane ^ 1
  return w[0];
}

template <int V>
__host__ __device__ constexpr int scatter_lane(int idx) {
  int lane = 0, weight = V / 2, bit = 5;
  for (int s = 0; s < 4; ++s, weight /= 2, --bit)
    if (weight >= 1 && (idx & weight)) lane |= 1 << bit;
  return lane;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// SiLU(g) = g / (1 + e^-g).  A gate that overflowed FP32 to -inf gets the
// limit, -0 (the quotient would be -inf / inf = NaN); +inf stays +inf.
__device__ __forceinline__ float silu(float g) {
  return g == -__builtin_huge_valf() ? -0.0f : g / (1.0f + __expf(-g));
}

// MI355X dispatches workgroup g to XCD (g mod 8); each XCD has its own L2.
// Remap the hardware workgroup id to a logical one so that every XCD works
// through one contiguous range of logical workgroups: work that shares weight
// rows and is adjacent in logical order then shares one L2.  Bijective on
// [0, G) for any G.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous_block(int g, int G) {
  const int x = g % kXcds, i = g / kXcds;
  const int q = G / kXcds, rem = G % kXcds;
  return (x < rem) ? x * (q + 1) + i : rem * (q + 1) + (x - rem) * q + i;
}

__device__ __forceinline__ float qnan() { return __builtin_bit_cast(float, 0x7FC00000u); }

}  // namespace moe
