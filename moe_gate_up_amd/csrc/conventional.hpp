// The conventional, expert-centric MoE decode path, built on the GPU as the
// A/B comparison for warp decode (blog post "warp decode", sections "The
// traditional MoE path", "Stage elimination", "Eliminating padding",
// "Eliminating scatter and combine", "Eliminating buffers" and "Accuracy
// improvement").  It computes the same layer the way an expert-centric
// pipeline does, stage by stage, through device buffers:
//   1. route:   count the slots per expert, pad each count to a power of two,
//               lay the experts' token lists out back to back (row -> slot,
//               row -> expert, slot -> row);
//   2. quant x: x to MXFP8 (E4M3 codes, one E8M0 scale per 32 along H);
//   3. scatter: the quantised activations copied into the expert-major
//               gather buffer, one row per padded list entry (padding rows 0);
//   4. gate/up: per row, SiLU(gate) * up against the row's expert, rounded to
//               bf16 into an expert-major intermediate buffer;
//   5. quant h: the intermediate to MXFP8 (blocks of 32 along I);
//   6. down:    per row, the down projection, rounded to bf16 into the
//               per-expert output buffer (B*k rows of H);
//   7. combine: y[b] = bf16(sum_j w[b,j] * out[row(b,j)]).
// Padding rows are computed like real ones (that is the cost of padding) and
// never read by the combine.  The GEMM stages use the same MXFP8 decode and
// bf16 dot2 arithmetic as the warp-decode kernels, with the activation block
// scale added to the weight block scale (exact power-of-two products).
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kConvMaxSlots = 1024;   // B*k limit (one workgroup routes)

// ---------------------------------------------------------------- MXFP8 encode
// E4M3 code of a >= 0 (already saturated to <= 448), rounded to nearest even.
__device__ __forceinline__ uint32_t e4m3_code(float a) {
  if (a < 0.015625f) {   // below 2^-6: subnormal, steps of 2^-9
    return (uint32_t)__builtin_rintf(a * 512.0f);   // 8 -> 0x08, the smallest normal
  }
  uint32_t bits = __builtin_bit_cast(uint32_t, a);
  bits += 0x7FFFFu + ((bits >> 20) & 1u);   // round the mantissa to 3 bits, ties to even
  const int ex = (int)(bits >> 23) - 127;   // -6 .. 8
  return ((uint32_t)(ex + 7) << 3) | ((bits >> 20) & 7u);
}

// One 32-element block of bf16 values -> 32 E4M3 codes + 1 E8M0 scale.  The
// scale is 2^(floor(log2 amax) - 8), so the largest magnitude maps to [256,
// 512) and saturates at 448; an all-zero block gets code 127 (2^0).  A scale
// below 2^-127 (amax < 2^-118) is clamped to 2^-127.
__device__ __forceinline__ void mx_quant_block(const uint16_t* src, uint8_t* codes, uint8_t* scale) {
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = __builtin_bit_cast(float, (uint32_t)src[i] << 16);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  int sexp = 0;   // scale exponent
  if (amax > 0.0f) {
    const int e = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
    const int fl = e == 0 ? -127 : e - 127;   // floor(log2 amax) for normals; subnormal bf16 never reaches here in practice
    sexp = max(fl - 8, -127);
  }
  *scale = (uint8_t)(sexp + 127);
  const float inv = __builtin_ldexpf(1.0f, -sexp);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float a = fminf(fabsf(v[i]) * inv, 448.0f);
    codes[i] = (uint8_t)(e4m3_code(a) | (v[i] < 0.0f ? 0x80u : 0u));
  }
}

// ---------------------------------------------------------------- 1. route
// A list of c tokens padded to the next power of two (0 stays 0).
__host__ __device__ constexpr int pow2_pad(int c) {
  int p = 1;
  while (p < c) p <<= 1;
  return c == 0 ? 0 : p;
}

// meta: counts [E] | padded offsets [E] | (unused) [E] | P, the padded total.
// Pmax = 2 * B*k bounds P (a count c pads to less than 2c).
__global__ __launch_bounds__(1024) void conv_route_kernel(const int32_t* __restrict__ ids, int slots, int E, int Pmax,
                                                          int* __restrict__ meta, int* __restrict__ row_slot,
                                                          int* __restrict__ row_expert, int* __restrict__ slot_row) {
  __shared__ int cnt[kConvMaxSlots], off[kConvMaxSlots], tot;
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < E; i += 1024) cnt[i] = 0;
  for (int p = tid; p < Pmax; p += 1024) row_slot[p] = -1;
  __syncthreads();
  const int e = tid < slots ? ids[tid] : -1;
  const bool ok = tid < slots && (unsigned)e < (unsigned)E;
  if (ok) atomicAdd(&cnt[e], 1);
  __syncthreads();
  if (tid < 64) {   // padded counts (next power of two) -> offsets
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int x = e0 + lane;
      const int c = x < E ? cnt[x] : 0;
      const int pcc = pow2_pad(c);
      int incl = pcc;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        incl += lane >= d ? t : 0;
      }
      if (x < E) {
        off[x] = carry + incl - pcc;
        meta[E + x] = carry + incl - pcc;
        meta[x] = c;
      }
      carry += __shfl(incl, 63);
    }
    if (lane == 0) tot = carry;
  }
  __syncthreads();
  if (tid == 0) meta[3 * E] = tot;
  // padding rows belong to their expert too
  for (int x = tid; x < E; x += 1024) {
    const int pcc = pow2_pad(cnt[x]);
    for (int i = 0; i < pcc; ++i) row_expert[off[x] + i] = x;
  }
  __syncthreads();
  if (tid < slots) {
    if (ok) {
      const int p = off[e] + atomicAdd(&cnt[e], -1) - 1;   // any order within the list
      row_slot[p] = tid;
      slot_row[tid] = p;
    } else {
      slot_row[tid] = -1;
    }
  }
}

// ---------------------------------------------------------------- 2./5. quant
// rows x n bf16 -> codes [rows, n] + scales [rows, n/32]; one thread per block.
// Rows at or beyond *nrows (when given) are skipped.
__global__ __launch_bounds__(256) void conv_quant_kernel(const uint16_t* __restrict__ src, int rows, int n,
                                                         const int* __restrict__ nrows, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int nb = n >> 5;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)rows * nb) return;
  const int r = (int)(t / nb), b = (int)(t - (long long)r * nb);
  if (nrows && r >= *nrows) return;
  mx_quant_block(src + (size_t)r * n + 32 * b, codes + (size_t)r * n + 32 * b, scales + (size_t)r * nb + b);
}

// ---------------------------------------------------------------- 3. scatter
// gather buffer row p = quantised x of the token of slot row_slot[p] (zeros for padding)
__global__ __launch_bounds__(256) void conv_scatter_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                           const int* __restrict__ row_slot, const int* __restrict__ meta,
                                                           int E, int Pmax, int H, int k, uint8_t* __restrict__ xg,
                                                           uint8_t* __restrict__ xgs) {
  const int per_row = H / 16 + H / 32;   // 16-byte code chunks, then scale bytes
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)Pmax * per_row) return;
  const int p = (int)(t / per_row), i = (int)(t - (long long)p * per_row);
  if (p >= meta[3 * E]) return;
  const int s = row_slot[p];
  const int b = s / k;
  if (i < H / 16) {
    u32x4 v = {{0u, 0u, 0u, 0u}};
    if (s >= 0) v = *reinterpret_cast<const u32x4*>(xq + (size_t)b * H + 16 * i);
    *reinterpret_cast<u32x4*>(xg + (size_t)p * H + 16 * i) = v;
  } else {
    const int j = i - H / 16;
    xgs[(size_t)p * (H / 32) + j] = s >= 0 ? xs[(size_t)b * (H / 32) + j] : (uint8_t)127;
  }
}

// ---------------------------------------------------------------- 4./6. grouped GEMV rows
// One wavefront per (tile of R rows of the weight, gather-buffer row p):
// out[p, n] for n in the tile, against expert row_expert[p].  Activations are
// MXFP8 (codes + scales along the reduction); each 16-element partial is
// scaled by 2^(weight scale + activation scale - 254).  SWIGLU: two weight
// tensors, out = SiLU(gate) * up; else out = the dot product.  Passes of
// 1024 elements over the reduction K as in the warp-decode kernels.
template <int NP, int R, bool SWIGLU, int CP>
__global__ __launch_bounds__(256) void conv_gemv_kernel(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ as,
                                                        const int* __restrict__ row_expert, const int* __restrict__ meta,
                                                        const uint8_t* __restrict__ w0, const uint8_t* __restrict__ s0,
                                                        const uint8_t* __restrict__ w1, const uint8_t* __restrict__ s1,
                                                        uint16_t* __restrict__ out, int E, int N, int K, int Pmax,
                                                        int n_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(xcd_contiguous_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6));
  if (wave >= n_tiles * Pmax) return;
  const int tile = __builtin_amdgcn_readfirstlane(wave / Pmax);
  const int p = wave - tile * Pmax;
  if (p >= __builtin_amdgcn_readfirstlane(meta[3 * E])) return;
  const int e = __builtin_amdgcn_readfirstlane(row_expert[p]);
  const int n0 = tile * R;
  const int nblk = K >> 5;
  uint32_t off[NP];
  int bias[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    const int o = 1024 * c + 16 * lane;
    off[c] = (uint32_t)min(o, K - 16);
    bias[c] = o < K ? -254 : 2 * kDeadChunk;   // dead: far below -2 * 255, so the product scale is still 0
  }
  const uint32_t wbytes = (uint32_t)E * (uint32_t)N * (uint32_t)K;
  const rsrc_t ar = make_rsrc(aq, (uint64_t)Pmax * K), asr = make_rsrc(as, (uint64_t)Pmax * nblk);
  const rsrc_t r0 = make_rsrc(w0, wbytes), rs0 = make_rsrc(s0, wbytes / 32);
  const rsrc_t r1 = make_rsrc(SWIGLU ? w1 : w0, wbytes), rs1 = make_rsrc(SWIGLU ? s1 : s0, wbytes / 32);

  u32x4 a[NP];
  uint32_t asc[NP];
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    a[c] = bload16(ar, off[c], (uint32_t)p * (uint32_t)K);
    asc[c] = bload8(asr, off[c] >> 5, (uint32_t)p * (uint32_t)nblk);
  }
  u32x4 g[R][NP], u[R][NP];
  uint32_t gs[R][NP], us[R][NP];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)(e * N + min(n0 + r, N - 1));
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      g[r][c] = bload16<CP>(r0, off[c], row * (uint32_t)K);
      gs[r][c] = bload8<CP>(rs0, off[c] >> 5, row * (uint32_t)nblk);
      if constexpr (SWIGLU) {
        u[r][c] = bload16<CP>(r1, off[c], row * (uint32_t)K);
        us[r][c] = bload8<CP>(rs1, off[c] >> 5, row * (uint32_t)nblk);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  float v[2 * R];
#pragma unroll
  for (int i = 0; i < 2 * R; ++i) v[i] = 0.0f;
  uint64_t nan_rows = 0;
#pragma unroll
  for (int c = 0; c < NP; ++c) {
    u32x4 xa[2];   // the lane's 16 activation codes as bf16 pairs
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      xa[d >> 1].v[2 * (d & 1)] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2(a[c].v[d], false));
      xa[d >> 1].v[2 * (d & 1) + 1] = __builtin_bit_cast(uint32_t, e4m3x2_to_bf16x2(a[c].v[d], true));
    }
    const int ab = bias[c] + (int)asc[c];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      v[r] += apply_e8m0(chunk_dot(g[r][c], xa, 0.0f), gs[r][c], ab);
      uint64_t nl = nan_scale_lanes(gs[r][c]);
      if constexpr (SWIGLU) {
        v[R + r] += apply_e8m0(chunk_dot(u[r][c], xa, 0.0f), us[r][c], ab);
        nl |= nan_scale_lanes(us[r][c]);
      }
      nan_rows |= (uint64_t)(nl != 0) << r;
    }
  }
  const float tot = wave_reduce_scatter<2 * R>(v, lane);
  float lo = tot, hi = tot;
  permlane32_swap(lo, hi);   // hi (lanes 0..31) = value R + r
  int r_out = -1;
#pragma unroll
  for (int r = 0; r < R; ++r) r_out = (lane == scatter_lane<2 * R>(r)) ? r : r_out;
  if (r_out >= 0 && n0 + r_out < N) {
    const bool nan_out = (nan_rows >> r_out) & 1;
    const float res = SWIGLU ? silu(tot) * hi : tot;
    out[(size_t)p * N + n0 + r_out] = f32_to_bf16_rne(nan_out ? qnan() : res);
  }
}

// ---------------------------------------------------------------- 7. combine
// y[b, o] = bf16(sum_j w[b,j] * out[slot_row[b*k + j], o]); NaN if a slot has an invalid id.
__global__ __launch_bounds__(256) void conv_combine_kernel(const uint16_t* __restrict__ ob, const int* __restrict__ slot_row,
                                                           const float* __restrict__ tw, uint16_t* __restrict__ y,
                                                           int B, int H, int k) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)B * H) return;
  const int b = (int)(t / H), o = (int)(t - (long long)b * H);
  float acc = 0.0f;
  bool bad = false;
  for (int j = 0; j < k; ++j) {
    const int p = slot_row[b * k + j];
    if (p < 0) {
      bad = true;
      continue;
    }
    acc = fmaf(tw[b * k + j], __builtin_bit_cast(float, (uint32_t)ob[(size_t)p * H + o] << 16), acc);
  }
  y[t] = f32_to_bf16_rne(bad ? qnan() : acc);
}

}  // namespace moe
