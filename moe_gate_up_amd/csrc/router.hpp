// Top-k router step in front of the layer.  The blog post ("warp decode",
// section "The traditional MoE path") routes each token to a few of many
// experts (8 of 128 in one layer) and gives no more detail; the step here is
// the plain top-k router: from one FP32 logit per expert, token b keeps its
// k largest logits, largest first and the lower expert id first among equal
// logits, and weights them with the softmax of the kept logits (equal to the
// softmax over all E renormalised over the kept k).
//
// One 64-lane wavefront routes one token, with no LDS: lane l holds the
// logits of experts l, l + 64, ... as order-preserving unsigned keys.  Each
// of the k selections is one round: the wave-wide maximum of the keys still
// in play (DPP), one ballot per 64 experts for the lowest id holding it, and
// that key taken out of play.  Selection j lands in lane j, in order.  A
// round is a chain of dependent instructions (about 25), and one wavefront
// issues them one after another: the selection costs a few hundred cycles
// per token whichever kernel runs it.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kRouteMaxExperts = 1024;       // up to 16 logits per lane
constexpr int kRouteMaxK = 64;               // selection j lives in lane j
constexpr int kRouteFusedMaxExperts = 128;   // the gate/up prologue holds 2 logits per lane

// Order-preserving map of a finite FP32 value to an unsigned key: a < b as
// floats iff key(a) < key(b), and -0 and +0 share a key (they are equal).
__device__ __forceinline__ uint32_t route_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_key_value(uint32_t key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Sum over the 64 lanes in a fixed order, returned wave-uniform.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = row_sum16(v);
  v += dpp<0x142, 0xA>(v);
  v += dpp<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum over the 64 lanes, returned wave-uniform.  A lane that a DPP
// operation does not write reads 0, the identity of an unsigned maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  int x = (int)v;
  x = (int)max((uint32_t)x, (uint32_t)dppi<0xB1>(x));         // quad_perm [1,0,3,2]
  x = (int)max((uint32_t)x, (uint32_t)dppi<0x4E>(x));         // quad_perm [2,3,0,1]
  x = (int)max((uint32_t)x, (uint32_t)dppi<0x141>(x));        // row_half_mirror
  x = (int)max((uint32_t)x, (uint32_t)dppi<0x140>(x));        // row_mirror: every lane has its row's max
  x = (int)max((uint32_t)x, (uint32_t)dppi<0x142, 0xA>(x));   // row_bcast:15 into rows 1 and 3
  x = (int)max((uint32_t)x, (uint32_t)dppi<0x143, 0xC>(x));   // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// The k selections of one token (k <= 64, k <= E <= 64 NV): lane j < k holds
// selection j (0 = the largest logit).
struct RouteSel {
  int id;         // lane j < k: expert of selection j
  uint32_t key;   // lane j < k: the key of its logit
};

// Selection of one token whose E logits start at `row`.  Ids are always in
// [0, E), whatever the logits hold.  All NV loads are issued before the first
// use (a buffer bounded to the row reads 0 past its end: no load is
// conditional).
template <int NV>
__device__ __forceinline__ RouteSel wave_select(const float* row, int E, int k, int lane) {
  const rsrc_t lr = make_rsrc(row, (uint64_t)E * 4);
  uint32_t key[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) key[v] = __builtin_amdgcn_raw_buffer_load_b32(lr, 4u * (uint32_t)(64 * v + lane), 0, 0);
  // used here, unconditionally: the compiler may not sink a load into the
  // branch of its use below (which would serialise their latencies)
#pragma unroll
  for (int v = 0; v < NV; ++v) asm volatile("" : "+v"(key[v]));
  // experts past E get key 0, real ones at least 1 (only the NaN patterns
  // 0xFFFFFFFF and 0xFFFFFFFE share key 1), and a selected one goes to 0:
  // while fewer than E are selected the maximum is >= 1 and belongs to an
  // expert still in play
#pragma unroll
  for (int v = 0; v < NV; ++v)
    key[v] = 64 * v + lane < E ? max(route_key(__builtin_bit_cast(float, key[v])), 1u) : 0u;
  RouteSel s{0, 0u};
  for (int j = 0; j < k; ++j) {
    uint32_t m = key[0];
#pragma unroll
    for (int v = 1; v < NV; ++v) m = max(m, key[v]);
    const uint32_t M = wave_max_u32(m);
    // the lowest id holding M: the first block of 64 experts with a hit, its lowest lane
    int best = 0;
    bool found = false;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(key[v] == M);
      if (!found && hit) {
        best = 64 * v + (int)__builtin_ctzll(hit);
        found = true;
      }
    }
    best = __builtin_amdgcn_readfirstlane(best);
    if (lane == j) {
      s.id = best;
      s.key = M;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) key[v] = (lane == (best & 63) && v == (best >> 6)) ? 0u : key[v];
  }
  return s;
}

// Expert of selection j (wave-uniform).
__device__ __forceinline__ int route_expert(const RouteSel& s, int j) { return __builtin_amdgcn_readlane(s.id, j); }

// Lane j < k: the routing weight of selection j, exp(l_j - l_0) / sum_i
// exp(l_i - l_0) over the k selections (l_0 is the largest); 0 elsewhere.
// The sum runs over the lanes in a fixed order.
__device__ __forceinline__ float route_weight(const RouteSel& s, int k, int lane) {
  const float top = route_key_value((uint32_t)__builtin_amdgcn_readlane((int)s.key, 0));
  const float ex = lane < k ? expf(route_key_value(s.key) - top) : 0.0f;
  return ex / wave_sum_f32(ex);
}

// Logits per lane for E experts: 1, 2, 4, 8 or 16.
__host__ __device__ constexpr int route_per_lane(int E) {
  return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
}

// One wavefront per token: ids [B,k] and weights [B,k] from logits [B,E]
// (E <= 64 NV).
template <int NV>
__global__ __launch_bounds__(256) void moe_route_w64(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                     float* __restrict__ tw, int B, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int b = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (b >= B) return;
  const RouteSel s = wave_select<NV>(logits + (size_t)b * E, E, k, lane);
  const float w = route_weight(s, k, lane);
  if (lane < k) {
    ids[(size_t)b * k + lane] = s.id;
    tw[(size_t)b * k + lane] = w;
  }
}

}  // namespace moe
