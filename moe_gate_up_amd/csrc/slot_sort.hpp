// Counting sort of a decode batch's B*k routed slots by expert, done by one
// workgroup in LDS (used by the expert-grouped kernels).  The scatter uses LDS
// atomics, so each expert's short segment is then put back in slot order by
// one thread: the result, and every sum built by walking it, is the same on
// every run.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kSortMaxSlots = 1024;     // B*k limit
constexpr int kSortMaxExperts = 1024;   // E limit (per-expert LDS counters)

__host__ __device__ constexpr int a16(int n) { return (n + 15) & ~15; }
// LDS bytes: per-expert counters [E] | routed experts [min(E, S)] | sorted slots [S] | 4 counters
__host__ __device__ constexpr int slot_sort_lds_bytes(int E, int S) {
  return a16(4 * E) + a16(4 * (E < S ? E : S)) + a16(4 * S) + 16;
}

struct SlotSort {
  int* cur;          // after the sort: end of expert e's range (its start is cur[e - 1], 0 for e = 0)
  int* used;         // routed experts, ascending
  uint32_t* sorted;  // slot | token << 16, grouped by expert
  int n_used;        // routed experts
  int n_bad;         // slots whose id is outside [0, E)

  __device__ int begin(int e) const { return e > 0 ? __builtin_amdgcn_readfirstlane(cur[e - 1]) : 0; }
  __device__ int end(int e) const { return __builtin_amdgcn_readfirstlane(cur[e]); }
};

// Sort by the NT threads of the workgroup (thread t owns slots t + NT j), in
// two phases so that a kernel can issue weight loads in between:
//  count():   per-expert counts, then (wavefront 0, one wave-wide scan per 64
//             experts) each expert's start and the routed experts in
//             ascending order -- enough to know which rows to read;
//  scatter(): the slots into their experts' ranges, each range put back in
//             slot order.
// Each phase ends with a barrier and leaves every thread the same view.  Keys
// are slot | token << 16 with token = slot / k increasing with the slot, so
// ordering keys orders slots.
template <int NT>
struct SlotSorter {
  static constexpr int J = kSortMaxSlots / NT;
  SlotSort o;
  int sid[J];   // expert of slot tid + NT j, -1 for an invalid id, -2 past the last slot
  int k;

  __device__ void count(uint8_t* lds, const int32_t* __restrict__ ids, int slots, int E, int k_) {
    k = k_;
    o.cur = reinterpret_cast<int*>(lds);
    o.used = reinterpret_cast<int*>(lds + a16(4 * E));
    o.sorted = reinterpret_cast<uint32_t*>(lds + a16(4 * E) + a16(4 * min(E, slots)));
    int* misc = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(o.sorted) + a16(4 * slots));
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    for (int i = tid; i < E; i += NT) o.cur[i] = 0;
    if (tid < 4) misc[tid] = 0;
    __syncthreads();
    const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);
    int v[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
      v[j] = (int)__builtin_bit_cast(
          uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)min(tid + NT * j, slots - 1) * 4u, 0, 0));
    // used unconditionally here, so the compiler cannot sink each load into the
    // branch that uses it (which serialised their latencies)
#pragma unroll
    for (int j = 0; j < J; ++j) asm volatile("" : "+v"(v[j]));
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int sl = tid + NT * j;
      sid[j] = sl < slots ? ((unsigned)v[j] < (unsigned)E ? v[j] : -1) : -2;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (sid[j] >= 0) atomicAdd(&o.cur[sid[j]], 1);
      else if (sid[j] == -1) atomicAdd(&misc[1], 1);
    }
    __syncthreads();
    if (tid < 64) {   // counts -> starts (exclusive scan), and the routed experts in ascending order
      int carry = 0, nu = 0;
      for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int c = e < E ? o.cur[e] : 0;
        int incl = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int t = __shfl_up(incl, d);
          incl += lane >= d ? t : 0;
        }
        if (e < E) o.cur[e] = carry + incl - c;
        const uint64_t m = __builtin_amdgcn_ballot_w64(c > 0);
        if (c > 0)
          o.used[nu + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = e;
        nu += __builtin_popcountll(m);
        carry += __shfl(incl, 63);
      }
      if (lane == 0) misc[0] = nu;
    }
    __syncthreads();
    o.n_used = __builtin_amdgcn_readfirstlane(misc[0]);
    o.n_bad = __builtin_amdgcn_readfirstlane(misc[1]);
  }

  __device__ void scatter() {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (sid[j] >= 0) {
        const int sl = tid + NT * j;
        o.sorted[atomicAdd(&o.cur[sid[j]], 1)] = (uint32_t)sl | ((uint32_t)(sl / k) << 16);
      }
    }
    __syncthreads();
    for (int u = tid; u < o.n_used; u += NT) {   // insertion sort of one expert's segment by slot
      const int e = o.used[u];
      const int b0 = e > 0 ? o.cur[e - 1] : 0, b1 = o.cur[e];
      for (int i = b0 + 1; i < b1; ++i) {
        const uint32_t key = o.sorted[i];
        int j = i - 1;
        for (; j >= b0 && o.sorted[j] > key; --j) o.sorted[j + 1] = o.sorted[j];
        o.sorted[j + 1] = key;
      }
    }
    __syncthreads();
  }
};

}  // namespace moe
