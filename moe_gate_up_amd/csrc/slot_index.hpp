// Expert index of a decode batch's B*k routed slots, built by one workgroup in
// LDS (used by the expert-grouped kernels): the slots sorted by expert, in
// slot order within each expert, and the routed experts' slots cut into work
// units of at most ch slots (so that an expert shared by many tokens is
// spread over several wavefronts or workgroups).
//
// Steps: per-expert counts with LDS atomics; wavefront 0 turns them into
// starts (one wave-wide scan per 64 experts) and lists the routed experts in
// ascending order and their work units; every slot is dropped into its
// expert's range with an LDS atomic (arbitrary order), then moved to its rank
// among that range's slots (the number of smaller slot indices in it), which
// puts each range in slot order.  The result -- and every sum built by
// walking it -- is the same on every run.  The ranking reads each slot's
// whole range once, so a range shared by n slots costs n reads per slot.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kSortMaxSlots = 1024;     // B*k limit
constexpr int kSortMaxExperts = 1024;   // E limit (per-expert LDS counters)

__host__ __device__ constexpr int a16(int n) { return (n + 15) & ~15; }
// LDS bytes: ends [E] | routed experts [min(E, S)] | arrival order [S] | sorted [S] | work units [S] | 4 counters
__host__ __device__ constexpr int slot_index_lds_bytes(int E, int S) {
  return a16(4 * E) + a16(4 * (E < S ? E : S)) + 3 * a16(4 * S) + 16;
}

struct SlotIndex {
  int* end_;         // end of expert e's range in `sorted` (its start is end_[e - 1], 0 for e = 0)
  int* used;         // routed experts, ascending
  uint32_t* sorted;  // slot | token << 16, grouped by expert, slot order within an expert
  uint32_t* units;   // work units: expert | first << 10 | count << 21 (its slots are sorted[first .. first + count))
  int n_used;        // routed experts
  int n_units;       // sum over routed experts of ceil(count / ch)
  int n_bad;         // slots whose id is outside [0, E)
  int ch;            // slots per work unit

  // expert of work unit n
  __device__ int unit_expert(int n) const { return __builtin_amdgcn_readfirstlane((int)(units[n] & 0x3FFu)); }
  // work unit n: its expert, the position of its first slot in `sorted`, and its slot count (1 .. ch)
  __device__ void unit(int n, int& e, int& first, int& count) const {
    const uint32_t v = (uint32_t)__builtin_amdgcn_readfirstlane((int)units[n]);   // one LDS read
    e = (int)(v & 0x3FFu);
    first = (int)((v >> 10) & 0x7FFu);
    count = (int)(v >> 21);
  }
};

template <int NT>
__device__ SlotIndex build_slot_index(uint8_t* lds, const int32_t* __restrict__ ids, int slots, int E, int k, int ch) {
  constexpr int J = (kSortMaxSlots + NT - 1) / NT;   // slots per thread, enough for kSortMaxSlots
  SlotIndex o;
  o.ch = ch;
  o.end_ = reinterpret_cast<int*>(lds);
  o.used = reinterpret_cast<int*>(lds + a16(4 * E));
  uint32_t* arrival = reinterpret_cast<uint32_t*>(lds + a16(4 * E) + a16(4 * min(E, slots)));
  o.sorted = arrival + a16(4 * slots) / 4;
  o.units = o.sorted + a16(4 * slots) / 4;
  int* misc = reinterpret_cast<int*>(o.units + a16(4 * slots) / 4);
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  for (int i = tid; i < E; i += NT) o.end_[i] = 0;
  if (tid < 4) misc[tid] = 0;
  __syncthreads();
  const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);
  int sid[J];   // expert of slot tid + NT j; -1 for an invalid id or past the last slot
#pragma unroll
  for (int j = 0; j < J; ++j)
    sid[j] = (int)__builtin_bit_cast(
        uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)min(tid + NT * j, slots - 1) * 4u, 0, 0));
  // used unconditionally here, so the compiler cannot sink each load into the
  // branch that uses it (which serialised their latencies)
#pragma unroll
  for (int j = 0; j < J; ++j) asm volatile("" : "+v"(sid[j]));
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int sl = tid + NT * j;
    const bool real = sl < slots, ok = (unsigned)sid[j] < (unsigned)E;
    if (real && !ok) atomicAdd(&misc[1], 1);
    sid[j] = real && ok ? sid[j] : -1;
    if (sid[j] >= 0) atomicAdd(&o.end_[sid[j]], 1);
  }
  __syncthreads();
  if (tid < 64) {   // counts -> starts; the routed experts in ascending order and their work units
    int carry = 0, nu = 0, nun = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? o.end_[e] : 0;
      const int nc = (c + ch - 1) / ch;   // work units of expert e
      const int incl = wave_incl_scan(c), uincl = wave_incl_scan(nc);
      const int start = carry + incl - c;
      if (e < E) o.end_[e] = start;   // start, for now
      const uint64_t m = __builtin_amdgcn_ballot_w64(c > 0);
      if (c > 0) {
        o.used[nu + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = e;
        for (int i = 0; i < nc; ++i)
          o.units[nun + uincl - nc + i] =
              (uint32_t)e | ((uint32_t)(start + i * ch) << 10) | ((uint32_t)min(ch, c - i * ch) << 21);
      }
      nu += __builtin_popcountll(m);
      carry += __builtin_amdgcn_readlane(incl, 63);
      nun += __builtin_amdgcn_readlane(uincl, 63);
    }
    if (lane == 0) {
      misc[0] = nu;
      misc[2] = nun;
    }
  }
  __syncthreads();
  // into the expert's range in arrival order; start[e] -> end[e]
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (sid[j] >= 0) arrival[atomicAdd(&o.end_[sid[j]], 1)] = (uint32_t)(tid + NT * j);
  __syncthreads();
  // to its rank within the range: slot order
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (sid[j] >= 0) {
      const int sl = tid + NT * j, e = sid[j];
      const int b0 = e > 0 ? o.end_[e - 1] : 0, b1 = o.end_[e];
      int rank = 0;
      for (int i = b0; i < b1; ++i) rank += arrival[i] < (uint32_t)sl;
      o.sorted[b0 + rank] = (uint32_t)sl | ((uint32_t)(sl / k) << 16);
    }
  }
  __syncthreads();
  o.n_used = __builtin_amdgcn_readfirstlane(misc[0]);
  o.n_bad = __builtin_amdgcn_readfirstlane(misc[1]);
  o.n_units = __builtin_amdgcn_readfirstlane(misc[2]);
  return o;
}

}  // namespace moe
