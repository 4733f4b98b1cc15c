// Expert index of a decode batch's B*k routed slots, built by one workgroup in
// LDS (used by the expert-grouped kernels): the slots grouped by expert, and
// the routed experts' slots cut into work units of at most ch slots (so that
// an expert shared by many tokens is spread over several wavefronts or
// workgroups).
//
// Steps: every thread requests the ids of its slots first; per-expert counts
// with LDS atomics; wavefront 0 turns them into range starts and work units in
// one pass -- lane l owns the EPL = ceil(E/64) consecutive experts from l*EPL,
// so two wave-wide scans (slots, units) cover every expert; every slot is
// then dropped into its expert's range with an LDS atomic, in an order that
// depends on timing.  A kernel whose outputs of one unit come from that
// unit's slots alone, with every unit handled inside the workgroup, can take
// that order as it is (each slot's result is computed from the slot alone).
// With STABLE, the ranges of experts with more than ch slots -- the ones cut
// into several units -- are put into slot order (each such slot counts the
// smaller slot indices in its range), so that every workgroup cuts them into
// the same units: needed when the units of one expert are shared out over
// several workgroups.
#pragma once

#include "prims.hpp"

namespace moe {

constexpr int kSortMaxSlots = 1024;     // B*k limit
constexpr int kSortMaxExperts = 1024;   // E limit (per-expert LDS counters)

__host__ __device__ constexpr int a16(int n) { return (n + 15) & ~15; }
// LDS bytes: slots by expert [S] | work units [S] | range ends [E] | counts [E] | arrival [S] | 4 counters.
// Only the first two are read after the build; a kernel may reuse the rest
// (from slot_index_live_bytes on) once every thread has passed a barrier
// after build_slot_index returns.
__host__ __device__ constexpr int slot_index_lds_bytes(int E, int S) { return 2 * a16(4 * E) + 3 * a16(4 * S) + 16; }
__host__ __device__ constexpr int slot_index_live_bytes(int S) { return 2 * a16(4 * S); }

struct SlotIndex {
  int* end_;         // end of expert e's range in `sorted` (its start is end_[e] - count_[e])
  int* count_;       // slots of expert e
  uint32_t* sorted;  // slot | token << 16, grouped by expert
  uint32_t* units;   // work units: expert | first << 10 | count << 21 (its slots are sorted[first .. first + count))
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

// Build the index of `slots` >= 1 slots (ids[s], s = b*k + j) with NT threads.
template <int NT, bool STABLE>
__device__ SlotIndex build_slot_index(uint8_t* lds, const int32_t* __restrict__ ids, int slots, int E, int k, int ch) {
  constexpr int J = (kSortMaxSlots + NT - 1) / NT;   // slots per thread, enough for kSortMaxSlots
  SlotIndex o;
  o.ch = ch;
  o.sorted = reinterpret_cast<uint32_t*>(lds);
  o.units = o.sorted + a16(4 * slots) / 4;
  o.end_ = reinterpret_cast<int*>(lds + slot_index_live_bytes(slots));
  o.count_ = reinterpret_cast<int*>(lds + slot_index_live_bytes(slots) + a16(4 * E));
  uint32_t* arrival = reinterpret_cast<uint32_t*>(lds + slot_index_live_bytes(slots) + 2 * a16(4 * E));
  int* misc = reinterpret_cast<int*>(arrival + a16(4 * slots) / 4);   // 1: invalid slots, 2: units, 3: split experts
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);
  int sid[J];   // expert of slot tid + NT j; -1 for an invalid id or past the last slot
#pragma unroll
  for (int j = 0; j < J; ++j)
    sid[j] = (int)__builtin_bit_cast(
        uint32_t, __builtin_amdgcn_raw_buffer_load_b32(idr, (uint32_t)min(tid + NT * j, slots - 1) * 4u, 0, 0));
  for (int i = tid; i < E; i += NT) o.count_[i] = 0;
  if (tid < 4) misc[tid] = 0;
  __syncthreads();
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
    if (sid[j] >= 0) atomicAdd(&o.count_[sid[j]], 1);
  }
  __syncthreads();
  if (tid < 64) {   // counts -> range starts and work units, experts in ascending order
    const int epl = (E + 63) >> 6;
    const int e0 = lane * epl, e1 = min(e0 + epl, E);
    int cnt = 0, nun = 0;
    for (int e = e0; e < e1; ++e) {
      const int c = o.count_[e];
      cnt += c;
      nun += (c + ch - 1) / ch;
    }
    const int ic = wave_incl_scan(cnt), iu = wave_incl_scan(nun);
    int start = ic - cnt, un = iu - nun;
    bool split = false;
    for (int e = e0; e < e1; ++e) {
      const int c = o.count_[e];
      o.end_[e] = start;   // start, for now
      for (int i = 0; i * ch < c; ++i)
        o.units[un++] = (uint32_t)e | ((uint32_t)(start + i * ch) << 10) | ((uint32_t)min(ch, c - i * ch) << 21);
      start += c;
      split |= c > ch;
    }
    if (lane == 63) misc[2] = iu;
    if (STABLE && __builtin_amdgcn_ballot_w64(split) != 0 && lane == 0) misc[3] = 1;
  }
  __syncthreads();
  // into the expert's range; start[e] -> end[e] (the ranges of split experts
  // via `arrival`, to be put into slot order below)
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int sl = tid + NT * j;
    if (sid[j] >= 0) {
      const int pos = atomicAdd(&o.end_[sid[j]], 1);
      if (STABLE && o.count_[sid[j]] > ch) arrival[pos] = (uint32_t)sl;
      else o.sorted[pos] = (uint32_t)sl | ((uint32_t)(sl / k) << 16);
    }
  }
  __syncthreads();
  if (STABLE && __builtin_amdgcn_readfirstlane(misc[3]) != 0) {   // some expert is cut into several units
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (sid[j] >= 0 && o.count_[sid[j]] > ch) {
        const int sl = tid + NT * j, e = sid[j];
        const int b1 = o.end_[e], b0 = b1 - o.count_[e];
        int rank = 0;
        for (int i = b0; i < b1; ++i) rank += arrival[i] < (uint32_t)sl;
        o.sorted[b0 + rank] = (uint32_t)sl | ((uint32_t)(sl / k) << 16);
      }
    }
    __syncthreads();
  }
  o.n_bad = __builtin_amdgcn_readfirstlane(misc[1]);
  o.n_units = __builtin_amdgcn_readfirstlane(misc[2]);
  return o;
}

}  // namespace moe
