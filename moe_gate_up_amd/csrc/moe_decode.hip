// C ABI of the warp-decode MoE layer for gfx950: argument validation, launch
// shape selection and kernel launches.  The contract of every entry point is
// stated in include/moe_decode.h.
#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>

#include "moe_decode.h"
#include "down_grouped.hpp"
#include "down_grouped_mfma.hpp"   // the matrix-core down kernel's limits (the kernel itself: down_mfma.hip)
#include "conventional.hpp"
#include "gate_up.hpp"
#include "gate_up_grouped.hpp"
#include "gate_up_grouped_mfma.hpp"
#include "peak.hpp"
#include "host.hpp"
#include "router.hpp"

namespace {

using moe_host::DownLaunch;
using moe_host::kLdsPerCu;
using moe_host::kMaxDevices;
using moe_host::kMaxDownPasses;
using moe_host::kWavesPerBlock;
using moe_host::PerDeviceOnce;
constexpr int kMaxGateUpPasses = 8;   // H <= 8 passes of 1024 elements = 8192

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

int check_shape(int B, int H, int I, int E, int k) {
  if (B < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_SHAPE;
  if (H % 32 || I % 32) return MOE_ERR_SHAPE;
  if (H > kMaxGateUpPasses * 1024) return MOE_ERR_SHAPE;
  if ((long long)k * I > (long long)kMaxDownPasses * 1024) return MOE_ERR_SHAPE;
  // wave ids, slot indices and buffer offsets are 32-bit
  if ((long long)B * k * I >= (1LL << 31) || (long long)B * H >= (1LL << 31)) return MOE_ERR_SHAPE;
  if ((long long)E * I * H >= (1LL << 32)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// passes of 1024 elements (64 lanes x 16) over a reduction of n elements
int passes(long long n) { return (int)((n + 1023) / 1024); }

// ---------------------------------------------------------------- gate/up
// register budget: R rows x NCH passes x (gate + up) x 4 VGPRs of weights
constexpr bool gate_up_fits(int nch, int r) { return nch * r <= 16; }
bool gate_up_allowed(int nch, int r) {
  return (r == 1 || r == 2 || r == 4 || r == 8) && nch >= 1 && nch <= kMaxGateUpPasses && gate_up_fits(nch, r);
}

// Rows per wave from a graph-timed sweep on MI355X (H = 2048 and 4096): more
// rows per wave amortise the x slice and the reductions, but the grid must
// keep at least ~16K wavefronts to cover memory latency, and beyond
// R * passes = 8 the register file limits occupancy to two waves per SIMD,
// which measured slower.
int gate_up_default_rows(int B, int H, int I, int k) {
  const int nch = passes(H);
  const long long slots = (long long)B * k;
  int r = 8;
  while (r > 1 && (!gate_up_allowed(nch, r) || nch * r > 8 || slots * ((I + r - 1) / r) < 16384)) r /= 2;
  return r;
}

// The router step in front of gate/up: logits in, ids and routing weights out.
struct RouteIO {
  const float* logits;   // [B, E]
  int32_t* ids;          // [B, k]
  float* tw;             // [B, k]
  bool fuse;             // as the per-slot kernel's prologue (else the router kernel first)
};

// The router step is fused into the per-slot kernel while B*k <= 16: every
// workgroup selects its token's experts again (a few hundred dependent
// instructions, ~1.5 us), which beats a launch of its own (~2.9 us per layer)
// only while there are few workgroups per CU (graph-timed, H = 2048, I = 768,
// 128 experts, top-8: 1 token 13.9 vs 15.3 us per layer, 2 tokens 20.2 vs
// 21.8, 4 tokens 32.5 vs 32.6, 8 tokens 54.1 vs 52.1).  The fused kernel
// takes 2 rows per wavefront (fewer workgroups, fewer selections).
constexpr long long kRouteFusedMaxSlots = 16;
constexpr int kRouteFusedRows = 2;

// Router kernel: one wavefront per token, 4 tokens per workgroup.
template <int NV>
void launch_route_t(hipStream_t st, const RouteIO& ro, int B, int E, int k) {
  hipLaunchKernelGGL((moe::moe_route_w64<NV>), dim3((unsigned)((B + kWavesPerBlock - 1) / kWavesPerBlock)),
                     dim3(64 * kWavesPerBlock), 0, st, ro.logits, ro.ids, ro.tw, B, E, k);
}
void launch_route(hipStream_t st, const RouteIO& ro, int B, int E, int k) {
  switch (moe::route_per_lane(E)) {
    case 1: return launch_route_t<1>(st, ro, B, E, k);
    case 2: return launch_route_t<2>(st, ro, B, E, k);
    case 4: return launch_route_t<4>(st, ro, B, E, k);
    case 8: return launch_route_t<8>(st, ro, B, E, k);
    default: return launch_route_t<16>(st, ro, B, E, k);
  }
}

// Every gate/up launcher returns its number of workgroups and launches only
// when `go` is set (the plan query calls it with go = false).  With `ro` set
// the router step runs too: as the per-slot kernel's prologue if ro->fuse,
// else as the router kernel before it.
//
// Per-slot grid: one wavefront per (tile of R neurons, slot).  k % 4 == 0:
// the 4 wavefronts of a workgroup serve one token and share x[b] through LDS.
template <int NCH, int R, bool ROUTE>
void launch_gate_up_k(dim3 grid, hipStream_t st, const void* x, const int32_t* ids, const uint8_t* wg,
                      const uint8_t* sg, const uint8_t* wu, const uint8_t* su, void* h, int B, int H, int I, int E,
                      int k, int tiles, const RouteIO* ro) {
  const float* lg = ro ? ro->logits : nullptr;
  int32_t* io = ro ? ro->ids : nullptr;
  float* to = ro ? ro->tw : nullptr;
  if (k % 4 == 0)   // dynamic LDS: x[b], and with the router step the 4 slots' experts
    hipLaunchKernelGGL((moe::moe_gate_up_3d_batched_w64<NCH, R, true, ROUTE>), grid, dim3(64 * kWavesPerBlock),
                       (unsigned)(2 * H + (ROUTE ? 16 : 0)), st, static_cast<const uint16_t*>(x), ids, wg, sg, wu, su,
                       static_cast<uint16_t*>(h), B, H, I, E, k, tiles, lg, io, to);
  else
    hipLaunchKernelGGL((moe::moe_gate_up_3d_batched_w64<NCH, R, false, ROUTE>), grid, dim3(64 * kWavesPerBlock), 0,
                       st, static_cast<const uint16_t*>(x), ids, wg, sg, wu, su, static_cast<uint16_t*>(h), B, H, I,
                       E, k, tiles, lg, io, to);
}

template <int NCH, int R>
long long launch_gate_up_t(bool go, hipStream_t st, const void* x, const int32_t* ids, const uint8_t* wg,
                           const uint8_t* sg, const uint8_t* wu, const uint8_t* su, void* h, int B, int H, int I, int E,
                           int k, const RouteIO* ro) {
  static_assert(kWavesPerBlock == 4, "x sharing assumes 4 slots per workgroup");
  const int tiles = (I + R - 1) / R;
  const long long blocks = ((long long)tiles * B * k + kWavesPerBlock - 1) / kWavesPerBlock;
  if (!go || blocks * kWavesPerBlock >= (1LL << 31)) return blocks;
  const dim3 grid((unsigned)blocks);
  if (ro && ro->fuse) {
    launch_gate_up_k<NCH, R, true>(grid, st, x, ids, wg, sg, wu, su, h, B, H, I, E, k, tiles, ro);
  } else {
    if (ro) {
      launch_route(st, *ro, B, E, k);
      ids = ro->ids;
    }
    launch_gate_up_k<NCH, R, false>(grid, st, x, ids, wg, sg, wu, su, h, B, H, I, E, k, tiles, nullptr);
  }
  return blocks;
}

using GateUpLaunch = long long (*)(bool, hipStream_t, const void*, const int32_t*, const uint8_t*, const uint8_t*,
                                   const uint8_t*, const uint8_t*, void*, int, int, int, int, int, const RouteIO*);

template <int NCH, int R>
GateUpLaunch gate_up_fn() {
  if constexpr (gate_up_fits(NCH, R)) return launch_gate_up_t<NCH, R>;
  else return nullptr;
}

template <int NCH>
GateUpLaunch pick_gate_up_r(int r) {
  switch (r) {
    case 1: return gate_up_fn<NCH, 1>();
    case 2: return gate_up_fn<NCH, 2>();
    case 4: return gate_up_fn<NCH, 4>();
    case 8: return gate_up_fn<NCH, 8>();
  }
  return nullptr;
}

GateUpLaunch pick_gate_up(int nch, int r) {
  switch (nch) {
    case 1: return pick_gate_up_r<1>(r);
    case 2: return pick_gate_up_r<2>(r);
    case 3: return pick_gate_up_r<3>(r);
    case 4: return pick_gate_up_r<4>(r);
    case 5: return pick_gate_up_r<5>(r);
    case 6: return pick_gate_up_r<6>(r);
    case 7: return pick_gate_up_r<7>(r);
    case 8: return pick_gate_up_r<8>(r);
  }
  return nullptr;
}

// ---------------------------------------------------------------- gate/up, expert-grouped
// the rows are converted to bf16 once (they are reused for every slot):
// R x passes x 2 x 8 VGPRs
constexpr bool grouped_fits(int nch, int r) { return nch * r <= 8; }
bool grouped_allowed(int nch, int r, long long slots, int E) {
  return (r == 1 || r == 2 || r == 4 || r == 8) && nch >= 1 && nch <= kMaxGateUpPasses && grouped_fits(nch, r) &&
         slots <= moe::kGroupedMaxSlots && E <= moe::kGroupedMaxExperts;
}

// Persistent grid of at most 2048 workgroups (8 per CU of MI355X's 256, 4 of
// which fit at once) and never more than the largest possible number of work
// item pairs; dynamic LDS: the slot index and the staged activations.  From a
// graph-timed sweep at 32 and 64 tokens: 1024 workgroups are ~3 % slower;
// 3072-4096 are up to 2 % faster under uniform routing but up to 13 % slower
// under Zipf routing, where hot experts make some work items much longer.
#ifndef MOE_GROUPED_BLOCKS
#define MOE_GROUPED_BLOCKS 2048
#endif
constexpr long long kGroupedBlocks = MOE_GROUPED_BLOCKS;
//
// With the router step, the router kernel runs first and the grouped kernel
// reads the ids it wrote: every grouped workgroup needs every token's ids, so
// selecting them in each workgroup would repeat B selections per workgroup.
template <int NCH, int R>
long long launch_grouped_t(bool go, hipStream_t st, const void* x, const int32_t* ids, const uint8_t* wg,
                           const uint8_t* sg, const uint8_t* wu, const uint8_t* su, void* h, int B, int H, int I, int E,
                           int k, const RouteIO* ro) {
  const long long slots = (long long)B * k;   // work units (<= slots) x groups of 4 tiles
  const long long items_max = slots * (long long)((I + 4 * R - 1) / (4 * R));
  const long long pairs = (items_max + 1) / 2;   // a workgroup takes its items in pairs
  const long long blocks = pairs < kGroupedBlocks ? pairs : kGroupedBlocks;
  if (!go) return blocks;
  if (ro) {
    launch_route(st, *ro, B, E, k);
    ids = ro->ids;
  }
  hipLaunchKernelGGL((moe::moe_gate_up_expert_grouped_w64<NCH, R>), dim3((unsigned)blocks), dim3(64 * kWavesPerBlock),
                     (unsigned)moe::grouped_lds_bytes(E, (int)slots, H), st, static_cast<const uint16_t*>(x), ids, wg,
                     sg, wu, su, static_cast<uint16_t*>(h), B, H, I, E, k);
  return blocks;
}

template <int NCH, int R>
GateUpLaunch grouped_fn() {
  if constexpr (grouped_fits(NCH, R)) return launch_grouped_t<NCH, R>;
  else return nullptr;
}

template <int NCH>
GateUpLaunch pick_grouped_r(int r) {
  switch (r) {
    case 1: return grouped_fn<NCH, 1>();
    case 2: return grouped_fn<NCH, 2>();
    case 4: return grouped_fn<NCH, 4>();
    case 8: return grouped_fn<NCH, 8>();
  }
  return nullptr;
}

GateUpLaunch pick_grouped(int nch, int r) {
  switch (nch) {
    case 1: return pick_grouped_r<1>(r);
    case 2: return pick_grouped_r<2>(r);
    case 3: return pick_grouped_r<3>(r);
    case 4: return pick_grouped_r<4>(r);
    case 5: return pick_grouped_r<5>(r);
    case 6: return pick_grouped_r<6>(r);
    case 7: return pick_grouped_r<7>(r);
    case 8: return pick_grouped_r<8>(r);
  }
  return nullptr;
}

// Matrix-core grouped kernel: a persistent grid of one resident round of
// workgroups on MI355X's 256 CUs (a sweep of 384 to 1024 workgroups at 32 and
// 64 tokens with two per CU found exactly one resident round fastest, partial
// rounds up to 25 % slower); dynamic LDS: the slot index, two chunk buffers
// and the item's scale codes.  Work units of 8 slots halve the activation
// half of the chunk buffers; where that lets three workgroups share a CU
// (up to ~40 tokens at H = 2048, 128 experts) it is the faster choice (32
// tokens: 64.3 vs 65.8 us; 16 tokens: 47.9 vs 49.6; Zipf, 32 tokens: 49.0
// vs 49.9), otherwise units of 16 slots with two workgroups per CU (64
// tokens: 74.7 vs 75.8 us, Zipf 71.5 vs 77.1: an expert shared by more
// tokens is cut into fewer units, each of which reads its rows).
constexpr long long kMfmaCus = 256;
// LDS the residency count is computed against: three workgroups of 54,272
// bytes each (162,816 in all) did not fit one CU on MI355X, three of 53,760 did
constexpr int kLdsPerCuUsable = kLdsPerCu - 2048;
struct MfmaShape {
  int ch;          // slots per work unit: 8 or 16
  int lds;         // dynamic LDS bytes
  long long per_cu;
};
MfmaShape mfma_shape(int H, long long slots, int E) {
  const int l8 = moe::mfma_lds_bytes(E, (int)slots, H, 8);
  if (kLdsPerCuUsable / l8 >= 3) return {8, l8, 3};
  const int l16 = moe::mfma_lds_bytes(E, (int)slots, H, 16);
  const long long fit = kLdsPerCuUsable / l16;
  return {16, l16, fit > 2 ? 2 : (fit < 1 ? 1 : fit)};
}
bool mfma_allowed(int H, long long slots, int E) {
  return H % 2048 == 0 && H <= 8192 && slots <= moe::kSortMaxSlots && E <= moe::kSortMaxExperts;
}

// Largest dynamic LDS the matrix-core kernel takes within its limits (1024
// slots over 1024 experts at H = 8192: ~91 KB).  The kernel's attribute is set
// to it once per device, before the first launch on that device, and never
// changed afterwards: a per-call value would be process-wide state that a
// concurrent call could lower between another thread's set and its launch.
// Occupancy follows the LDS size each launch asks for, not this maximum.
constexpr int kMfmaMaxLds = moe::mfma_lds_bytes(moe::kSortMaxExperts, moe::kSortMaxSlots, 8192, moe::kMfmaColumns);
static_assert(kMfmaMaxLds <= kLdsPerCu, "the matrix-core kernel's largest LDS must fit one CU");

PerDeviceOnce g_gate_up_mfma_setup;

// hipSuccess once the attribute is in place on the current device.
hipError_t mfma_setup_current_device() {
  return g_gate_up_mfma_setup([] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&moe::moe_gate_up_grouped_mfma_w64),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaMaxLds);
  });
}

long long launch_mfma(bool go, hipStream_t st, const void* x, const int32_t* ids, const uint8_t* wg,
                      const uint8_t* sg, const uint8_t* wu, const uint8_t* su, void* h, int B, int H, int I, int E,
                      int k, const RouteIO* ro) {
  const long long slots = (long long)B * k;   // work units (<= slots) x groups of 16 neurons
  const long long items_max = slots * (long long)((I + moe::kMfmaRows - 1) / moe::kMfmaRows);
  const MfmaShape sh = mfma_shape(H, slots, E);
  const long long blocks = items_max < kMfmaCus * sh.per_cu ? items_max : kMfmaCus * sh.per_cu;
  if (!go) return blocks;
  if (ro) {
    launch_route(st, *ro, B, E, k);
    ids = ro->ids;
  }
  hipLaunchKernelGGL(moe::moe_gate_up_grouped_mfma_w64, dim3((unsigned)blocks), dim3(256), (unsigned)sh.lds, st,
                     static_cast<const uint16_t*>(x), ids, wg, sg, wu, su, static_cast<uint16_t*>(h), B, H, I, E, k,
                     sh.ch);
  return blocks;
}

// Variant table from graph-timed sweeps on MI355X (128 experts, top-8;
// gate/up alone, uniform routing unless stated).  While the average routed
// expert serves few slots, the per-slot kernel wins: it needs no sort and its
// grid has no per-workgroup setup (H = 2048, per-slot against matrix cores:
// 8 tokens 27.6 vs 29.3 us, 9 tokens 30.5 vs 31.4).  Once tokens share
// experts the expert-grouped product on the matrix cores reads each routed
// row once and wins: at H = 2048 from 0.625 slots per expert (10 tokens 33.0
// vs 33.0, 12 tokens 38.3 vs 37.2, 16 tokens 47.2 vs 43.5, 32 tokens 87.1 vs
// 57.1), at H = 6144 and 8192 from half a slot (I = 1024, 8 tokens: 110.5
// vs 104.4 and 142.6 vs 135.2; 5 tokens at H = 6144: 73.7 vs 76.2).  Skewed
// routing favours it earlier (H = 2048, 8 tokens, Zipf: 23.6 vs 22.6); the
// table follows uniform routing.  At H = 4096 the vector-unit grouped kernel
// beats both from 5/16 of a slot per expert up to 7/4 (I = 1536, per-slot /
// vector-unit grouped / matrix cores: 5 tokens 73.8 / 71.9 / 76.6, 8 tokens
// 109.5 / 101.3 / 106.6, 16 tokens 198.4 / 164.2 / 169.7, 24 tokens 284.8 /
// 207.3 / 209.7; I = 1024 alike), the matrix cores from there (28 tokens
// 223.5 vs 215.6, 32 tokens 240.3 vs 232.7).  Where the matrix-core kernel's
// limits exclude the shape, the vector-unit grouped kernel takes over from
// one slot per expert, or half a slot at H >= 4096 (per-slot against it:
// H = 2048, 12 tokens 38.3 vs 38.4, 16 tokens 47.2 vs 46.8).
int gate_up_default_variant(int B, int H, int I, int E, int k) {
  (void)I;
  const long long slots = (long long)B * k;
  const bool grouped_ok = grouped_allowed(passes(H), 1, slots, E);
  if (H == 4096 && 16 * slots >= 5LL * E && 4 * slots < 7LL * E && grouped_ok) return MOE_GATE_UP_EXPERT_GROUPED;
  const bool wide = H >= 4096 && 2 * slots >= E;
  if ((8 * slots >= 5LL * E || wide) && mfma_allowed(H, slots, E)) return MOE_GATE_UP_EXPERT_GROUPED_MFMA;
  if ((slots >= E || wide) && grouped_ok) return MOE_GATE_UP_EXPERT_GROUPED;
  return MOE_GATE_UP_PER_SLOT;
}

// 4 rows per wave for one pass of 1024 elements, 2 for two, 1 beyond: the
// rows, converted to bf16 once, stay within 64 VGPRs (same sweep)
int grouped_default_rows(int H) {
  const int nch = passes(H);
  return nch <= 1 ? 4 : (nch == 2 ? 2 : 1);
}

// The launcher for (variant, rows); 0 selects the table's choice.  nullptr for
// an unknown variant or a combination beyond the kernel's limits.
GateUpLaunch gate_up_launcher(int& variant, int nch, int& rows, int B, int H, int I, int E, int k) {
  if (variant == 0) variant = gate_up_default_variant(B, H, I, E, k);
  if (variant == MOE_GATE_UP_PER_SLOT) {
    if (rows == 0) rows = gate_up_default_rows(B, H, I, k);
    return gate_up_allowed(nch, rows) ? pick_gate_up(nch, rows) : nullptr;
  }
  if (variant == MOE_GATE_UP_EXPERT_GROUPED) {
    if (rows == 0) rows = grouped_default_rows(H);
    return grouped_allowed(nch, rows, (long long)B * k, E) ? pick_grouped(nch, rows) : nullptr;
  }
  if (variant == MOE_GATE_UP_EXPERT_GROUPED_MFMA) {
    if (rows == 0) rows = moe::kMfmaRows;
    return rows == moe::kMfmaRows && mfma_allowed(H, (long long)B * k, E) ? launch_mfma : nullptr;
  }
  return nullptr;
}

// Router limits: E logits per token held 16 per lane, selection j in lane j,
// and 32-bit byte offsets into the logits.
int check_route_shape(int B, int E, int k) {
  if (B < 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_SHAPE;
  if (E > moe::kRouteMaxExperts || k > moe::kRouteMaxK) return MOE_ERR_SHAPE;
  if ((long long)B * E * 4 >= (1LL << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// The router's outputs must not overlap its logits or each other.
int check_route_io(const RouteIO& ro, int B, int E, int k) {
  if (!ro.logits || !ro.ids || !ro.tw) return MOE_ERR_NULL;
  if (!aligned(ro.logits, 4) || !aligned(ro.ids, 4) || !aligned(ro.tw, 4)) return MOE_ERR_ALIGN;
  const size_t lb = (size_t)B * E * 4, ob = (size_t)B * k * 4;
  if (overlaps(ro.ids, ob, ro.logits, lb) || overlaps(ro.tw, ob, ro.logits, lb) || overlaps(ro.ids, ob, ro.tw, ob))
    return MOE_ERR_ALIAS;
  return MOE_OK;
}

// ro == nullptr: ids are an input.  Else ids is unused and the router step
// writes ro->ids and ro->tw from ro->logits.
int gate_up_impl(const void* x, const int32_t* ids, const uint8_t* wg, const uint8_t* sg, const uint8_t* wu,
                 const uint8_t* su, void* h, int B, int H, int I, int E, int k, int variant, int rows, void* stream,
                 const RouteIO* ro = nullptr) {
  int rc = check_shape(B, H, I, E, k);
  if (!rc && ro) rc = check_route_shape(B, E, k);
  if (rc) return rc;
  if (B == 0) return MOE_OK;
  if (!x || (!ro && !ids) || !wg || !sg || !wu || !su || !h) return MOE_ERR_NULL;
  if (ro && (rc = check_route_io(*ro, B, E, k))) return rc;
  if (!aligned(x, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(h, 16) || (!ro && !aligned(ids, 4)))
    return MOE_ERR_ALIGN;
  const size_t hb = (size_t)B * k * I * 2, wb = (size_t)E * I * H, sb = wb / 32;
  if (overlaps(h, hb, x, (size_t)B * H * 2) || (!ro && overlaps(h, hb, ids, (size_t)B * k * 4)) ||
      overlaps(h, hb, wg, wb) || overlaps(h, hb, wu, wb) || overlaps(h, hb, sg, sb) || overlaps(h, hb, su, sb))
    return MOE_ERR_ALIAS;
  if (ro) {   // every output against every input and the other outputs
    const size_t ob = (size_t)B * k * 4, lb = (size_t)B * E * 4;
    const void* outs[] = {ro->ids, ro->tw};
    for (const void* o : outs)
      if (overlaps(o, ob, x, (size_t)B * H * 2) || overlaps(o, ob, wg, wb) || overlaps(o, ob, wu, wb) ||
          overlaps(o, ob, sg, sb) || overlaps(o, ob, su, sb) || overlaps(o, ob, h, hb))
        return MOE_ERR_ALIAS;
    if (overlaps(h, hb, ro->logits, lb)) return MOE_ERR_ALIAS;
  }
  const int nch = passes(H);
  RouteIO rt{};
  if (ro) {   // fused: the table's choice for small batches, or the per-slot variant asked for
    rt = *ro;
    const bool small = (long long)B * k <= kRouteFusedMaxSlots;
    if (variant == 0 && small && E <= moe::kRouteFusedMaxExperts) {
      variant = MOE_GATE_UP_PER_SLOT;
      if (rows == 0 && gate_up_allowed(nch, kRouteFusedRows)) rows = kRouteFusedRows;
    }
    rt.fuse = variant == MOE_GATE_UP_PER_SLOT && E <= moe::kRouteFusedMaxExperts;
    ro = &rt;
  }
  const bool asked = variant != 0;
  GateUpLaunch fn = gate_up_launcher(variant, nch, rows, B, H, I, E, k);
  if (!fn) return MOE_ERR_ARG;
  if (variant == MOE_GATE_UP_EXPERT_GROUPED_MFMA && (!aligned(sg, 16) || !aligned(su, 16))) {
    if (asked) return MOE_ERR_ALIGN;   // the matrix-core kernel copies 16-byte pieces of the scales
    variant = MOE_GATE_UP_EXPERT_GROUPED;   // the table's choice: fall back
    rows = 0;
    fn = gate_up_launcher(variant, nch, rows, B, H, I, E, k);
    if (!fn) return MOE_ERR_ARG;
  }
  const long long blocks = fn(false, nullptr, x, ids, wg, sg, wu, su, h, B, H, I, E, k, ro);
  if (blocks * kWavesPerBlock >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (variant == MOE_GATE_UP_EXPERT_GROUPED_MFMA && mfma_setup_current_device() != hipSuccess) return MOE_ERR_LAUNCH;
  (void)hipGetLastError();
  fn(true, static_cast<hipStream_t>(stream), x, ids, wg, sg, wu, su, h, B, H, I, E, k, ro);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// ---------------------------------------------------------------- down
bool down_allowed(int np, int r) {
  return (r == 1 || r == 2 || r == 4 || r == 8) && np >= 1 && np <= kMaxDownPasses && moe_host::down_fits(np, r);
}

// The down wave streams k rows per output, so far fewer wavefronts suffice:
// the sweep favours the largest register-feasible R with >= 1024 wavefronts.
int down_default_rows(int B, int H, int I, int k) {
  const int np = passes((long long)k * I);
  int r = 8;
  while (r > 1 && (!down_allowed(np, r) || (long long)B * ((H + r - 1) / r) < 1024)) r /= 2;
  return r;
}

// Down launchers, like the gate/up ones, return their number of workgroups
// and launch only when `go` is set (moe_host::DownLaunch).  The per-token and
// the matrix-core kernels are launched from their own translation units
// (down_token.hip, down_mfma.hip); the vector-unit grouped one from here.

// ---------------------------------------------------------------- down, expert-grouped
// One workgroup per 8 (I <= 1024) or 4 output dimensions, at most two passes
// of 1024 elements over I (the rows stay in registers for every slot of an
// expert); one token per lane: B <= 64.
constexpr int kMaxDownGroupedPasses = 2;
bool down_grouped_allowed(int I, long long slots, int B, int E) {
  return passes(I) <= kMaxDownGroupedPasses && slots <= moe::kSortMaxSlots && E <= moe::kSortMaxExperts &&
         B <= moe::kDownGroupedMaxTokens;
}

template <int NP>
long long launch_down_grouped_t(bool go, hipStream_t st, const void* h, const int32_t* ids, const float* tw,
                                const uint8_t* wd, const uint8_t* sd, void* y, int B, int H, int I, int E, int k) {
  const long long blocks = H / moe::down_grouped_rows(NP);   // H is a multiple of 32
  if (!go) return blocks;
  hipLaunchKernelGGL((moe::moe_down_expert_grouped_w64<NP>), dim3((unsigned)blocks),
                     dim3(64 * moe::down_grouped_waves(NP)),
                     (unsigned)moe::down_grouped_lds_bytes(NP, E, B * k), st, static_cast<const uint16_t*>(h), ids,
                     tw, wd, sd, static_cast<uint16_t*>(y), B, H, I, E, k);
  return blocks;
}

DownLaunch pick_down_grouped(int np) {
  switch (np) {
    case 1: return launch_down_grouped_t<1>;
    case 2: return launch_down_grouped_t<2>;
  }
  return nullptr;
}

// ---------------------------------------------------------------- down, expert-grouped on the matrix cores
// One workgroup per 8 output dimensions; rounds of 256 elements over I (I <= 2048).
bool down_mfma_allowed(int I, long long slots, int E) {
  return (I + 255) / 256 <= moe::kDownMfmaMaxRounds && slots <= moe::kSortMaxSlots && E <= moe::kSortMaxExperts;
}

// Variant table (graph-timed sweeps of the down kernel alone on MI355X, 128
// experts, top-8, uniform routing unless stated): the per-token kernel while
// few tokens share an expert, the matrix-core grouped one from 5/16 of a slot
// per expert on (H = 2048, I = 768: 4 tokens 10.4 per-token vs 11.4 us, 5
// tokens 13.1 vs 12.9, 6 tokens 14.0 vs 14.2; H = 4096, I = 1536: 4 tokens
// 34.8 vs 38.2, 5 tokens 42.1 vs 43.7, 6 tokens 49.5 vs 49.2, 7 tokens 56.9
// vs 54.7, 8 tokens 62.9 vs 57.4).  Skewed routing favours the grouped
// kernels earlier (Zipf: H = 2048, 6 tokens 12.2 per-token vs 11.7; H =
// 4096, 5 tokens 37.7 vs 35.6, 6 tokens 43.9 vs 39.0), so the one threshold
// stays where uniform routing at H = 2048 puts it, although uniform routing
// at H = 4096 alone would move it to 6 tokens.  The vector-unit grouped kernel is
// never the table's choice: every shape it takes, the matrix-core kernel
// takes too, faster (per-token against it: H = 2048, 8 tokens 17.8 vs 17.3,
// 16 tokens 30.3 vs 25.3; H = 4096, 8 tokens 66.1 vs 62.8); it runs on
// request, as the vector-unit-only form of the grouped product.
int down_default_variant(int B, int H, int I, int E, int k) {
  (void)H;
  const long long slots = (long long)B * k;
  if (16 * slots >= 5LL * E && down_mfma_allowed(I, slots, E)) return MOE_DOWN_EXPERT_GROUPED_MFMA;
  return MOE_DOWN_PER_TOKEN;
}

// The launcher for (variant, rows); 0 selects the table's choice.  The
// grouped kernel takes a fixed number of rows per wavefront (8 for I <= 1024,
// else 4).
DownLaunch down_launcher(int& variant, int& rows, int B, int H, int I, int E, int k) {
  if (variant == 0) variant = down_default_variant(B, H, I, E, k);
  if (variant == MOE_DOWN_PER_TOKEN) {
    const int np = passes((long long)k * I);
    if (rows == 0) rows = down_default_rows(B, H, I, k);
    return down_allowed(np, rows) ? moe_host::pick_down(np, rows) : nullptr;
  }
  if (variant == MOE_DOWN_EXPERT_GROUPED) {
    const int ro = moe::down_grouped_rows(passes(I));
    if (rows == 0) rows = ro;
    if (rows != ro || !down_grouped_allowed(I, (long long)B * k, B, E)) return nullptr;
    return pick_down_grouped(passes(I));
  }
  if (variant == MOE_DOWN_EXPERT_GROUPED_MFMA) {
    if (rows == 0) rows = moe::kDownMfmaRows;
    if (rows != moe::kDownMfmaRows || !down_mfma_allowed(I, (long long)B * k, E)) return nullptr;
    return moe_host::pick_down_mfma(I);
  }
  return nullptr;
}

int down_impl(const void* h, const int32_t* ids, const float* tw, const uint8_t* wd, const uint8_t* sd, void* y,
              int B, int H, int I, int E, int k, int variant, int rows, void* stream) {
  int rc = check_shape(B, H, I, E, k);
  if (rc) return rc;
  if (B == 0) return MOE_OK;
  if (!h || !ids || !tw || !wd || !sd || !y) return MOE_ERR_NULL;
  if (!aligned(h, 16) || !aligned(wd, 16) || !aligned(y, 2) || !aligned(ids, 4) || !aligned(tw, 4))
    return MOE_ERR_ALIGN;
  const size_t yb = (size_t)B * H * 2, wb = (size_t)E * H * I;
  if (overlaps(y, yb, h, (size_t)B * k * I * 2) || overlaps(y, yb, ids, (size_t)B * k * 4) ||
      overlaps(y, yb, tw, (size_t)B * k * 4) || overlaps(y, yb, wd, wb) || overlaps(y, yb, sd, wb / 32))
    return MOE_ERR_ALIAS;
  DownLaunch fn = down_launcher(variant, rows, B, H, I, E, k);
  if (!fn) return MOE_ERR_ARG;
  if (variant == MOE_DOWN_EXPERT_GROUPED_MFMA && moe_host::down_mfma_setup_current_device() != hipSuccess)
    return MOE_ERR_LAUNCH;
  (void)hipGetLastError();
  fn(true, static_cast<hipStream_t>(stream), h, ids, tw, wd, sd, y, B, H, I, E, k);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// ---------------------------------------------------------------- conventional path
// Workspace layout (every part 256-byte aligned).
struct ConvLayout {
  size_t meta, row_slot, row_expert, slot_row, xq, xs, xg, xgs, hb, hq, hs, ob, total;
  ConvLayout(int B, int H, int I, int E, int k) {
    const size_t S = (size_t)B * k, P = 2 * S;
    size_t o = 0;
    auto take = [&](size_t n) { const size_t r = o; o += (n + 255) & ~(size_t)255; return r; };
    meta = take(4 * (3 * (size_t)E + 1));
    row_slot = take(4 * P);
    row_expert = take(4 * P);
    slot_row = take(4 * S);
    xq = take((size_t)B * H);
    xs = take((size_t)B * H / 32);
    xg = take(P * H);
    xgs = take(P * H / 32);
    hb = take(P * I * 2);
    hq = take(P * I);
    hs = take(P * I / 32);
    ob = take(P * H * 2);
    total = o;
  }
};

constexpr int kConvMaxPasses = 8;   // H and I up to 8192

using ConvGemv = void (*)(dim3, hipStream_t, const uint8_t*, const uint8_t*, const int*, const int*, const uint8_t*,
                          const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*, int, int, int, int, int, bool);

template <int NP, bool SWIGLU>
void launch_conv_gemv_t(dim3 grid, hipStream_t st, const uint8_t* aq, const uint8_t* as, const int* row_expert,
                        const int* meta, const uint8_t* w0, const uint8_t* s0, const uint8_t* w1, const uint8_t* s1,
                        uint16_t* out, int E, int N, int K, int Pmax, int tiles, bool stream) {
  constexpr int R = SWIGLU ? (NP <= 2 ? 2 : 1) : (NP <= 2 ? 4 : (NP <= 4 ? 2 : 1));
  if (stream)
    hipLaunchKernelGGL((moe::conv_gemv_kernel<NP, R, SWIGLU, moe::kStream>), grid, dim3(64 * kWavesPerBlock), 0, st, aq,
                       as, row_expert, meta, w0, s0, w1, s1, out, E, N, K, Pmax, tiles);
  else
    hipLaunchKernelGGL((moe::conv_gemv_kernel<NP, R, SWIGLU, moe::kCached>), grid, dim3(64 * kWavesPerBlock), 0, st, aq,
                       as, row_expert, meta, w0, s0, w1, s1, out, E, N, K, Pmax, tiles);
}
constexpr int conv_rows(int np, bool swiglu) { return swiglu ? (np <= 2 ? 2 : 1) : (np <= 2 ? 4 : (np <= 4 ? 2 : 1)); }

template <bool SWIGLU, int... NPs>
ConvGemv pick_conv_np(int np, std::integer_sequence<int, NPs...>) {
  ConvGemv fn = nullptr;
  ((np == NPs + 1 ? (fn = launch_conv_gemv_t<NPs + 1, SWIGLU>, 0) : 0), ...);
  return fn;
}

// Every check of the conventional path's arguments except the workspace's.
int conventional_check(const void* x, const int32_t* ids, const float* tw, const uint8_t* wg, const uint8_t* sg,
                       const uint8_t* wu, const uint8_t* su, const uint8_t* wd, const uint8_t* sd, const void* y,
                       int B, int H, int I, int E, int k) {
  int rc = check_shape(B, H, I, E, k);
  if (rc) return rc;
  if ((long long)B * k > moe::kConvMaxSlots || E > moe::kConvMaxSlots || passes(H) > kConvMaxPasses ||
      passes(I) > kConvMaxPasses)
    return MOE_ERR_SHAPE;
  if (B == 0) return MOE_OK;
  if (!x || !ids || !tw || !wg || !sg || !wu || !su || !wd || !sd || !y) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) || !aligned(y, 2) ||
      !aligned(ids, 4) || !aligned(tw, 4))
    return MOE_ERR_ALIGN;
  const size_t yb = (size_t)B * H * 2, wb = (size_t)E * I * H;
  const void* ins[] = {x, ids, tw, wg, sg, wu, su, wd, sd};
  const size_t insz[] = {(size_t)B * H * 2, (size_t)B * k * 4, (size_t)B * k * 4, wb, wb / 32, wb, wb / 32, wb, wb / 32};
  for (int i = 0; i < 9; ++i)
    if (overlaps(y, yb, ins[i], insz[i])) return MOE_ERR_ALIAS;
  return MOE_OK;
}

int conventional_impl(const void* x, const int32_t* ids, const float* tw, const uint8_t* wg, const uint8_t* sg,
                      const uint8_t* wu, const uint8_t* su, const uint8_t* wd, const uint8_t* sd, void* y, void* ws,
                      size_t ws_bytes, int B, int H, int I, int E, int k, void* stream) {
  int rc = conventional_check(x, ids, tw, wg, sg, wu, su, wd, sd, y, B, H, I, E, k);
  if (rc || B == 0) return rc;
  if (!ws) return MOE_ERR_NULL;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGN;
  const ConvLayout L(B, H, I, E, k);
  if (ws_bytes < L.total) return MOE_ERR_ARG;
  const size_t wb = (size_t)E * I * H;
  const void* ins[] = {x, ids, tw, wg, sg, wu, su, wd, sd, y};
  const size_t insz[] = {(size_t)B * H * 2, (size_t)B * k * 4, (size_t)B * k * 4, wb, wb / 32, wb, wb / 32, wb, wb / 32,
                         (size_t)B * H * 2};
  for (int i = 0; i < 10; ++i)
    if (overlaps(ws, L.total, ins[i], insz[i])) return MOE_ERR_ALIAS;
  ConvGemv gu = pick_conv_np<true>(passes(H), std::make_integer_sequence<int, kConvMaxPasses>{});
  ConvGemv dn = pick_conv_np<false>(passes(I), std::make_integer_sequence<int, kConvMaxPasses>{});
  if (!gu || !dn) return MOE_ERR_SHAPE;

  uint8_t* w8 = static_cast<uint8_t*>(ws);
  int* meta = reinterpret_cast<int*>(w8 + L.meta);
  int* row_slot = reinterpret_cast<int*>(w8 + L.row_slot);
  int* row_expert = reinterpret_cast<int*>(w8 + L.row_expert);
  int* slot_row = reinterpret_cast<int*>(w8 + L.slot_row);
  const int S = B * k, Pmax = 2 * S;
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto blocks = [](long long n) { return dim3((unsigned)((n + 255) / 256)); };
  (void)hipGetLastError();
  hipLaunchKernelGGL(moe::conv_route_kernel, dim3(1), dim3(1024), 0, st, ids, S, E, Pmax, meta, row_slot, row_expert,
                     slot_row);
  hipLaunchKernelGGL(moe::conv_quant_kernel, blocks((long long)B * (H / 32)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(x), B, H, nullptr, w8 + L.xq, w8 + L.xs);
  hipLaunchKernelGGL(moe::conv_scatter_kernel, blocks((long long)Pmax * (H / 16 + H / 32)), dim3(256), 0, st,
                     w8 + L.xq, w8 + L.xs, row_slot, meta, E, Pmax, H, k, w8 + L.xg, w8 + L.xgs);
  // weight rows as streaming data while an expert's padded rows are few
  // (graph-timed, H = 2048, I = 768, 128 experts, top-8: 1 token 29.9 vs 32.0
  // us, 8 tokens 71.3 vs 73.4, 12 tokens 91.9 vs 92.8); from one slot per
  // expert on the padded rows of one expert re-read its rows from L2, and the
  // default policy keeps them there (16 tokens 110.5 vs 112.0, 32 tokens
  // 181.8 vs 192.0)
  const bool stream_rows = (long long)B * k < E;
  const int rg = conv_rows(passes(H), true), tg = (I + rg - 1) / rg;
  gu(dim3((unsigned)(((long long)tg * Pmax + kWavesPerBlock - 1) / kWavesPerBlock)), st, w8 + L.xg, w8 + L.xgs,
     row_expert, meta, wg, sg, wu, su, reinterpret_cast<uint16_t*>(w8 + L.hb), E, I, H, Pmax, tg, stream_rows);
  hipLaunchKernelGGL(moe::conv_quant_kernel, blocks((long long)Pmax * (I / 32)), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(w8 + L.hb), Pmax, I, meta + 3 * E, w8 + L.hq, w8 + L.hs);
  const int rd = conv_rows(passes(I), false), td = (H + rd - 1) / rd;
  dn(dim3((unsigned)(((long long)td * Pmax + kWavesPerBlock - 1) / kWavesPerBlock)), st, w8 + L.hq, w8 + L.hs,
     row_expert, meta, wd, sd, nullptr, nullptr, reinterpret_cast<uint16_t*>(w8 + L.ob), E, H, I, Pmax, td, stream_rows);
  hipLaunchKernelGGL(moe::conv_combine_kernel, blocks((long long)B * H), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(w8 + L.ob), slot_row, tw, static_cast<uint16_t*>(y), B, H, k);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

// ---------------------------------------------------------------- conventional path, no allocation
// A fixed device buffer for callers that cannot allocate (code under graph
// capture, serving loops, harnesses that forbid hipMalloc): it stands in for
// the caller's workspace.  32 MiB holds the workspace of every decode shape
// measured here (H=2048, I=768, 128 experts, top-8 up to 128 tokens: 17 MB;
// H=4096, I=1536 up to 64 tokens: 17 MB).  Each device holds its own copy from
// module load until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kConvScratchBytes = size_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kConvScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (nullptr on failure).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_rc[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_rc[dev] == hipSuccess ? p : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_decode_gate_up(const void* x, const int32_t* topk_ids, const uint8_t* w_gate, const uint8_t* s_gate,
                       const uint8_t* w_up, const uint8_t* s_up, void* h_out, int B, int H, int I, int E, int k,
                       void* stream) {
  return gate_up_impl(x, topk_ids, w_gate, s_gate, w_up, s_up, h_out, B, H, I, E, k, 0, 0, stream);
}

int moe_decode_gate_up_ex(const void* x, const int32_t* topk_ids, const uint8_t* w_gate, const uint8_t* s_gate,
                          const uint8_t* w_up, const uint8_t* s_up, void* h_out, int B, int H, int I, int E, int k,
                          int variant, int rows_per_wave, void* stream) {
  if (rows_per_wave < 0 || variant < 0) return MOE_ERR_ARG;
  return gate_up_impl(x, topk_ids, w_gate, s_gate, w_up, s_up, h_out, B, H, I, E, k, variant, rows_per_wave, stream);
}

int moe_decode_route(const float* logits, int32_t* topk_ids, float* topk_weights, int B, int E, int k,
                     void* stream) {
  int rc = check_route_shape(B, E, k);
  if (rc) return rc;
  if (B == 0) return MOE_OK;
  const RouteIO ro{logits, topk_ids, topk_weights, false};
  if ((rc = check_route_io(ro, B, E, k))) return rc;
  (void)hipGetLastError();
  launch_route(static_cast<hipStream_t>(stream), ro, B, E, k);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_decode_gate_up_routed(const void* x, const float* logits, const uint8_t* w_gate, const uint8_t* s_gate,
                              const uint8_t* w_up, const uint8_t* s_up, void* h_out, int32_t* topk_ids_out,
                              float* topk_weights_out, int B, int H, int I, int E, int k, void* stream) {
  const RouteIO ro{logits, topk_ids_out, topk_weights_out, false};
  return gate_up_impl(x, nullptr, w_gate, s_gate, w_up, s_up, h_out, B, H, I, E, k, 0, 0, stream, &ro);
}

int moe_decode_gate_up_routed_ex(const void* x, const float* logits, const uint8_t* w_gate, const uint8_t* s_gate,
                                 const uint8_t* w_up, const uint8_t* s_up, void* h_out, int32_t* topk_ids_out,
                                 float* topk_weights_out, int B, int H, int I, int E, int k, int variant,
                                 int rows_per_wave, void* stream) {
  if (rows_per_wave < 0 || variant < 0) return MOE_ERR_ARG;
  const RouteIO ro{logits, topk_ids_out, topk_weights_out, false};
  return gate_up_impl(x, nullptr, w_gate, s_gate, w_up, s_up, h_out, B, H, I, E, k, variant, rows_per_wave, stream,
                      &ro);
}

int moe_decode_down(const void* h, const int32_t* topk_ids, const float* topk_weights, const uint8_t* w_down,
                    const uint8_t* s_down, void* y_out, int B, int H, int I, int E, int k, void* stream) {
  return down_impl(h, topk_ids, topk_weights, w_down, s_down, y_out, B, H, I, E, k, 0, 0, stream);
}

int moe_decode_down_ex(const void* h, const int32_t* topk_ids, const float* topk_weights, const uint8_t* w_down,
                       const uint8_t* s_down, void* y_out, int B, int H, int I, int E, int k, int variant,
                       int rows_per_wave, void* stream) {
  if (rows_per_wave < 0 || variant < 0) return MOE_ERR_ARG;
  return down_impl(h, topk_ids, topk_weights, w_down, s_down, y_out, B, H, I, E, k, variant, rows_per_wave, stream);
}

int moe_decode_conventional_workspace(int B, int H, int I, int E, int k, size_t* bytes) {
  int rc = check_shape(B, H, I, E, k);
  if (rc) return rc;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = ConvLayout(B, H, I, E, k).total;
  return MOE_OK;
}

int moe_decode_conventional(const void* x, const int32_t* topk_ids, const float* topk_weights, const uint8_t* w_gate,
                            const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                            const uint8_t* s_down, void* y_out, void* workspace, size_t workspace_bytes, int B, int H,
                            int I, int E, int k, void* stream) {
  return conventional_impl(x, topk_ids, topk_weights, w_gate, s_gate, w_up, s_up, w_down, s_down, y_out, workspace,
                           workspace_bytes, B, H, I, E, k, stream);
}

int moe_decode_conventional_noalloc(const void* x, const int32_t* topk_ids, const float* topk_weights,
                                    const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                                    const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down, void* y_out,
                                    int B, int H, int I, int E, int k, void* stream) {
  // Every check that needs no device comes first; then the fixed buffer's size.
  int rc = conventional_check(x, topk_ids, topk_weights, w_gate, s_gate, w_up, s_up, w_down, s_down, y_out, B, H, I,
                              E, k);
  if (rc || B == 0) return rc;
  if (ConvLayout(B, H, I, E, k).total > kConvScratchBytes) return MOE_ERR_SCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_LAUNCH;
  return conventional_impl(x, topk_ids, topk_weights, w_gate, s_gate, w_up, s_up, w_down, s_down, y_out, ws,
                           kConvScratchBytes, B, H, I, E, k, stream);
}

int moe_decode_gate_up_plan(int B, int H, int I, int E, int k, int* variant, int* rows_per_wave, int* workgroups) {
  int rc = check_shape(B, H, I, E, k);
  if (rc) return rc;
  if (!variant || !rows_per_wave || !workgroups) return MOE_ERR_NULL;
  int v = 0, r = 0;
  GateUpLaunch fn = gate_up_launcher(v, passes(H), r, B, H, I, E, k);
  if (!fn) return MOE_ERR_ARG;
  *variant = v;
  *rows_per_wave = r;
  *workgroups =
      (int)fn(false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, I, E, k, nullptr);
  return MOE_OK;
}

int moe_decode_down_plan(int B, int H, int I, int E, int k, int* variant, int* rows_per_wave, int* workgroups) {
  int rc = check_shape(B, H, I, E, k);
  if (rc) return rc;
  if (!variant || !rows_per_wave || !workgroups) return MOE_ERR_NULL;
  int v = 0, r = 0;
  DownLaunch fn = down_launcher(v, r, B, H, I, E, k);
  if (!fn) return MOE_ERR_ARG;
  *variant = v;
  *rows_per_wave = r;
  *workgroups = (int)fn(false, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H, I, E, k);
  return MOE_OK;
}

int moe_decode_copy_peak(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (bytes == 0 || bytes % 16) return MOE_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_ALIGN;
  if (overlaps(src, bytes, dst, bytes)) return MOE_ERR_ALIAS;
  const size_t n = bytes / 16;
  const size_t want = (n + moe::kPeakThreads - 1) / moe::kPeakThreads;
  const dim3 grid((unsigned)(want < moe::kPeakMaxBlocks ? want : moe::kPeakMaxBlocks));
  (void)hipGetLastError();
  hipLaunchKernelGGL(moe::copy_peak_kernel, grid, dim3(moe::kPeakThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const moe::u32x4*>(src), static_cast<moe::u32x4*>(dst), n);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_decode_read_peak(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return MOE_ERR_NULL;
  if (bytes == 0 || bytes % 16) return MOE_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return MOE_ERR_ALIGN;
  const size_t n = bytes / 16;
  const size_t want = (n + moe::kPeakThreads - 1) / moe::kPeakThreads;
  const dim3 grid((unsigned)(want < moe::kPeakMaxBlocks ? want : moe::kPeakMaxBlocks));
  (void)hipGetLastError();
  hipLaunchKernelGGL(moe::read_peak_kernel, grid, dim3(moe::kPeakThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const moe::u32x4*>(src), n, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

const char* moe_decode_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "unsupported or invalid shape";
    case MOE_ERR_ALIGN: return "misaligned pointer (x, h, weights need 16 bytes; ids and router weights 4)";
    case MOE_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case MOE_ERR_ALIAS: return "an output overlaps an input";
    case MOE_ERR_ARG: return "invalid tuning argument";
    case MOE_ERR_SCRATCH: return "the shape needs more scratch memory than the library's fixed buffer holds (32 MiB)";
  }
  return "unknown error code";
}

}  // extern "C"
