// Gate/up kernel, expert-grouped variant on the matrix cores (blog post "warp
// decode", section "How the two kernels work" for the arithmetic; section
// "Warp decode and Composer training" for the regime where several tokens
// share an expert).  Every output h[b,j,n] is still SiLU(gate) * up of one
// neuron, from the MXFP8 rows of expert ids[b,j] dotted with the bf16 x[b] in
// FP32 and written once as bf16, with no padding, gather buffer or combine.
//
// Once several tokens share an expert, the product of that expert's gate/up
// rows with those tokens' activations is a small dense product, and the dot
// products go to v_mfma_f32_16x16x32_bf16: 16 rows (neurons) by 16 columns
// (the tokens of one work unit).  The vector units only decode the weights.
//
// Work item: 16 neurons of one work unit (one routed expert, up to 16 of its
// slots).  The workgroup streams the reduction in chunks of 512 elements:
// the 32 rows' chunks (16 gate rows, 16 up rows; 512 bytes each) and the
// tokens' activations (1 KB each) are copied straight from memory into LDS
// (buffer loads with the LDS bit, 1 KB per wave instruction, each row read
// as one contiguous run), double-buffered, so the copies of chunk c + 1 run
// while chunk c is multiplied.  Every lane's 16-byte piece lands at a fixed
// LDS position (16 x lane), so the pieces are swizzled on the way in: lane l
// fetches piece l ^ (row mod 16) of a weight row and piece l ^ 2 (token mod
// 16) -- two times the token's index mod 16 -- of an activation row, which
// makes the MFMA operand reads from LDS free of bank conflicts.  The 4 wavefronts split a chunk's eight 64-element
// tiles; in a tile, lane (r, q) (r = lane mod 16, q = lane / 16) takes
// elements 16 q .. 16 q + 15 of row r and of token r, the first 8 for one
// MFMA and the last 8 for another (the same K order on both operands).
// E4M3 pairs become bf16 with v_cvt_scalef32_pk_bf16_fp8 and the block's
// E8M0 scale folded in: the scaled weight rounded to bf16, exact whenever
// it is a normal bf16.  So that no scaled weight overflows, a row whose
// largest code exceeds 246 has all its codes lowered by d and its sums
// multiplied by 2^d (exact); so that the weights of a row of tiny blocks
// stay normal, a row whose largest code is below 64 has all its codes
// raised by d and its sums multiplied by 2^-d.  Every block within 2^54 of
// its row's largest is then exact; blocks further below round to bf16
// subnormals or zero, far below FP32 resolution of the sum.  NaN scale
// codes and E4M3 NaN codes give NaN outputs.
//
// After the last chunk each wavefront's 16 x 16 gate and up partial sums go
// to LDS (the chunk buffer the last chunk leaves free) and threads (n, t) add
// the 4 partials in wavefront order (a fixed order) and write
// h = bf16(SiLU(g) * u).  Items go out round-robin over a grid of one
// resident round (LDS: under 54 KB with units of 8 slots for up to ~40
// tokens at H = 2048, three workgroups per CU; under 80 KB with units of 16
// for the other decode shapes, two per CU).  Limits: H a multiple of 2048 up to 8192 (an item's scale codes are
// copied in whole KB pieces, one matrix per piece), B*k <= 1024, E <= 1024,
// scale tensors 16-byte aligned.
#pragma once

#include "slot_index.hpp"

namespace moe {

constexpr int kMfmaChunk = 512;                       // reduction elements per LDS chunk
constexpr int kMfmaRows = 16;                         // neurons per work item (MFMA rows)
constexpr int kMfmaColumns = 16;                      // MFMA columns: the most slots a work unit can have
constexpr int kMfmaSafeScale = 246;                   // 448 * 2^(246 - 127) < 2^128
constexpr int kMfmaLowScale = 64;                     // rows whose largest code is below: raised to it
constexpr int kMfmaWBytes = 2 * kMfmaRows * kMfmaChunk;     // weight chunk: 32 rows x 512 bytes

// One chunk buffer: the weight chunk and the unit's activations over the chunk
// (ch tokens x 1 KB, ch = 8 or 16 slots per work unit).
__host__ __device__ constexpr int mfma_buf_bytes(int ch) { return kMfmaWBytes + ch * kMfmaChunk * 2; }
// LDS: the slot index's live part | 2 chunk buffers | the scale codes of the
// item's 32 rows (the chunk buffers also cover the index build's scratch,
// and the partial sums [4 waves][2][16][16] reuse the buffer the last chunk
// leaves free)
__host__ __device__ constexpr int mfma_lds_bytes(int E, int S, int H, int ch) {
  return slot_index_live_bytes(S) + 2 * mfma_buf_bytes(ch) + 2 * kMfmaRows * (H / 32) > slot_index_lds_bytes(E, S)
             ? slot_index_live_bytes(S) + 2 * mfma_buf_bytes(ch) + 2 * kMfmaRows * (H / 32)
             : slot_index_lds_bytes(E, S);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Eight E4M3 bytes (lo: bytes 0-3, hi: bytes 4-7) to bf16 times the power of
// two whose exponent field is sc's, in byte order.
__device__ __forceinline__ bf16x8_t e4m3x8_scaled(uint32_t lo, uint32_t hi, float sc) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
  bf16x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Byte address in LDS of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Nonzero iff a byte of v is an E8M0 code in [247, 255].
__device__ __forceinline__ uint32_t has_big_scale(uint32_t v) {
  const uint32_t t = ~v;
  return (t - 0x09090909u) & ~t & 0x80808080u;
}
// Nonzero iff a byte of v is an E8M0 code below 64 (a borrow out of a byte
// only starts at a byte that is itself below 64).
__device__ __forceinline__ uint32_t has_small_scale(uint32_t v) {
  static_assert(kMfmaLowScale == 64, "the byte constant below");
  return (v - 0x40404040u) & ~v & 0x80808080u;
}

__global__ __launch_bounds__(256) void moe_gate_up_grouped_mfma_w64(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
    const uint8_t* __restrict__ wg, const uint8_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint8_t* __restrict__ su,
    uint16_t* __restrict__ h, int B, int H, int I, int E, int k, int ch) {
  typedef __attribute__((address_space(3))) void lds_void;
  const int slots = B * k;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SlotIndex si = build_slot_index<256, true>(lds, ids, slots, E, k, ch);
  __syncthreads();   // every thread has read the build's counters: its scratch becomes chunk buffer space
  const int bufb = mfma_buf_bytes(ch);
  uint8_t* buf = lds + slot_index_live_bytes(slots);                 // 2 x (weights | activations)
  const int nblk = H >> 5;
  uint8_t* scl = buf + 2 * bufb;                                     // [2][16 rows][nblk] codes

  const uint32_t wbytes = (uint32_t)E * (uint32_t)I * (uint32_t)H;   // < 2^32, checked on the host
  const rsrc_t gr = make_rsrc(wg, wbytes), ur = make_rsrc(wu, wbytes);
  const rsrc_t gsr = make_rsrc(sg, wbytes / 32), usr = make_rsrc(su, wbytes / 32);
  const rsrc_t xr = make_rsrc(x, (uint64_t)B * H * 2);
  const rsrc_t idr = make_rsrc(ids, (uint64_t)slots * 4);
  const int n_grp = (I + kMfmaRows - 1) / kMfmaRows;
  const int n_items = si.n_units * n_grp;
  const int n_chunks = H / kMfmaChunk;   // >= 4
  const int lr = lane & 15, lq = lane >> 4;

  // partial sums [4][2][16][16]: in the buffer of chunk n_chunks, which no chunk
  // of the item fills after chunk n_chunks - 2 has been used
  float* part = reinterpret_cast<float*>(buf + (n_chunks & 1) * bufb);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int un = __builtin_amdgcn_readfirstlane(item / n_grp);
    int e, first, count;   // count: 1 .. 16
    si.unit(un, e, first, count);
    const int n0 = (item - un * n_grp) * kMfmaRows;

    // copies of chunk c into buffer c % 2: wavefront w takes weight rows
    // 8w .. 8w + 7 (two per instruction, one matrix each) and tokens w, w + 4, ...
    auto copy_chunk = [&](int c) {
      uint8_t* wb = buf + (c & 1) * bufb;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r2 = 8 * w + 2 * p;                 // rows r2, r2 + 1 (both gate or both up)
        const int rr = r2 + (lane >> 5);             // this lane's row, 0..31
        const int mr = rr & 15;                      // row within its matrix
        const uint32_t row = (uint32_t)(e * I + min(n0 + mr, I - 1));   // ragged: clamp, not stored
        const uint32_t piece = (uint32_t)((lane & 31) ^ mr);
        const uint32_t off = row * (uint32_t)H + (uint32_t)(c * kMfmaChunk) + 16u * piece;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r2 < 16 ? gr : ur, (lds_void*)(wb + r2 * kMfmaChunk), 16, off, 0, 0, kStream);
      }
      uint8_t* xb = wb + kMfmaWBytes;
      for (int m = w; m < count; m += 4) {
        const uint32_t tok = (uint32_t)__builtin_amdgcn_readfirstlane((int)(si.sorted[first + m] >> 16));
        const uint32_t piece = (uint32_t)(lane ^ (2 * (m & 15)));
        const uint32_t off = tok * (uint32_t)H * 2u + (uint32_t)(c * kMfmaChunk) * 2u + 16u * piece;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xb + m * 1024), 16, off, 0, 0, 0);
      }
    };
    // the 32 rows' scale codes: 16 x nblk contiguous bytes per matrix
    for (int p = w; p < (2 * kMfmaRows * nblk) / 1024; p += 4) {   // whole KB pieces
      const int mat = (p * 1024) / (kMfmaRows * nblk);
      const uint32_t base = (uint32_t)(e * I + n0) * (uint32_t)nblk;
      const uint32_t o = (uint32_t)(p * 1024 - mat * kMfmaRows * nblk);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mat ? usr : gsr, (lds_void*)(scl + p * 1024), 16, base + o + 16u * lane, 0, 0, kStream);
    }
    copy_chunk(0);

    f32x4_t accg = {0.0f, 0.0f, 0.0f, 0.0f}, accu = {0.0f, 0.0f, 0.0f, 0.0f};
    int dg = 0, du = 0;   // this lane's row's shift (gate / up)
    bool shifted = false;
    const int tc = lr < count ? lr : count - 1;   // this lane's token column (past the unit: repeat, unused)
    for (int c = 0; c < n_chunks; ++c) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wavefront's copies of chunk c (and the scales)
      __syncthreads();                            // everyone's; and everyone is done with chunk c - 1
      // codes above 246 or below 64 anywhere in the item's rows (a wave-wide
      // check), read before the copies of chunk 1 are issued so that these
      // reads wait for nothing
      if (c == 0) {
        uint32_t any = 0;
        for (int i = lane * 16; i < 2 * kMfmaRows * nblk; i += 1024) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(scl + i);
#pragma unroll
          for (int q = 0; q < 4; ++q) any |= has_big_scale(v.v[q]) | has_small_scale(v.v[q]);
        }
        shifted = __builtin_amdgcn_ballot_w64(any != 0) != 0;
        if (shifted) {   // this lane's rows' largest non-NaN codes
          int mg = 0, mu = 0;
          for (int b = 0; b < nblk; ++b) {
            const int cg = scl[lr * nblk + b], cu = scl[(kMfmaRows + lr) * nblk + b];
            mg = (cg != 255 && cg > mg) ? cg : mg;
            mu = (cu != 255 && cu > mu) ? cu : mu;
          }
          // lowered by d > 0 or raised by -d > 0; raised codes stay below 128
          dg = mg > kMfmaSafeScale ? mg - kMfmaSafeScale : (mg < kMfmaLowScale ? mg - kMfmaLowScale : 0);
          du = mu > kMfmaSafeScale ? mu - kMfmaSafeScale : (mu < kMfmaLowScale ? mu - kMfmaLowScale : 0);
        }
      }
      if (c + 1 < n_chunks) copy_chunk(c + 1);
      const uint8_t* wb = buf + (c & 1) * bufb;
      const uint8_t* xb = wb + kMfmaWBytes;
      // This wavefront's operands of chunk c: its tiles tl = 2w and 2w + 1 (64
      // elements each).  Lane (lr, lq) takes the 16-byte piece 4 tl + lq of gate
      // row lr and of up row lr (8192 bytes further), the pieces 8 tl + 2 lq and
      // + 1 of token tc's activations, and the E8M0 codes of the gate and up
      // blocks those pieces belong to (the second tile's: 2 bytes further).
      // The reads are one asm block with its own wait: as plain loads the
      // compiler, which cannot tell them from the copies of chunk c + 1 into
      // the other buffer, waited for those copies first, and nothing overlapped.
      static_assert(kMfmaRows * kMfmaChunk == 8192 && kMfmaChunk / 32 / 8 == 2, "offsets in the asm below");
      typedef uint32_t v4u __attribute__((ext_vector_type(4)));
      v4u ag0, au0, xa0, xb0, ag1, au1, xa1, xb1;
      uint32_t cg0, cu0, cg1, cu1;
      {
        const int tl0 = 2 * w;
        const uint32_t pa0 = lds_addr(wb + lr * kMfmaChunk + 16 * ((4 * tl0 + lq) ^ lr));
        const uint32_t pa1 = lds_addr(wb + lr * kMfmaChunk + 16 * ((4 * tl0 + 4 + lq) ^ lr));
        const uint32_t px0 = lds_addr(xb + tc * 1024 + 16 * ((8 * tl0 + 2 * lq) ^ (2 * (tc & 15))));
        const uint32_t px1 = lds_addr(xb + tc * 1024 + 16 * ((8 * tl0 + 8 + 2 * lq) ^ (2 * (tc & 15))));
        const int blk = c * (kMfmaChunk / 32) + 2 * tl0 + (lq >> 1);
        const uint32_t psg = lds_addr(scl + lr * nblk + blk), psu = lds_addr(scl + (kMfmaRows + lr) * nblk + blk);
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %12 offset:8192\n\t"
            "ds_read_b128 %2, %14\n\t"
            "ds_read_b128 %3, %14 offset:16\n\t"
            "ds_read_b128 %4, %13\n\t"
            "ds_read_b128 %5, %13 offset:8192\n\t"
            "ds_read_b128 %6, %15\n\t"
            "ds_read_b128 %7, %15 offset:16\n\t"
            "ds_read_u8 %8, %16\n\t"
            "ds_read_u8 %9, %17\n\t"
            "ds_read_u8 %10, %16 offset:2\n\t"
            "ds_read_u8 %11, %17 offset:2\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(ag0), "=&v"(au0), "=&v"(xa0), "=&v"(xb0), "=&v"(ag1), "=&v"(au1), "=&v"(xa1), "=&v"(xb1),
              "=&v"(cg0), "=&v"(cu0), "=&v"(cg1), "=&v"(cu1)
            : "v"(pa0), "v"(pa1), "v"(px0), "v"(px1), "v"(psg), "v"(psu)
            : "memory");
      }
      const v4u a_g[2] = {ag0, ag1}, a_u[2] = {au0, au1}, b0[2] = {xa0, xa1}, b1[2] = {xb0, xb1};
      const int cg[2] = {(int)cg0, (int)cg1}, cu[2] = {(int)cu0, (int)cu1};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float sgf = __builtin_bit_cast(float, (uint32_t)(cg[tt] == 255 ? 255 : max(cg[tt] - dg, 0)) << 23);
        const float suf = __builtin_bit_cast(float, (uint32_t)(cu[tt] == 255 ? 255 : max(cu[tt] - du, 0)) << 23);
        const bf16x8_t x0 = __builtin_bit_cast(bf16x8_t, b0[tt]);
        const bf16x8_t x1 = __builtin_bit_cast(bf16x8_t, b1[tt]);
        accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_scaled(a_g[tt][0], a_g[tt][1], sgf), x0, accg, 0, 0, 0);
        accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_scaled(a_g[tt][2], a_g[tt][3], sgf), x1, accg, 0, 0, 0);
        accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_scaled(a_u[tt][0], a_u[tt][1], suf), x0, accu, 0, 0, 0);
        accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_scaled(a_u[tt][2], a_u[tt][3], suf), x1, accu, 0, 0, 0);
      }
    }
    // lane l holds rows 4 (l / 16) + j of column l % 16
    if (shifted) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rsrc = 4 * (4 * lq + j);   // lane 4 lq + j (< 16) holds that row's shifts
        accg[j] = __builtin_ldexpf(accg[j], __builtin_amdgcn_ds_bpermute(rsrc, dg));
        accu[j] = __builtin_ldexpf(accu[j], __builtin_amdgcn_ds_bpermute(rsrc, du));
      }
    }
    float* pw = part + w * 512;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pw[(4 * lq + j) * 16 + lr] = accg[j];
      pw[256 + (4 * lq + j) * 16 + lr] = accu[j];
    }
    __syncthreads();
    {
      const int n = tid >> 4, tk = tid & 15;
      if (tk < count && n0 + n < I) {
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          g += part[v * 512 + n * 16 + tk];
          u += part[v * 512 + 256 + n * 16 + tk];
        }
        const int s = (int)(si.sorted[first + tk] & 0xFFFFu);
        h[(size_t)s * I + n0 + n] = f32_to_bf16_rne(silu(g) * u);
      }
    }
    __syncthreads();   // partial sums, scale codes and buffer 0 free for the next item
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
