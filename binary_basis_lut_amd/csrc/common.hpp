// common.hpp -- types, argument blocks and device helpers shared by the gfx950
// (CDNA4) kernels of the FluxBin LUT GEMV.
//
// Method (FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by
// Algorithm-Kernel Synergy, paperlayer.ai summary, section 3 bullets
// "LUT-Based GEMV Kernel" and "Virtual Columnar Mapping", appendix C.1; the
// ainews.surl.tw article on FluxBin, paragraph on the execution layer):
//   * scale-fused tables: for every g-column sub-vector the 2^g signed sums of
//     v_t = c_t * x_t are tabulated, so the column scale never reaches the
//     main loop; only 2^(g-1) sums are computed, the other half is their
//     negation (LUT[~p] = -LUT[p], LUT Tensor Core notes, section 3.1.2);
//   * the packed sign bits of a row are used directly as table indices;
//   * lookups accumulate in fp32 registers; the row scale is applied once per
//     segment after accumulation, or, in the block-wise format (one row scale
//     per 128-column group, FluxBin summary appendix C.2), to each group's
//     partial sum;
//   * salient bases run through the same code on their compact columns, with
//     x gathered through the salient index while the tables are built (VCM).
//
// Mapping onto CDNA4 (not the pages' A100 tiling):
//   * one wave = 64 output rows, lane l = row l of its tile; all 64 lanes read
//     the SAME 2^g-entry table at each step: at g = 4 a read of 16
//     consecutive dwords, conflict-free; at g = 8 (one batch row, per-row
//     scales, fp32 entries) the tables are instead laid out one per LDS bank
//     and the lanes spread over them (gemv_banked.hpp);
//   * weights are streamed from the TILED layout: a wave's 16-byte-per-lane
//     load of one 128-column chunk is 1 KiB of contiguous memory, loaded with
//     non-temporal 128-bit loads (streamed once, kept out of L2);
//   * a workgroup of WAVES waves shares the tables of CPB consecutive chunks of
//     the concatenated column space of all segments; a grid of
//     row_blocks x splits workgroups (a 2D grid) covers the layer;
//   * a workgroup's column range never leaves one segment, so its sign words
//     are consecutive 1 KiB blocks and its partial sum takes one row scale;
//   * splits > 1: each workgroup adds its fp32 partial of every row, as an
//     exact fixed-point integer, into a per-row 64-bit word that also counts
//     arrivals; the lane whose atomic brings the last contribution writes the
//     fp16 row.  One launch does the whole GEMV, the result is bitwise
//     deterministic, and no workgroup ever waits for another.  A partial too
//     large for the fixed-point range sets a sticky flag in the word, and the
//     row is then written as NaN instead of a wrong number.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fluxbin {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkCols = 128;  // columns per chunk = 4 sign words per row
constexpr int kTileRows = 64;    // rows per tile = one wave, one row per lane
constexpr int kMaxSeg = 6;       // kb <= 4 global + ks <= 2 salient bases
// Split reduction: one 64-bit word per (batch row, output row).  Bit 63 is a
// sticky overflow flag, bits 55-62 count the contributions so far and bits
// 0-54 hold the sum of their biased fixed-point values.  A contribution is
// round(partial * 2^29) + 2^46, which lies in [0, 2^47) for |partial| < 2^17;
// up to 255 of them sum below 2^55, so the value never carries into the count
// and the count (at most 255) never reaches the flag.  A partial outside that
// range is clamped and also ORs the flag into the word before it adds itself:
// both are atomics on the same word from the same lane, so the flag precedes
// the contribution in the word's modification order and the last arriver sees
// it.
constexpr int kCountShift = 55;
constexpr int kMaxSplits = 255;
constexpr uint64_t kOneArrival = 1ull << kCountShift;
constexpr uint64_t kValueMask = kOneArrival - 1;
constexpr uint64_t kOverflow = 1ull << 63;
constexpr int64_t kFixBias = 1ll << 46;
constexpr float kFixScale = 536870912.0f;           // 2^29
constexpr float kFixInv = 1.0f / 536870912.0f;      // 2^-29
constexpr float kFixLimit = 70368744177664.0f;      // 2^46: |partial * 2^29| must stay below it
constexpr uint16_t kHalfNaN = 0x7e00;

// The segments of one layer (kb global bases over k columns, then ks salient
// bases over s compact columns), addressed arithmetically: the descriptor of
// any chunk or segment follows from these scalars without further loads.
struct LayerArgs {
  const u32x4 *bits_g;  // tiled words of global basis b at bits_g + b * tv_g
  const u32x4 *bits_s;  // tiled words of salient basis b at bits_s + b * tv_s
  const uint16_t *c_g;  // fp16 [kb][k]
  const uint16_t *c_s;  // fp16 [ks][s], compact order
  const uint16_t *r_g;  // fp16 [kb][n]
  const uint16_t *r_s;  // fp16 [ks][n]
  const int32_t *sal_idx;
  int64_t tv_g, tv_s;   // 16-byte elements per tiled segment block
  int64_t n, k, s;
  int32_t kb, ks;
  int32_t nc_g, nc_s;   // 128-column chunks per global / salient segment
};

#define FB_GLOBAL __attribute__((address_space(1)))

// Uniform copies of kernel arguments.  readfirstlane makes each value an
// opaque scalar-register value, so a later choice between two fields stays a
// scalar select instead of becoming a per-lane load through a chosen address.
// Pointers come back typed in the global address space (global_load, not flat).
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint64_t u = (uint64_t)v;
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)u));
}
template <typename T>
__device__ __forceinline__ const FB_GLOBAL T *uni(const T *p) {
  return (const FB_GLOBAL T *)(uintptr_t)uni((int64_t)reinterpret_cast<uintptr_t>(p));
}

// A layer's arguments in scalar registers.
struct ULayer {
  const FB_GLOBAL u32x4 *bits_g, *bits_s;
  const FB_GLOBAL uint16_t *c_g, *c_s, *r_g, *r_s;
  const FB_GLOBAL int32_t *sal_idx;
  int64_t tv_g, tv_s, n, k, s;
  int32_t kb, ks, nc_g, nc_s;
};

__device__ __forceinline__ ULayer uniform_layer(const LayerArgs &a) {
  ULayer L;
  L.bits_g = uni(a.bits_g);
  L.bits_s = uni(a.bits_s);
  L.c_g = uni(a.c_g);
  L.c_s = uni(a.c_s);
  L.r_g = uni(a.r_g);
  L.r_s = uni(a.r_s);
  L.sal_idx = uni(a.sal_idx);
  L.tv_g = uni(a.tv_g);
  L.tv_s = uni(a.tv_s);
  L.n = uni(a.n);
  L.k = uni(a.k);
  L.s = uni(a.s);
  L.kb = uni(a.kb);
  L.ks = uni(a.ks);
  L.nc_g = uni(a.nc_g);
  L.nc_s = uni(a.nc_s);
  return L;
}

// One segment as seen by the kernels.
struct SegRef {
  const FB_GLOBAL u32x4 *bits;  // element ((tile * nchunks + chunk) * 64 + lane)
  const FB_GLOBAL uint16_t *c;
  const FB_GLOBAL uint16_t *r;
  int64_t len;
  int32_t nchunks;
  int32_t salient;
};

// Branch-free (scalar selects): loop bodies that step through segments stay
// one basic block, so the compiler keeps each chunk's work together.
__device__ __forceinline__ SegRef segment(const ULayer &L, int sidx) {
  const bool g = sidx < L.kb;
  const int b = g ? sidx : sidx - L.kb;
  SegRef r;
  r.bits = (g ? L.bits_g : L.bits_s) + b * (g ? L.tv_g : L.tv_s);
  r.c = (g ? L.c_g : L.c_s) + b * (g ? L.k : L.s);
  r.r = (g ? L.r_g : L.r_s) + b * L.n;
  r.len = g ? L.k : L.s;
  r.nchunks = g ? L.nc_g : L.nc_s;
  r.salient = !g;
  return r;
}

// One segment as the GEMV kernel receives it: base pointers precomputed on
// the host, so that the kernel reads them (scalar loads from its argument
// block, indexed by a uniform segment number) instead of recomputing them.
struct SegDesc {
  const u32x4 *bits;     // tiled words: element (tile * nchunks + chunk) * 64 + lane
  const uint16_t *c;     // fp16 column scales of the segment
  const uint16_t *r;     // fp16 row scales of the segment: [n], or block-wise in the tiled scale
                         // layout, m per lane per chunk: element ((tile * nchunks + chunk) * 64 + lane) * m
  int32_t len;           // columns
  int32_t nchunks;       // ceil(len / 128)
};

// Segment `sidx` (uniform) of a GEMV call, pointers in the global address space.
__device__ __forceinline__ SegRef gemv_segment(const SegDesc (&seg)[kMaxSeg], int kb, int sidx) {
  const SegDesc &d = seg[sidx];
  SegRef r;
  r.bits = (const FB_GLOBAL u32x4 *)(uintptr_t)d.bits;
  r.c = (const FB_GLOBAL uint16_t *)(uintptr_t)d.c;
  r.r = (const FB_GLOBAL uint16_t *)(uintptr_t)d.r;
  r.len = d.len;
  r.nchunks = d.nchunks;
  r.salient = sidx >= kb;
  return r;
}

struct GemvArgs {
  SegDesc seg[kMaxSeg];   // kb global segments, then ks salient ones
  const int32_t *idx_or_dummy;  // sal_idx, or a valid one-element array when ks == 0
  const uint16_t *x;      // fp16 [batch][k]
  uint16_t *y;            // fp16 [batch][n]
  uint64_t *acc;          // [batch][n_pad] split-reduction words; zero between calls
  int64_t n;              // output rows
  int64_t k;              // input columns (x row stride)
  int64_t n_pad;          // row_tiles * 64
  int32_t kb, ks;
  int32_t cpb;            // longest column range, in chunks
  int32_t tb;             // chunks whose tables the dynamic LDS holds (>= cpb: the whole range at once)
  int32_t row_tiles;
  int32_t splits;         // column ranges (the grid's y dimension; x is the row block)
  int32_t batch;
  int32_t sal16;          // block-wise: 16 salient row-scale groups per chunk (8 columns each), else 8
  // Column range of split sp, decoded on the host (range_word): segment in
  // bits 0-2, chunk count in bits 3-8, first chunk in bits 9-31.  Every
  // segment is cut into equal-as-possible ranges of consecutive chunks.
  uint32_t range[kMaxSplits];
};

__host__ __device__ constexpr uint32_t range_word(int sg, int c_lo, int nch) {
  return (uint32_t)sg | ((uint32_t)nch << 3) | ((uint32_t)c_lo << 9);
}

typedef void (*gemv_fn)(const GemvArgs);

// GEMV kernel instances, one translation unit per table width g, row-scale
// format (rs 0: per row, 1: block-wise) and table entry type (t32: fp32,
// t16: fp16): the instance for batch width nb, waves per workgroup and
// prefetch depth pf, or nullptr.
gemv_fn gemv_pick_g4_rs0_t32(int nb, int waves, int pf);
gemv_fn gemv_pick_g4_rs1_t32(int nb, int waves, int pf);
gemv_fn gemv_pick_g8_rs0_t32(int nb, int waves, int pf);
gemv_fn gemv_pick_g8_rs1_t32(int nb, int waves, int pf);
gemv_fn gemv_pick_g4_rs0_t16(int nb, int waves, int pf);
gemv_fn gemv_pick_g4_rs1_t16(int nb, int waves, int pf);
gemv_fn gemv_pick_g8_rs0_t16(int nb, int waves, int pf);
gemv_fn gemv_pick_g8_rs1_t16(int nb, int waves, int pf);
// g = 4, one batch row, per-row scales, fp32 entries, ks (2 or 4) waves per
// row tile: the instance for waves per workgroup and prefetch depth pf.
gemv_fn gemv_pick_g4_ks(int ks, int waves, int pf);
// The g = 8 kernel with bank-private tables (one batch row, per-row scales,
// fp32 entries) for column ranges of up to `regions` (1, or 2 for region 2)
// regions of `region` (2 or 4) chunks.
gemv_fn gemv_pick_g8_banked(int region, int regions, int waves);

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

#define FB_LDS __attribute__((address_space(3)))

// fp32 at LDS byte address `addr`: the address goes to the instruction as is
// (constant parts in its offset field), with no base added per access.
__device__ __forceinline__ float lds_f32(uint32_t addr) {
  return *reinterpret_cast<const FB_LDS float *>((uintptr_t)addr);
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const FB_LDS void *)p;
}

// Byte `kk` of v, zero-extended (v_perm_b32: opaque to the optimiser, one VALU op).
template <int kk>
__device__ __forceinline__ uint32_t byte_of(uint32_t v) {
  return __builtin_amdgcn_perm(0u, v, 0x0c0c0c00u | kk);
}

// Table address of one lookup: byte kk of v (a pattern already scaled to a
// byte offset) in bits 0-7, bits 8-23 taken from `base`, the LDS offset of the
// chunk's tables (a multiple of 256 below 2^24): a single v_perm_b32.
template <int kk>
__device__ __forceinline__ uint32_t addr_of(uint32_t v, uint32_t base) {
  return __builtin_amdgcn_perm(base, v, 0x0c060500u | kk);
}

// fp16 at LDS byte address `addr` (raw bits, zero-extended).
__device__ __forceinline__ uint32_t lds_u16(uint32_t addr) {
  return *reinterpret_cast<const FB_LDS uint16_t *>((uintptr_t)addr);
}

// acc + (the fp16 value in the low half of h), one rounding: v_fma_mix_f32
// computes acc + h * 1.0 with h read as fp16, the same single instruction and
// rounding as a fp32 add of the converted value.
__device__ __forceinline__ float add_f16_bits(float acc, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(acc));
  return r;
}

// acc + (the fp16 value in the high half of h): the same instruction reading
// the upper half (op_sel).
__device__ __forceinline__ float add_f16_hi_bits(float acc, uint32_t h) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(acc));
  return r;
}

__device__ __forceinline__ uint32_t lds_u32(uint32_t addr) {
  return *reinterpret_cast<const FB_LDS uint32_t *>((uintptr_t)addr);
}

// Table entries of EB bytes: 4 = fp32, 2 = fp16 (quantised tables).
template <int EB>
__device__ __forceinline__ float add_entry(float acc, uint32_t addr) {
  if constexpr (EB == 4) {
    return acc + lds_f32(addr);
  } else {
    return add_f16_bits(acc, lds_u16(addr));
  }
}

template <int EB>
__device__ __forceinline__ float entry_value(uint32_t addr) {
  if constexpr (EB == 4) {
    return lds_f32(addr);
  } else {
    return add_f16_bits(0.0f, lds_u16(addr));  // exact conversion
  }
}

// Byte offsets (pattern * EB) of the 4-bit patterns of a word: A holds
// nibbles 0, 2, 4, 6 and B nibbles 1, 3, 5, 7, one per byte.
template <int EB>
__device__ __forceinline__ uint32_t nibbles_even(uint32_t w) {
  return EB == 4 ? (w << 2) & 0x3c3c3c3cu : (w << 1) & 0x1e1e1e1eu;
}
template <int EB>
__device__ __forceinline__ uint32_t nibbles_odd(uint32_t w) {
  return EB == 4 ? (w >> 2) & 0x3c3c3c3cu : (w >> 3) & 0x1e1e1e1eu;
}
// Byte offset (pattern * EB) of byte kk of a word (an 8-bit pattern).
template <int EB, int kk>
__device__ __forceinline__ uint32_t byte_pattern(uint32_t w) {
  constexpr int SH = EB == 4 ? 2 : 1;
  if constexpr (kk == 0) {
    return (w << SH) & (0xffu << SH);
  } else {
    return (w >> (8 * kk - SH)) & (0xffu << SH);
  }
}

// fp16 tables of several batch rows at g = 4, in batch-row pairs: in a
// chunk's table block, dword ((q * 32 + j) * 16 + p) holds entry p of
// sub-vector j for batch row 2q (low half) and row 2q + 1 (high half); the
// block has the size of the unpaired fp16 tables.
__host__ __device__ constexpr int pair_table_dword(int q, int j, int p) { return (q * 32 + j) * 16 + p; }

// Accumulate the lookups of one 32-bit word (32 columns) of one row.  `base`
// is the LDS byte address of the chunk's table block (a multiple of 256, or of
// 1024 for 256-entry tables, below 2^24); j0 is the first sub-vector of the
// word.  Sub-vector j of batch row b has its TAB-entry table at
// base + ((b * SUB + j) * TAB) * EB.  Even sub-vectors (low nibbles / bytes 0
// and 2) go to acc0, odd ones to acc1: two independent chains of fp32 adds,
// or one when the caller passes the same array twice (wide batches, whose NB
// rows already give independent chains).
template <int G, int NB, int EB, bool PAIRS = false>
__device__ __forceinline__ void lookup_word(uint32_t w, uint32_t base, float (&acc0)[NB], float (&acc1)[NB],
                                            int j0) {
  constexpr int SUB = kChunkCols / G;
  constexpr int TAB = 1 << G;
  if constexpr (PAIRS) {
    // fp16 tables in batch-row pairs (pair_table_dword): one dword read gives
    // the entries of rows 2q (low half) and 2q + 1 (high half), so a lookup
    // returns 2 bytes of LDS data per batch row instead of 4.  Each row still
    // adds its even sub-vector's entry, then its odd one's, as above.
    static_assert(G == 4 && EB == 2 && NB % 2 == 0, "pairs: g = 4, fp16 entries, an even batch width");
    const uint32_t A = nibbles_even<4>(w);
    const uint32_t B = nibbles_odd<4>(w);
    const uint32_t ia[4] = {addr_of<0>(A, base), addr_of<1>(A, base), addr_of<2>(A, base), addr_of<3>(A, base)};
    const uint32_t ib[4] = {addr_of<0>(B, base), addr_of<1>(B, base), addr_of<2>(B, base), addr_of<3>(B, base)};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int q = 0; q < NB / 2; ++q) {
        const int off0 = ((q * SUB + j0 + 2 * kk) * TAB) * 4;
        const uint32_t e = lds_u32(ia[kk] + off0);
        const uint32_t f = lds_u32(ib[kk] + off0 + TAB * 4);
        acc0[2 * q] = add_f16_bits(acc0[2 * q], e);
        acc0[2 * q + 1] = add_f16_hi_bits(acc0[2 * q + 1], e);
        acc1[2 * q] = add_f16_bits(acc1[2 * q], f);
        acc1[2 * q + 1] = add_f16_hi_bits(acc1[2 * q + 1], f);
      }
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  } else if constexpr (G == 4) {
    const uint32_t A = nibbles_even<EB>(w);
    const uint32_t B = nibbles_odd<EB>(w);
    const uint32_t ia[4] = {addr_of<0>(A, base), addr_of<1>(A, base), addr_of<2>(A, base), addr_of<3>(A, base)};
    const uint32_t ib[4] = {addr_of<0>(B, base), addr_of<1>(B, base), addr_of<2>(B, base), addr_of<3>(B, base)};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + 2 * kk) * TAB) * EB;
        acc0[b] = add_entry<EB>(acc0[b], ia[kk] + off0);
        acc1[b] = add_entry<EB>(acc1[b], ib[kk] + off0 + TAB * EB);
      }
      // wide batches: at most 2 * NB table reads in flight per step, or the
      // scheduler hoists all of them and runs out of registers
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  } else {
    // byte kk of w is the 8-bit pattern of sub-vector j0 + kk
    const uint32_t ix[4] = {byte_pattern<EB, 0>(w) | base, byte_pattern<EB, 1>(w) | base,
                            byte_pattern<EB, 2>(w) | base, byte_pattern<EB, 3>(w) | base};
#pragma unroll
    for (int kk = 0; kk < 4; kk += 2) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + kk) * TAB) * EB;
        acc0[b] = add_entry<EB>(acc0[b], ix[kk] + off0);
        acc1[b] = add_entry<EB>(acc1[b], ix[kk + 1] + off0 + TAB * EB);
      }
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  }
}

// Block-wise variant: the lookups of each byte of w (8 columns: two
// sub-vectors at g = 4, one at g = 8) are summed and added into `part`
// scaled by that byte's row scale s0..s3.
template <int G, int NB, int EB>
__device__ __forceinline__ void lookup_word_scaled(uint32_t w, uint32_t base, float (&part)[NB], int j0, float s0,
                                                   float s1, float s2, float s3) {
  constexpr int SUB = kChunkCols / G;
  constexpr int TAB = 1 << G;
  const float sc[4] = {s0, s1, s2, s3};
  if constexpr (G == 4) {
    const uint32_t A = nibbles_even<EB>(w);
    const uint32_t B = nibbles_odd<EB>(w);
    const uint32_t ia[4] = {addr_of<0>(A, base), addr_of<1>(A, base), addr_of<2>(A, base), addr_of<3>(A, base)};
    const uint32_t ib[4] = {addr_of<0>(B, base), addr_of<1>(B, base), addr_of<2>(B, base), addr_of<3>(B, base)};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + 2 * kk) * TAB) * EB;
        const float t = add_entry<EB>(entry_value<EB>(ia[kk] + off0), ib[kk] + off0 + TAB * EB);
        part[b] = fmaf(sc[kk], t, part[b]);
      }
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  } else {
    const uint32_t ix[4] = {byte_pattern<EB, 0>(w) | base, byte_pattern<EB, 1>(w) | base,
                            byte_pattern<EB, 2>(w) | base, byte_pattern<EB, 3>(w) | base};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + kk) * TAB) * EB;
        part[b] = fmaf(sc[kk], entry_value<EB>(ix[kk] + off0), part[b]);
      }
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  }
}

// Dynamic LDS of the GEMV kernel: [cpb][NB][SUB][TAB] tables of eb-byte
// entries (fp32, or fp16 when quantised), then [cpb][NB][128] fp32
// scale-fused inputs, then a 64-float sink for the stores of unused input
// slots.
constexpr int kLdsBudget = 80 * 1024;  // per workgroup: two workgroups per CU
constexpr int kMaxCpb = 32;            // chunks per workgroup
constexpr int kLdsSink = 64 * 4;

__host__ __device__ constexpr int lds_per_chunk(int g, int nb, int eb) {
  return nb * (kChunkCols / g) * (1 << g) * eb + nb * kChunkCols * 4;
}

__host__ __device__ constexpr int lds_bytes(int g, int nb, int cpb, int eb) {
  return cpb * lds_per_chunk(g, nb, eb) + kLdsSink;
}

// LDS of the g = 8 bank-private-table kernel over ranges of nreg regions of r
// chunks: one region's tables (16 r x 256 fp32), then the scale-fused inputs
// of all the range's chunks (nreg r x 128 fp32).
__host__ __device__ constexpr int banked_lds_bytes(int r, int nreg) {
  return r * 16 * 256 * 4 + nreg * r * kChunkCols * 4;
}

__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Table-build inputs (c * x) each thread stages per round (the first round's
// loads are all in flight at once): with one batch row 4 (4 waves) or 2 (8
// waves), so that one round covers an 8-chunk range; 8 for several rows.
// Longer ranges stage in further rounds.
__host__ __device__ constexpr int stage_items(int nb, int waves) { return nb == 1 ? (waves >= 8 ? 2 : 4) : 8; }

// Most chunks one workgroup may take for table width g, batch width nb and
// eb-byte entries: its tables and inputs must fit the LDS budget.
__host__ __device__ constexpr int cpb_cap(int g, int nb, int eb) {
  return cmin(kMaxCpb, (kLdsBudget - kLdsSink) / lds_per_chunk(g, nb, eb)) < 1
             ? 1
             : cmin(kMaxCpb, (kLdsBudget - kLdsSink) / lds_per_chunk(g, nb, eb));
}

// Chunks of weights in flight per wave for ranges of up to cpb chunks, for
// several batch rows and for g = 8 outside the bank-private kernel (one batch
// row at g = 4 takes two or three whatever the range length: make_plan).
__host__ __device__ constexpr int prefetch_depth(int cpb) { return cpb >= 4 ? 4 : 2; }

// The column range of split sp (uniform): segment sg, chunks [c_lo, c_lo +
// nch) of it, from the host-decoded table in the argument block.
struct ColRange {
  SegRef S;
  int sg, c_lo, nch;
};

__device__ __forceinline__ ColRange column_range(const GemvArgs &a, int sp) {
  const uint32_t w = a.range[sp];
  ColRange c;
  c.sg = (int)(w & 7u);
  c.nch = (int)((w >> 3) & 63u);
  c.c_lo = (int)(w >> 9);
  c.S = gemv_segment(a.seg, a.kb, c.sg);
  return c;
}

// One g = 8 table build unit: the 16 entries p = (hb << 7) | (m << 3) | q3,
// m = 0..15, of the sub-vector whose scale-fused inputs are v[0..7], for the
// unit un = (hb << 3) | q3.  Entry p is the sum, in this order, of
// sgn_7 v_7, sgn_0 v_0, sgn_1 v_1, ..., sgn_6 v_6 (sgn_t = +1 where bit t of
// p is set, -1 where it is clear); the tree below shares the leading terms,
// so every entry rounds exactly like that sequence, and the units with hb = 0
// are the exact negations of those with hb = 1 (LUT[~p] = -LUT[p]).
__device__ __forceinline__ void g8_unit_entries(const float *v, int un, float (&e)[16]) {
  const float4 va = *reinterpret_cast<const float4 *>(v);
  const float4 vb = *reinterpret_cast<const float4 *>(v + 4);
  const int hb = un >> 3, q3 = un & 7;
  float base = hb ? vb.w : -vb.w;
  base = (q3 & 1) ? base + va.x : base - va.x;
  base = (q3 & 2) ? base + va.y : base - va.y;
  base = (q3 & 4) ? base + va.z : base - va.z;
  const float l1[2] = {base - va.w, base + va.w};
  float l2[4], l3[8];
#pragma unroll
  for (int i = 0; i < 2; ++i) l2[i] = l1[i] - vb.x, l2[i + 2] = l1[i] + vb.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) l3[i] = l2[i] - vb.y, l3[i + 4] = l2[i] + vb.y;
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = l3[i] - vb.z, e[i + 8] = l3[i] + vb.z;
}

// The output of one lane's row: part[b] is the row's partial sum over the
// workgroup's column range for batch row b, already row-scaled.
//
// One range per row (splits == 1): a direct fp16 store.  Several ranges:
// every workgroup adds its partial of each row into that row's packed word
// with one agent-scope atomic (performed at the memory side, coherent across
// XCDs).  The atomic returns the previous word, so the lane that brings the
// last of `splits` contributions knows it is last and holds the complete sum:
// it writes y and clears the word for the next call.  No workgroup waits for
// another, and since integer addition is exact the result does not depend on
// the order in which the splits arrive.  A partial outside the fixed-point
// range first sets the word's overflow flag (a rare second atomic on the same
// word, ordered before the add), and the row is written as NaN.
//
// With several batch rows, all NB atomics are issued before any result is
// examined, so that their round trips overlap instead of queueing one behind
// the other.
template <int NB>
__device__ __forceinline__ void finish_rows(const GemvArgs &a, int row, bool row_ok, const float (&part)[NB]) {
  if (a.splits == 1) {
    if (row_ok) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (b < a.batch) a.y[(int64_t)b * a.n + row] = f2h(part[b]);
    }
    return;
  }
  if (!row_ok) return;
  uint64_t contrib[NB], old[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float scaled = part[b] * kFixScale;
    const bool ovf = !(fabsf(scaled) < kFixLimit);      // NaN and inf overflow too
    const int64_t q = ovf ? 0 : __float2ll_rn(scaled);  // an overflowing partial adds 0 (the row is NaN)
    contrib[b] = (uint64_t)(q + kFixBias);
    old[b] = 0;
    if (b < a.batch) {
      uint64_t *slot = a.acc + (int64_t)b * a.n_pad + row;
      if (ovf) __hip_atomic_fetch_or(slot, kOverflow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old[b] = __hip_atomic_fetch_add(slot, contrib[b] + kOneArrival, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < a.batch && (int)((old[b] >> kCountShift) & 0xffu) == a.splits - 1) {
      const int64_t total = (int64_t)((old[b] & kValueMask) + contrib[b]) - (int64_t)a.splits * kFixBias;
      a.y[(int64_t)b * a.n + row] = (old[b] & kOverflow) ? kHalfNaN : f2h(__ll2float_rn(total) * kFixInv);
      __hip_atomic_store(a.acc + (int64_t)b * a.n_pad + row, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

}  // namespace fluxbin
