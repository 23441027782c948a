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
//     the SAME 2^g-entry table at each step, so table reads are broadcasts
//     within 16 (g=4) or 256 (g=8) consecutive dwords;
//   * weights are streamed from the TILED layout: a wave's 16-byte-per-lane
//     load of one 128-column chunk is 1 KiB of contiguous memory, loaded with
//     non-temporal 128-bit loads (streamed once, kept out of L2);
//   * a workgroup of WAVES waves shares the tables of CPB consecutive chunks of
//     the concatenated column space of all segments; a grid of
//     row_blocks x splits workgroups covers the layer;
//   * splits > 1: each workgroup adds its fp32 partial of every row, as an
//     exact fixed-point integer, into a per-row 64-bit word that also counts
//     arrivals; the lane whose atomic brings the last contribution writes the
//     fp16 row.  One launch does the whole GEMV, the result is bitwise
//     deterministic, and no workgroup ever waits for another.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fluxbin {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkCols = 128;  // columns per chunk = 4 sign words per row
constexpr int kTileRows = 64;    // rows per tile = one wave, one row per lane
constexpr int kMaxSeg = 6;       // kb <= 4 global + ks <= 2 salient bases
// Split reduction: one 64-bit word per (batch row, output row) holds the
// number of contributions so far (top 8 bits) and the sum of the
// contributions' biased fixed-point values (low 56 bits).  Each contribution
// is round(partial * 2^30), clamped to |.| < 2^47, plus a bias of 2^47, so it
// lies in [0, 2^48) and up to 255 of them never carry into the count.
constexpr int kCountShift = 56;
constexpr int kMaxSplits = 255;
constexpr uint64_t kOneArrival = 1ull << kCountShift;
constexpr uint64_t kValueMask = kOneArrival - 1;
constexpr int64_t kFixBias = 1ll << 47;
constexpr float kFixScale = 1073741824.0f;          // 2^30
constexpr float kFixInv = 1.0f / 1073741824.0f;     // 2^-30
constexpr float kFixClamp = 140737479966720.0f;     // 2^47 - 2^23, the largest float below 2^47

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

// Segment of chunk gc of the concatenated chunk space, and the chunk's index inside it.
__device__ __forceinline__ int seg_of(const ULayer &L, int gc, int *cis) {
  const int gch = L.kb * L.nc_g;
  if (gc < gch) {
    const int b = gc / L.nc_g;
    *cis = gc - b * L.nc_g;
    return b;
  }
  const int b = (gc - gch) / L.nc_s;
  *cis = gc - gch - b * L.nc_s;
  return L.kb + b;
}

struct GemvArgs {
  SegDesc seg[kMaxSeg];   // kb global segments, then ks salient ones
  LayerArgs L;
  const int32_t *idx_or_dummy;  // sal_idx, or a valid one-element array when ks == 0
  int32_t cpb;            // 128-column chunks per workgroup (tables sized in dynamic LDS)
  int32_t total_chunks;
  int32_t row_tiles;
  int32_t row_blocks;
  int32_t splits;
  int32_t batch;
  int64_t n_pad;          // row_tiles * 64
  const uint16_t *x;      // fp16 [batch][k]
  uint16_t *y;            // fp16 [batch][n]
  uint64_t *acc;          // [batch][n_pad] packed (arrivals, fixed-point sum); zero between calls
  // Workgroup ranges: splits [0, gsplits) cover chunks [0, gchunks) and the
  // rest cover [gchunks, total_chunks), cpb chunks each (the last range of
  // each part may be shorter).  Per-row scales: one part (gsplits = splits,
  // gchunks = total_chunks).  Block-wise scales: global and salient chunks
  // never share a workgroup (gchunks = kb * ceil(k / 128)).
  int32_t gsplits;
  int32_t gchunks;
  int32_t sal16;          // block-wise: 16 salient row-scale groups per chunk (8 columns each), else 8
};

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

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// Value number s of six scalars (s uniform).  Plain SSA values, never an
// aggregate: an array or struct indexed by a runtime segment number would be
// placed in LDS or scratch memory by the compiler.
__device__ __forceinline__ float pick6(int s, float v0, float v1, float v2, float v3, float v4, float v5) {
  float r = v0;
  r = s == 1 ? v1 : r;
  r = s == 2 ? v2 : r;
  r = s == 3 ? v3 : r;
  r = s == 4 ? v4 : r;
  r = s == 5 ? v5 : r;
  return r;
}

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

// Accumulate the lookups of one 32-bit word (32 columns) of one row.  `base`
// is the LDS byte address of the chunk's table block (a multiple of 256, or of
// 512 for 256-entry tables, below 2^24); j0 is the first sub-vector of the
// word.  Sub-vector j of batch row b has its TAB-entry table at
// base + ((b * SUB + j) * TAB) * EB.
template <int G, int NB, int EB>
__device__ __forceinline__ void lookup_word(uint32_t w, uint32_t base, float (&acc)[NB], int j0) {
  constexpr int SUB = kChunkCols / G;
  constexpr int TAB = 1 << G;
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
        acc[b] = add_entry<EB>(acc[b], ia[kk] + off0);
        acc[b] = add_entry<EB>(acc[b], ib[kk] + off0 + TAB * EB);
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
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + kk) * TAB) * EB;
        acc[b] = add_entry<EB>(acc[b], ix[kk] + off0);
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

// Segment and chunk-in-segment stepped to the next chunk when step is 1
// (unchanged when 0), in integer arithmetic: uniform booleans are held as lane
// masks, and turning them back into integers takes vector instructions.
__device__ __forceinline__ void next_chunk(const ULayer &L, int &sg, int &cis, int step = 1) {
  const int n1 = cis + step;                                // <= the segment's chunk count
  const int nc = sg < L.kb ? L.nc_g : L.nc_s;
  const int wrap = (int)((uint32_t)(nc - n1 - 1) >> 31);    // 1 when n1 == nc
  cis = n1 - (nc & -wrap);
  sg += wrap;
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

constexpr int kMaxItems = 8;  // table-build inputs per thread (registers)

__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Most chunks one workgroup may take for table width g, batch width nb,
// `waves` waves and eb-byte entries: its tables must fit the LDS budget, and
// its table-build inputs (nb * 128 per chunk) at most kMaxItems per thread.
__host__ __device__ constexpr int cpb_cap(int g, int nb, int waves, int eb) {
  return cmin(cmin(kMaxCpb, (kLdsBudget - kLdsSink) / lds_per_chunk(g, nb, eb)),
              kMaxItems * waves * 64 / (nb * kChunkCols)) < 1
             ? 1
             : cmin(cmin(kMaxCpb, (kLdsBudget - kLdsSink) / lds_per_chunk(g, nb, eb)),
                    kMaxItems * waves * 64 / (nb * kChunkCols));
}

// Prefetch depth for a workgroup range of cpb chunks: the deepest of 8, 4, 2
// that the range fills (a shorter range would re-read its last chunk).
__host__ __device__ constexpr int prefetch_depth(int cpb) { return cpb >= 8 ? 8 : cpb >= 4 ? 4 : 2; }

// Most chunks a kernel instance with prefetch depth pf serves.
__host__ __device__ constexpr int cpb_for_depth(int pf, int cap) { return pf == 8 ? cap : cmin(2 * pf - 1, cap); }

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

}  // namespace fluxbin
