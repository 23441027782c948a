// kernels.hpp -- gfx950 (CDNA4) kernels of the FluxBin LUT GEMV.
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
//     segment after accumulation;
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
  const uint16_t *r;     // fp16 row scales of the segment
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
};

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

// Accumulate the lookups of one 32-bit word (32 columns) of one row.  `base`
// is the LDS byte address of the chunk's table block (a multiple of 256
// below 2^24); j0 is the first sub-vector of the word.  Sub-vector j of batch
// row b has its TAB-entry table at base + ((b * SUB + j) * TAB) * 4.
template <int G, int NB>
__device__ __forceinline__ void lookup_word(uint32_t w, uint32_t base, float (&acc)[NB], int j0) {
  constexpr int SUB = kChunkCols / G;
  constexpr int TAB = 1 << G;
  if constexpr (G == 4) {
    // nibble m of w at bits [4m, 4m+4); A holds nibbles 0,2,4,6 and B nibbles
    // 1,3,5,7, each as a byte offset (index * 4) into a 16-entry fp32 table.
    const uint32_t A = (w << 2) & 0x3c3c3c3cu;
    const uint32_t B = (w >> 2) & 0x3c3c3c3cu;
    const uint32_t ia[4] = {addr_of<0>(A, base), addr_of<1>(A, base), addr_of<2>(A, base), addr_of<3>(A, base)};
    const uint32_t ib[4] = {addr_of<0>(B, base), addr_of<1>(B, base), addr_of<2>(B, base), addr_of<3>(B, base)};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + 2 * kk) * TAB) * 4;
        acc[b] += lds_f32(ia[kk] + off0);
        acc[b] += lds_f32(ib[kk] + off0 + TAB * 4);
      }
      // wide batches: at most 2 * NB table reads in flight per step, or the
      // scheduler hoists all of them and runs out of registers
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  } else {
    // byte kk of w is the 8-bit pattern of sub-vector j0 + kk; table offset = pattern * 4
    uint32_t ix[4];
    ix[0] = ((w << 2) & 0x3fcu) | base;
    ix[1] = ((w >> 6) & 0x3fcu) | base;
    ix[2] = ((w >> 14) & 0x3fcu) | base;
    ix[3] = ((w >> 22) & 0x3fcu) | base;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int off0 = ((b * SUB + j0 + kk) * TAB) * 4;
        acc[b] += lds_f32(ix[kk] + off0);
      }
      if constexpr (NB >= 8) asm volatile("" ::: "memory");
    }
  }
}

// Segment and chunk-in-segment stepped to the next chunk (when `step`),
// branch-free: scalar selects, so that loop bodies stay one basic block.
__device__ __forceinline__ void next_chunk(const ULayer &L, int &sg, int &cis, bool step = true) {
  const int n1 = cis + 1;
  const bool wrap = n1 == (sg < L.kb ? L.nc_g : L.nc_s);
  cis = step ? (wrap ? 0 : n1) : cis;
  sg = step ? sg + (int)wrap : sg;
}

// Dynamic LDS of the GEMV kernel: [cpb][NB][SUB][TAB] fp32 tables, then
// [cpb][NB][128] fp32 scale-fused inputs, then a 64-float sink for the
// stores of unused input slots.
constexpr int kLdsBudget = 80 * 1024;  // per workgroup: two workgroups per CU
constexpr int kMaxCpb = 32;            // chunks per workgroup
constexpr int kLdsSink = 64 * 4;

__host__ __device__ constexpr int lds_per_chunk(int g, int nb) {
  return nb * (kChunkCols / g) * (1 << g) * 4 + nb * kChunkCols * 4;
}

__host__ __device__ constexpr int lds_bytes(int g, int nb, int cpb) { return cpb * lds_per_chunk(g, nb) + kLdsSink; }

constexpr int kMaxItems = 8;  // table-build inputs per thread (registers)

__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Most chunks one workgroup may take for table width g, batch width nb and
// `waves` waves: its tables must fit the LDS budget, and its table-build
// inputs (nb * 128 per chunk) at most kMaxItems per thread.
__host__ __device__ constexpr int cpb_cap(int g, int nb, int waves) {
  return cmin(cmin(kMaxCpb, (kLdsBudget - kLdsSink) / lds_per_chunk(g, nb)), kMaxItems * waves * 64 / (nb * kChunkCols)) < 1
             ? 1
             : cmin(cmin(kMaxCpb, (kLdsBudget - kLdsSink) / lds_per_chunk(g, nb)), kMaxItems * waves * 64 / (nb * kChunkCols));
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

template <int G, int NB, int WAVES, int PF>
__global__ __launch_bounds__(WAVES * 64) void lut_gemv_kernel(const GemvArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int SUB = kChunkCols / G;      // sub-vectors per chunk
  constexpr int TAB = 1 << G;              // full table entries
  constexpr int HALF = TAB / 2;
  constexpr int WPL = kChunkCols / 32;     // words per lane per chunk (4)
  constexpr int CTB = NB * SUB * TAB * 4;  // table bytes of one chunk (all batch rows)
  static_assert(CTB % 256 == 0, "chunk table blocks must be 256-byte aligned");
  static_assert(NT % HALF == 0, "thread count must be a multiple of the half-table size");
  static_assert(PF >= 1 && PF <= 8, "prefetch depth");
  extern __shared__ __align__(1024) float smem[];

  const ULayer L = uniform_layer(a.L);  // scalar registers: field selects stay scalar
  const int cpb = a.cpb;
  float *s_tab = smem;
  const uint32_t tab_base = lds_addr(s_tab);  // 1024-aligned (table addresses are merged bytewise)
  float *s_v = smem + cpb * (CTB / 4);
  float *s_sink = s_v + cpb * NB * kChunkCols;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address arithmetic
  const int rb = blockIdx.x % a.row_blocks;
  const int sp = blockIdx.x / a.row_blocks;
  const int tile = rb * WAVES + wave;
  const bool tile_ok = tile < a.row_tiles;
  const int ltile = min(tile, a.row_tiles - 1);  // waves past the last tile read the last one, store nothing
  const int row = tile * kTileRows + lane;
  const bool row_ok = tile_ok && row < L.n;
  const int rrow = row_ok ? row : 0;
  const int c0 = sp * cpb;
  const int nch = min(cpb, a.total_chunks - c0);

  // Chunk map of the workgroup's range, one chunk per lane (nch <= 32 < 64):
  // lane l holds the segment and chunk-in-segment of chunk c0 + l, and a
  // uniform chunk's entry is read out of its lane.
  int mcis;
  const int mseg = seg_of(L, c0 + min(lane, nch - 1), &mcis);
  auto seg_at = [&](int ch) { return __builtin_amdgcn_readlane(mseg, ch); };
  auto cis_at = [&](int ch) { return __builtin_amdgcn_readlane(mcis, ch); };
  const int s0 = seg_at(0), cis0 = cis_at(0), s_last = seg_at(nch - 1);

  // The rest of the kernel exists twice: for workgroups whose range holds
  // global segments only, and for those that reach a salient segment (these
  // fetch gather indices before their activations).  Separate copies keep
  // each copy's memory waits exact: where two paths join, the compiler's
  // waits are those of the slower path.  The branch is uniform.
  auto body = [&](auto sal_tag) {
    constexpr bool SAL = decltype(sal_tag)::value;
    // Vector-memory loads complete in issue order, and the compiler's waits are
    // exact only for loads issued on every path of a branch-free stretch.  The
    // prologue requests row scales, column scales and activations first and PF
    // chunks of weights after them (a workgroup with fewer chunks re-reads its
    // last one), so that waiting for the table-build inputs never waits for
    // HBM and the weights stay in flight during the table build.  A workgroup
    // whose range reaches a salient segment fetches gather indices (VCM)
    // instead of activations before the weights, and the activations after.
    const FB_GLOBAL int32_t *uidx = uni(a.idx_or_dummy);
    const FB_GLOBAL uint16_t *ux = uni(a.x);
    // row scales of the segments this workgroup touches (s0 .. s_last, consecutive)
    auto rptr = [&](int j) { return gemv_segment(a.seg, L.kb, min(s0 + j, s_last)).r + rrow; };
    const uint16_t rr0 = *rptr(0), rr1 = *rptr(1), rr2 = *rptr(2), rr3 = *rptr(3), rr4 = *rptr(4), rr5 = *rptr(5);

    u32x4 wb[PF];
    int ps = s0, pcis = cis0, pidx = 0;  // next chunk to load and its index in the range
    auto load_next = [&]() -> u32x4 {
      const SegRef S = gemv_segment(a.seg, L.kb, ps);
      const FB_GLOBAL u32x4 *base = S.bits + ((int64_t)ltile * S.nchunks + pcis) * kTileRows;
      const u32x4 w = __builtin_nontemporal_load(base + lane);
      const bool step = pidx < nch - 1;  // past the last chunk the last one is read again
      next_chunk(L, ps, pcis, step);
      pidx += (int)step;
      return w;
    };
    auto issue_weights = [&]() {
#pragma unroll
      for (int u = 0; u < PF; ++u) wb[u] = load_next();
    };

    // Table-build items (chunk, batch row, column) of the range: item e is
    // handled by thread e % NT; a wave's 64 items share chunk and batch row.
    // Every item slot loads (items past the range re-read the last chunk's
    // inputs and are dropped).
    constexpr int CMAX = cpb_for_depth(PF, cpb_cap(G, NB, WAVES));  // chunks, at most
    constexpr int VPT = (CMAX * NB * kChunkCols + NT - 1) / NT;  // items per thread, at most
    static_assert(VPT <= kMaxItems, "table-build inputs per thread");
    static_assert(kChunkCols % 64 == 0 && NT % 64 == 0, "a wave's items must share chunk and batch row");
    const int items = nch * NB * kChunkCols;
    // Per item: uniform row pointer into x, per-lane 32-bit column offsets
    // (loads then take a scalar base and a 32-bit vector offset).
    bool live[VPT], sal[VPT];
    const FB_GLOBAL uint16_t *xrow[VPT];
    uint32_t ccl[VPT];
    uint32_t cvl[VPT], xvl[VPT];  // 32-bit: the compiler would otherwise pack pairs, waiting early
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int ebase = min(i * NT + wave * 64, items - 64);  // uniform
      const int ch = ebase / (NB * kChunkCols);
      const int b = (ebase / kChunkCols) % NB;
      const int sg = seg_at(ch);
      const int cis = cis_at(ch);
      const SegRef S = gemv_segment(a.seg, L.kb, sg);
      const bool brow = b < a.batch;  // uniform; batch rows past `batch` do not exist
      const uint32_t cc = (uint32_t)(cis * kChunkCols + (ebase & (kChunkCols - 1)) + lane);
      live[i] = brow & (cc < (uint32_t)S.len);  // non-short-circuit: a select, not a branch
      sal[i] = S.salient;
      ccl[i] = live[i] ? cc : 0u;
      xrow[i] = ux + (brow ? b : 0) * L.k;
      cvl[i] = S.c[ccl[i]];
    }
    // Inputs to LDS.  No select or branch takes a loaded value as an operand
    // (the compiler would turn it into a branch around the load): unused slots
    // are zeroed by masking the fp16 bits and stored to the sink.
    float rv0, rv1, rv2, rv3, rv4, rv5;  // row scales as fp32
    auto stage = [&]() {
      rv0 = h2f(rr0), rv1 = h2f(rr1), rv2 = h2f(rr2), rv3 = h2f(rr3), rv4 = h2f(rr4), rv5 = h2f(rr5);
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t m = live[i] ? 0xffffu : 0u;
        float *dst = i * NT + wave * 64 < items ? s_v + i * NT + tid : s_sink + lane;
        *dst = h2f((uint16_t)(cvl[i] & m)) * h2f((uint16_t)(xvl[i] & m));
      }
    };
    // sched_barrier: the scheduler must not move work that waits for earlier
    // loads above the weight requests (that wait would hold them back).
    if constexpr (!SAL) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) xvl[i] = xrow[i][ccl[i]];
      __builtin_amdgcn_sched_barrier(0);
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
      stage();
      asm volatile("; lut_gemv prologue: global segments" ::: "memory");
    } else {
      uint32_t gi[VPT];
#pragma unroll
      for (int i = 0; i < VPT; ++i) gi[i] = (uint32_t)uidx[sal[i] ? ccl[i] : 0u];
      __builtin_amdgcn_sched_barrier(0);
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t sm = 0u - (uint32_t)sal[i];  // all ones on salient items
        xvl[i] = xrow[i][ccl[i] + ((gi[i] - ccl[i]) & sm)];
      }
      stage();
      asm volatile("; lut_gemv prologue: salient segments" ::: "memory");
    }
    __syncthreads();

    // Tables: the half with the top input at +1 is summed, the rest negated.
    // Entry q of a sub-vector is v_{G-1} + sum_{i<G-1} sgn_i(q) * v_i in that
    // order; sgn_i = +-1 exactly, so each fma rounds like the add or subtract.
    // NT is a multiple of HALF, so a thread's pattern q is fixed.
    {
      const int q = tid & (HALF - 1);
      float sgn[G - 1];
#pragma unroll
      for (int i = 0; i < G - 1; ++i) sgn[i] = ((q >> i) & 1) ? 1.0f : -1.0f;
      const int tcount = nch * NB * SUB * HALF;
#pragma unroll 4
      for (int e = tid; e < tcount; e += NT) {
        const int j = (e / HALF) & (SUB - 1);
        const int cb = e / (HALF * SUB);  // chunk * NB + batch row
        const float *v = &s_v[cb * kChunkCols + j * G];
        float t = v[G - 1];
#pragma unroll
        for (int i = 0; i < G - 1; ++i) t = fmaf(sgn[i], v[i], t);
        float *tb = &s_tab[(cb * SUB + j) * TAB];
        tb[q | HALF] = t;
        tb[(HALF - 1) ^ q] = -t;
      }
    }
    __syncthreads();

    // Lookups, chunk by chunk, with PF chunks of weights in flight: once a
    // chunk's 16 bytes are consumed the chunk PF ahead is requested in its place.
    float part[NB], acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) part[b] = acc[b] = 0.0f;
    int cur = s0;              // segment being accumulated
    int ls = s0, lcis = cis0;  // chunk being looked up
    // After each chunk, if the next one starts another segment, the finished
    // segment is folded in with its row scale.  Branch-free (selects), so a
    // chunk's table reads and the adds that consume them share one block.
    auto consume = [&](int ch, const u32x4 w) {
      const uint32_t base = tab_base + (uint32_t)(ch * CTB);
#pragma unroll
      for (int q = 0; q < WPL; ++q) {
        lookup_word<G, NB>(w[q], base, acc, q * (32 / G));
        // wider batches: one word's table reads at a time
        if constexpr (NB >= 4) asm volatile("" ::: "memory");
      }
      next_chunk(L, ls, lcis);
      const bool fold = ls != cur;  // uniform
      const float rc = pick6(cur - s0, rv0, rv1, rv2, rv3, rv4, rv5);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        part[b] = fold ? fmaf(rc, acc[b], part[b]) : part[b];
        acc[b] = fold ? 0.0f : acc[b];
      }
      cur = ls;
      // the next chunk's table reads stay behind this chunk's (registers)
      asm volatile("" ::: "memory");
    };
    int ch0 = 0;
    for (; ch0 + PF < nch; ch0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        // consumed before the refill is issued into the same registers: with
        // both alive the compiler would rotate registers with copies that wait
        consume(ch0 + u, wb[u]);
        wb[u] = load_next();
        __builtin_amdgcn_sched_barrier(0);  // issue the refill here, not later
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (ch0 + u < nch) consume(ch0 + u, wb[u]);
    if (cur <= s_last) {  // the range ended inside a segment: fold its remainder
      const float rc = pick6(cur - s0, rv0, rv1, rv2, rv3, rv4, rv5);
#pragma unroll
      for (int b = 0; b < NB; ++b) part[b] = fmaf(rc, acc[b], part[b]);
    }

    // Output
    if (a.splits == 1) {
      if (row_ok) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (b < a.batch) a.y[(int64_t)b * L.n + row] = f2h(part[b]);
      }
      return;
    }
    // splits > 1: every workgroup adds its partial sum of each row into that
    // row's packed word with one agent-scope atomic (performed at the memory
    // side, coherent across XCDs).  The atomic returns the previous word, so the
    // lane that brings the last of `splits` contributions knows it is last and
    // holds the complete sum: it writes y and clears the word for the next call.
    // No workgroup waits for another, and since integer addition is exact the
    // result does not depend on the order in which the splits arrive.
    //
    // The fixed-point step quantises each partial to 2^-31 (absolute) and
    // saturates partials beyond +-2^17, twice the largest fp16 output.
    if (row_ok) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < a.batch) {
          const float scaled = fminf(fmaxf(part[b] * kFixScale, -kFixClamp), kFixClamp);
          const uint64_t contrib = (uint64_t)(__float2ll_rn(scaled) + kFixBias);
          uint64_t *slot = a.acc + (int64_t)b * a.n_pad + row;
          const uint64_t old =
              __hip_atomic_fetch_add(slot, contrib + kOneArrival, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int)(old >> kCountShift) == a.splits - 1) {
            const int64_t total = (int64_t)((old & kValueMask) + contrib) - (int64_t)a.splits * kFixBias;
            a.y[(int64_t)b * L.n + row] = f2h(__ll2float_rn(total) * kFixInv);
            __hip_atomic_store(slot, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    if constexpr (SAL) {
      asm volatile("; lut_gemv end: salient" ::: "memory");
    } else {
      asm volatile("; lut_gemv end: global" ::: "memory");
    }
  };
  if (s_last < L.kb) {
    body(BoolTag<false>{});
  } else {
    body(BoolTag<true>{});
  }
}

// --------------------------------------------------------------------------
// Half tables to global memory (the exported table builder)
// --------------------------------------------------------------------------
struct LutArgs {
  LayerArgs L;
  int32_t g;
  int32_t batch;
  int64_t sub_g, sub_s;     // sub-vectors per global / salient segment: ceil(len/g)
  int64_t subs_per_batch;   // kb * sub_g + ks * sub_s
  const uint16_t *x;
  float *lut;               // [batch][subs_per_batch][2^(g-1)]
};

template <int G>
__global__ __launch_bounds__(256) void build_lut_kernel(const LutArgs a) {
  constexpr int HALF = 1 << (G - 1);
  const ULayer L = uniform_layer(a.L);
  const int64_t total = (int64_t)a.batch * a.subs_per_batch * HALF;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int q = (int)(e % HALF);
    const int64_t sub = (e / HALF) % a.subs_per_batch;
    const int b = (int)(e / (HALF * a.subs_per_batch));
    const int64_t gsubs = L.kb * a.sub_g;
    const int sidx = sub < gsubs ? (int)(sub / a.sub_g) : L.kb + (int)((sub - gsubs) / a.sub_s);
    const int64_t j = sub < gsubs ? sub - (int64_t)sidx * a.sub_g : sub - gsubs - (int64_t)(sidx - L.kb) * a.sub_s;
    const SegRef sg = segment(L, sidx);
    float v[G];
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int64_t cc = j * G + t;
      float val = 0.0f;
      if (cc < sg.len) {
        const int64_t xi = sg.salient ? (int64_t)L.sal_idx[cc] : cc;
        val = h2f(sg.c[cc]) * h2f(a.x[(int64_t)b * L.k + xi]);
      }
      v[t] = val;
    }
    float t = v[G - 1];
#pragma unroll
    for (int i = 0; i < G - 1; ++i) t = ((q >> i) & 1) ? t + v[i] : t - v[i];
    a.lut[e] = t;
  }
}

// --------------------------------------------------------------------------
// Packing, relayout and VCM gather (offline helpers, bit-exact)
// --------------------------------------------------------------------------

// One thread per output word.  layout 0 = row-major canonical, 1 = tiled.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t *signs, int64_t rows, int64_t cols, int64_t ld,
                                                   int32_t layout, uint32_t *packed, uint32_t *invalid,
                                                   int64_t total_words) {
  const int64_t wpr = (cols + 31) / 32;
  const int64_t nc = (cols + 127) / 128;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total_words;
       o += (int64_t)gridDim.x * blockDim.x) {
    int64_t r, w;
    if (layout == 0) {
      r = o / wpr;
      w = o - r * wpr;
    } else {
      const int64_t q = o & 3, lane = (o >> 2) & 63, tc = o >> 8;  // tc = tile * nc + chunk
      r = (tc / nc) * 64 + lane;
      w = (tc % nc) * 4 + q;
    }
    uint32_t word = 0, bad = 0;
    if (r < rows && w < wpr) {
      const int8_t *p = signs + r * ld + w * 32;
      const int lim = (int)min((int64_t)32, cols - w * 32);
      for (int t = 0; t < lim; ++t) {
        const int8_t s = p[t];
        word |= (s == 1 ? 1u : 0u) << t;
        bad += (s != 1 && s != -1) ? 1u : 0u;
      }
    }
    packed[o] = word;
    if (bad && invalid) atomicAdd(invalid, bad);
  }
}

// One thread per destination word.
__global__ __launch_bounds__(256) void relayout_kernel(const uint32_t *src, int64_t rows, int64_t cols,
                                                       int32_t src_layout, int32_t dst_layout, uint32_t *dst,
                                                       int64_t total_words) {
  const int64_t wpr = (cols + 31) / 32;
  const int64_t nc = (cols + 127) / 128;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total_words;
       o += (int64_t)gridDim.x * blockDim.x) {
    int64_t r, w;
    if (dst_layout == 0) {
      r = o / wpr;
      w = o - r * wpr;
    } else {
      const int64_t q = o & 3, lane = (o >> 2) & 63, tc = o >> 8;
      r = (tc / nc) * 64 + lane;
      w = (tc % nc) * 4 + q;
    }
    uint32_t word = 0;
    if (r < rows && w < wpr) {
      const int64_t si = src_layout == 0 ? r * wpr + w : (((r / 64) * nc + w / 4) * 64 + (r % 64)) * 4 + (w % 4);
      word = src[si];
    }
    dst[o] = word;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void vcm_gather_values_kernel(const int32_t *idx, int64_t s, const T *src,
                                                                int64_t rows, int64_t cols, T *dst, T fill) {
  const int64_t total = rows * s;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = o / s, c = o - r * s;
    const int32_t j = idx[c];
    dst[o] = (j >= 0 && j < cols) ? src[r * cols + j] : fill;
  }
}

__global__ __launch_bounds__(256) void vcm_gather_bits_kernel(const int32_t *idx, int64_t s, const uint32_t *src,
                                                              int64_t rows, int64_t cols, uint32_t *dst) {
  const int64_t wk = (cols + 31) / 32, ws = (s + 31) / 32;
  const int64_t total = rows * ws;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = o / ws, w = o - r * ws;
    uint32_t word = 0;
    for (int t = 0; t < 32; ++t) {
      const int64_t c = w * 32 + t;
      if (c >= s) break;
      const int32_t j = idx[c];
      if (j >= 0 && j < cols) word |= ((src[r * wk + (j >> 5)] >> (j & 31)) & 1u) << t;
    }
    dst[o] = word;
  }
}

// --------------------------------------------------------------------------
// Dense fp16 GEMV (context kernel): one wave per row, 16-byte loads
// --------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void dense_f16_gemv_kernel(const uint16_t *w, int64_t n, int64_t k,
                                                             const uint16_t *x, uint16_t *y, int batch) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
  const u32x4 *wr = reinterpret_cast<const u32x4 *>(w + row * k);
  const int64_t k8 = k / 8;
  for (int64_t i = lane; i < k8; i += 64) {
    const u32x4 wv = __builtin_nontemporal_load(wr + i);
    float wf[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wf[2 * q] = h2f((uint16_t)(wv[q] & 0xffffu));
      wf[2 * q + 1] = h2f((uint16_t)(wv[q] >> 16));
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < batch) {
        const u32x4 xv = *reinterpret_cast<const u32x4 *>(x + (int64_t)b * k + i * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[b] = fmaf(wf[2 * q], h2f((uint16_t)(xv[q] & 0xffffu)), acc[b]);
          acc[b] = fmaf(wf[2 * q + 1], h2f((uint16_t)(xv[q] >> 16)), acc[b]);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float v = acc[b];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && b < batch) y[(int64_t)b * n + row] = f2h(v);
  }
}

}  // namespace fluxbin
