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

// One segment as seen by the kernels.
struct SegRef {
  const u32x4 *bits;    // element ((tile * nchunks + chunk) * 64 + lane)
  const uint16_t *c;
  const uint16_t *r;
  int64_t len;
  int32_t nchunks;
  int32_t salient;
};

__device__ __forceinline__ SegRef segment(const LayerArgs &L, int sidx) {
  SegRef r;
  if (sidx < L.kb) {
    r.bits = L.bits_g + sidx * L.tv_g;
    r.c = L.c_g + sidx * L.k;
    r.r = L.r_g + sidx * L.n;
    r.len = L.k;
    r.nchunks = L.nc_g;
    r.salient = 0;
  } else {
    const int b = sidx - L.kb;
    r.bits = L.bits_s + b * L.tv_s;
    r.c = L.c_s + b * L.s;
    r.r = L.r_s + b * L.n;
    r.len = L.s;
    r.nchunks = L.nc_s;
    r.salient = 1;
  }
  return r;
}

// Segment of chunk gc of the concatenated chunk space, and the chunk's index inside it.
__device__ __forceinline__ int seg_of(const LayerArgs &L, int gc, int *cis) {
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
  LayerArgs L;
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

// Byte `kk` of v, zero-extended (v_perm_b32: opaque to the optimiser, one VALU op).
template <int kk>
__device__ __forceinline__ uint32_t byte_of(uint32_t v) {
  return __builtin_amdgcn_perm(0u, v, 0x0c0c0c00u | kk);
}

template <int G, int NB>
__device__ __forceinline__ void lookup_word(uint32_t w, const char *tb, float (&acc)[NB], int j0) {
  constexpr int SUB = kChunkCols / G;
  constexpr int TAB = 1 << G;
  if constexpr (G == 4) {
    // nibble m of w at bits [4m, 4m+4); A holds nibbles 0,2,4,6 and B nibbles
    // 1,3,5,7 as byte offsets (index * 4) of a 16-entry fp32 table.
    const uint32_t A = (w << 2) & 0x3c3c3c3cu;
    const uint32_t B = (w >> 2) & 0x3c3c3c3cu;
    const uint32_t ia[4] = {byte_of<0>(A), byte_of<1>(A), byte_of<2>(A), byte_of<3>(A)};
    const uint32_t ib[4] = {byte_of<0>(B), byte_of<1>(B), byte_of<2>(B), byte_of<3>(B)};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const char *t0 = tb + ((b * SUB + j0 + 2 * kk) * TAB) * 4;
        acc[b] += *reinterpret_cast<const float *>(t0 + ia[kk]);
        acc[b] += *reinterpret_cast<const float *>(t0 + TAB * 4 + ib[kk]);
      }
    }
  } else {
    // byte kk of w is the 8-bit pattern of sub-vector j0 + kk
    const uint32_t W = w;
    uint32_t ix[4];
    ix[0] = (W << 2) & 0x3fcu;
    ix[1] = (W >> 6) & 0x3fcu;
    ix[2] = (W >> 14) & 0x3fcu;
    ix[3] = (W >> 22) & 0x3fcu;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const char *t0 = tb + ((b * SUB + j0 + kk) * TAB) * 4;
        acc[b] += *reinterpret_cast<const float *>(t0 + ix[kk]);
      }
    }
  }
}

template <int G, int NB, int CPB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void lut_gemv_kernel(const GemvArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int SUB = kChunkCols / G;  // sub-vectors per chunk
  constexpr int TAB = 1 << G;          // full table entries
  constexpr int HALF = TAB / 2;
  constexpr int WPL = kChunkCols / 32;  // words per lane per chunk (4)
  __shared__ float s_tab[CPB * NB * SUB * TAB];  // [chunk][batch][sub-vector][pattern]
  __shared__ float s_v[CPB * NB * kChunkCols];   // [chunk][batch][column] scale-fused inputs

  const LayerArgs &L = a.L;
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
  const int c0 = sp * CPB;
  const int nch = min(CPB, a.total_chunks - c0);

  // Segment and chunk-in-segment of each of the workgroup's chunks (uniform).
  // Chunks past the range repeat the last one: a redundant load, never used.
  int cseg[CPB], ccis[CPB];
  {
    int cis;
    int sg = seg_of(L, c0, &cis);
#pragma unroll
    for (int ch = 0; ch < CPB; ++ch) {
      cseg[ch] = sg;
      ccis[ch] = cis;
      if (ch + 1 < nch) {
        ++cis;
        if (cis == (sg < L.kb ? L.nc_g : L.nc_s)) {
          cis = 0;
          ++sg;
        }
      }
    }
  }
  const int s_first = cseg[0];
  const int s_lastseg = cseg[CPB - 1];
  const bool any_salient = s_lastseg >= L.kb;  // segments run global first, then salient

  // 1. Loads.  Inputs of the table build go first so that waiting for them
  //    (loads retire in order) does not wait for the weight stream.  Every
  //    load is unconditional from a valid address and dead items are zeroed
  //    by a select, so all loads of a phase are in flight together.
  constexpr int VPC = (NB * kChunkCols + NT - 1) / NT;  // v items per thread per chunk
  bool vlive[CPB][VPC];
  uint16_t vc[CPB][VPC];   // fp16 column scale
  uint16_t vxv[CPB][VPC];  // fp16 activation
  u32x4 w[CPB];            // this lane's 16 bytes of every chunk
  int64_t xrow[CPB][VPC];  // b * k
  int32_t xcol[CPB][VPC];  // column of x (gathered through sal_idx on salient segments)
#pragma unroll
  for (int ch = 0; ch < CPB; ++ch) {
    const SegRef sg = segment(L, cseg[ch]);
#pragma unroll
    for (int i = 0; i < VPC; ++i) {
      const int e = tid + i * NT;
      const int b = e / kChunkCols;
      const int cc = ccis[ch] * kChunkCols + (e & (kChunkCols - 1));
      // non-short-circuit: a select, not a branch
      const bool live = (ch < nch) & (e < NB * kChunkCols) & (b < a.batch) & (cc < sg.len);
      vlive[ch][i] = live;
      xrow[ch][i] = live ? (int64_t)b * L.k : 0;
      xcol[ch][i] = live ? cc : 0;
      vc[ch][i] = sg.c[xcol[ch][i]];
    }
  }
  auto stream_weights = [&]() {
#pragma unroll
    for (int ch = 0; ch < CPB; ++ch) {
      const SegRef sg = segment(L, cseg[ch]);
      const u32x4 *base = sg.bits + ((int64_t)ltile * sg.nchunks + ccis[ch]) * kTileRows;
      w[ch] = __builtin_nontemporal_load(base + lane);
    }
  };
  if (!any_salient) {
    // global chunks only: activations, then the weight stream
#pragma unroll
    for (int ch = 0; ch < CPB; ++ch)
#pragma unroll
      for (int i = 0; i < VPC; ++i) vxv[ch][i] = a.x[xrow[ch][i] + xcol[ch][i]];
    stream_weights();
  } else {
    // some chunk is salient: gather indices first (VCM), then activations, then weights
#pragma unroll
    for (int ch = 0; ch < CPB; ++ch) {
      const bool sal = cseg[ch] >= L.kb;
#pragma unroll
      for (int i = 0; i < VPC; ++i) {
        const int32_t gi = L.sal_idx[sal ? xcol[ch][i] : 0];
        xcol[ch][i] = sal ? gi : xcol[ch][i];
      }
    }
#pragma unroll
    for (int ch = 0; ch < CPB; ++ch)
#pragma unroll
      for (int i = 0; i < VPC; ++i) vxv[ch][i] = a.x[xrow[ch][i] + xcol[ch][i]];
    stream_weights();
  }
  // row scales of the segments this workgroup touches (s_first .. s_lastseg, consecutive)
  auto rptr = [&](int j) -> const uint16_t * { return segment(L, min(s_first + j, s_lastseg)).r + rrow; };
  const uint16_t rr0 = *rptr(0), rr1 = *rptr(1), rr2 = *rptr(2), rr3 = *rptr(3), rr4 = *rptr(4), rr5 = *rptr(5);

  // 2. scale-fused inputs v = c * x (exact in fp32: product of two fp16 values)
#pragma unroll
  for (int ch = 0; ch < CPB; ++ch)
#pragma unroll
    for (int i = 0; i < VPC; ++i) {
      const int e = tid + i * NT;
      if (e < NB * kChunkCols) s_v[ch * NB * kChunkCols + e] = vlive[ch][i] ? h2f(vc[ch][i]) * h2f(vxv[ch][i]) : 0.0f;
    }
  const float rv0 = h2f(rr0), rv1 = h2f(rr1), rv2 = h2f(rr2), rv3 = h2f(rr3), rv4 = h2f(rr4), rv5 = h2f(rr5);
  __syncthreads();

  // 3. tables: the half with the top input at +1 is summed, the rest negated.
  //    Entry q of a sub-vector is v_{G-1} + sum_{i<G-1} sgn_i(q) * v_i in that
  //    order; sgn_i = +-1 exactly, so each fma rounds like the add or subtract.
  //    NT is a multiple of HALF, so a thread's pattern q (and its signs) is the
  //    same in every iteration.
  static_assert(NT % HALF == 0, "thread count must be a multiple of the half-table size");
  constexpr int TITEMS = (CPB * NB * SUB * HALF + NT - 1) / NT;
  {
    const int q = tid & (HALF - 1);
    float sgn[G - 1];
#pragma unroll
    for (int i = 0; i < G - 1; ++i) sgn[i] = ((q >> i) & 1) ? 1.0f : -1.0f;
#pragma unroll
    for (int it = 0; it < TITEMS; ++it) {
      const int e = tid + it * NT;
      if (e < nch * NB * SUB * HALF) {
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
  }
  __syncthreads();

  // 4. lookups: sign patterns index the tables; fp32 accumulation per segment
  float part[NB], acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) part[b] = acc[b] = 0.0f;
  int cur = s_first;
#pragma unroll
  for (int ch = 0; ch < CPB; ++ch) {
    if (ch < nch) {
      const int s = cseg[ch];
      if (s != cur) {
        const float rc = pick6(cur - s_first, rv0, rv1, rv2, rv3, rv4, rv5);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          part[b] += rc * acc[b];
          acc[b] = 0.0f;
        }
        cur = s;
      }
      const char *tb = reinterpret_cast<const char *>(&s_tab[ch * NB * SUB * TAB]);
#pragma unroll
      for (int q = 0; q < WPL; ++q) lookup_word<G, NB>(w[ch][q], tb, acc, q * (32 / G));
    }
  }
  {
    const float rc = pick6(cur - s_first, rv0, rv1, rv2, rv3, rv4, rv5);
#pragma unroll
    for (int b = 0; b < NB; ++b) part[b] += rc * acc[b];
  }

  // 5. output
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
  const LayerArgs &L = a.L;
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
