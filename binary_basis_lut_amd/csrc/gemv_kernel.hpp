// gemv_kernel.hpp -- the LUT GEMV kernel template (gfx950 / CDNA4).  Included
// by the translation units that instantiate it (one per table width, row-scale
// format and table entry type), so that the instances compile in parallel.
#pragma once

#include "common.hpp"

namespace fluxbin {

// RS selects the row-scale format: 0 = one scale per row per basis, applied
// to the range's accumulated sum; 1 = block-wise, one scale per row per basis
// per 128-column group (FluxBin summary, appendix C.2), streamed with the
// weights from the tiled scale layout.  In the block-wise format a global
// chunk is one group, scaled once its lookups are summed; a salient chunk
// holds 16 groups of 8 or 8 groups of 16 compact columns, and each sum of 8
// columns (one byte of a sign word) is scaled as it is formed.
//
// TQ selects the table entries: 0 = fp32; 1 = fp16 (quantised tables, LUT
// Tensor Core notes, section 3.1.3): each entry is summed in fp32 as before
// and rounded to fp16 once, halving the tables' LDS; lookups add the fp16
// entry into the fp32 accumulator with one v_fma_mix_f32.
//
// Block-wise single-row g = 4 instances are held to 6 waves per SIMD (at most
// 80 VGPRs): left alone the compiler keeps the salient lookup loop's 32-byte
// scale slots and expanded scales live at once, which would cap every
// workgroup of the call, global or salient, at 4-5 waves.  So are the per-row
// g = 4 instances of 4 batch rows.
template <int G, int NB, int WAVES, int PF, int RS, int TQ>
constexpr int lut_waves_per_eu() {
  if (G != 4) return 1;
  if (RS == 1) return NB == 1 ? 6 : 1;
  return NB == 4 ? 6 : 1;
}

// One workgroup = WAVES waves = 64 * WAVES output rows (lane = row) x one
// column range: up to cpb consecutive 128-column chunks of one segment.
//
//  1. inputs: the range's row scales (per-row format), column scales and
//     activations are requested first (salient ranges: the gather indices
//     first, the activations they select after the weights), then the first
//     PF chunks of sign words; vector loads return in issue order, so waiting
//     for the inputs never waits for HBM and the weights stay in flight;
//  2. v = c * x (exact in fp32) to LDS; barrier;
//  3. tables: each build unit sums 8 (g = 4) or 16 (g = 8) entries of one
//     sub-vector as a tree that shares the common leading terms; barrier;
//  4. lookups chunk by chunk, PF chunks in flight, each consumed slot refilled
//     with the chunk PF ahead (past the range's end the last chunk is read
//     again, which keeps the compiler's load counters exact);
//  5. row scale, then a direct fp16 store (one range per row) or the packed
//     fixed-point atomic (several ranges).
//
// KS = 2 or 4 (one batch row): the WAVES waves cover WAVES / KS row tiles, KS
// waves per tile, each over one KS-th of the range's chunks; the other waves'
// row-scaled partials reach the first through LDS, which adds them in wave
// order and makes the row's one atomic: 1 / KS of the split atomics for the
// same waves.
template <int G, int NB, int WAVES, int PF, int RS, int TQ, int KS>
__device__ __forceinline__ void lut_gemv_body(const GemvArgs &a) {
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && NB == 1), "several waves per row tile with one batch row only");
  constexpr int NT = WAVES * 64;
  constexpr int TW = WAVES / KS;           // row tiles of the workgroup
  constexpr int SUB = kChunkCols / G;      // sub-vectors per chunk
  constexpr int TAB = 1 << G;              // full table entries
  constexpr int WPL = kChunkCols / 32;     // words per lane per chunk (4)
  constexpr int EB = TQ ? 2 : 4;           // bytes per table entry
  constexpr int CTB = NB * SUB * TAB * EB; // table bytes of one chunk (all batch rows)
  constexpr int VPT = stage_items(NB, WAVES);
  constexpr bool TWO = NB == 1;            // two add chains in the lookups of a single batch row
  // fp16 tables of several batch rows at g = 4 (per-row scales): batch-row
  // pairs share each table dword (pair_table_dword), one LDS read per pair
  constexpr bool PAIRS = G == 4 && TQ == 1 && NB % 2 == 0 && RS == 0;
  static_assert(CTB % 256 == 0 && (G == 4 || CTB % 1024 == 0), "chunk table blocks must stay aligned");
  static_assert(PF >= 1 && PF <= 8, "prefetch depth");
  static_assert(kChunkCols % 64 == 0 && NT % 64 == 0, "a wave's staged items must share chunk and batch row");
  extern __shared__ __align__(1024) float smem[];

  const int tbc = a.tb;  // chunks whose tables the LDS holds at once
  float *s_tab = smem;
  const uint32_t tab_base = lds_addr(s_tab);  // 1024-aligned (table addresses are merged bytewise)
  float *s_v = smem + tbc * (CTB / 4);
  float *s_sink = s_v + tbc * NB * kChunkCols;
  float *s_red = s_sink + 64;  // KS > 1: the other waves' partials, (KS - 1) * TW * 64 floats

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address arithmetic
  const int rb = blockIdx.x;  // row block
  const int sp = blockIdx.y;  // column range
  const int wt = KS == 1 ? wave : wave % TW;  // the wave's row tile within the workgroup (uniform)
  const int kh = KS == 1 ? 0 : wave / TW;     // and which part of the range it looks up (uniform)
  const int tile = rb * TW + wt;
  const int ltile = min(tile, a.row_tiles - 1);  // waves past the last tile read the last one, store nothing
  const int row = tile * kTileRows + lane;
  const bool row_ok = tile < a.row_tiles && row < a.n;
  const int rrow = row_ok ? row : 0;

  // The column range: segment sg, chunks [c_lo, c_lo + nch) of it; this
  // wave's part of it: chunks [k0, k0 + nk) of the range (all of it when KS = 1)
  const ColRange cr = column_range(a, sp);
  const SegRef S = cr.S;
  const int sg = cr.sg, c_lo = cr.c_lo, nch = cr.nch;
  const int k0 = KS == 1 ? 0 : kh * nch / KS, nk = KS == 1 ? nch : (kh + 1) * nch / KS - k0;
  // element of this lane's 16 bytes in the part's first chunk; chunk u is 64 elements further
  const int64_t te0 = ((int64_t)ltile * S.nchunks + c_lo + k0) * kTileRows + lane;
  const FB_GLOBAL u32x4 *wp = S.bits + te0;

  auto body = [&](auto sal_tag) {
    constexpr bool SAL = decltype(sal_tag)::value;
    const FB_GLOBAL int32_t *uidx = uni(a.idx_or_dummy);
    const FB_GLOBAL uint16_t *ux = uni(a.x);
    uint16_t rr16 = 0;
    if constexpr (RS == 0) rr16 = S.r[rrow];

    // Weight slots: D chunks in flight, each 16 bytes of sign words per lane
    // and, in the block-wise format, the lane's row scales for that chunk
    // (global: one fp16; salient: 16 or 8 fp16 in 32 bytes, the second 16
    // bytes re-read from the first when there are 8).  Block-wise salient
    // workgroups keep at most 4 slots: their 32-byte slots would otherwise
    // set the register count, and so the occupancy, of every workgroup.
    constexpr int D = (RS == 1 && SAL && PF > 4) ? 4 : PF;
    u32x4 wb[D];
    uint32_t rg[D];
    u32x4 rsa[D], rsb[D];
    const int sal_hi = a.sal16 ? 1 : 0;  // uniform
    int pidx = 0;                        // next chunk of the range to load
    auto load_into = [&](int u) {
      // past the part's end its last chunk is read again (a part without
      // chunks, KS > 1 over a range shorter than KS chunks, reads the range's first)
      const int ci = KS == 1 ? min(pidx, nch - 1) : min(pidx, max(nk, 1) - 1);
      wb[u] = __builtin_nontemporal_load(wp + ci * kTileRows);
      if constexpr (RS == 1 && !SAL) rg[u] = __builtin_nontemporal_load(S.r + te0 + ci * kTileRows);
      if constexpr (RS == 1 && SAL) {
        const FB_GLOBAL u32x4 *rp =
            reinterpret_cast<const FB_GLOBAL u32x4 *>(S.r) + (te0 + ci * kTileRows) * (1 + sal_hi);
        rsa[u] = __builtin_nontemporal_load(rp);
        rsb[u] = __builtin_nontemporal_load(rp + sal_hi);
      }
      ++pidx;
    };
    auto issue_weights = [&]() {
#pragma unroll
      for (int u = 0; u < D; ++u) load_into(u);
    };

    // Table groups: the tables of chunks [g0, g0 + gn) of the range are in LDS
    // at a time.  One batch row: the whole range (the host sizes the LDS for
    // it).  Several batch rows, whose tables are NB times larger: groups of
    // a.tb chunks, a multiple of D, built in turn while the weight slots keep
    // streaming, so that a range need not fit the LDS (fewer, longer ranges).
    int g0 = 0;
    int gn = min(nch, tbc);
    // Staged items (chunk, batch row, column) of the group: item e is handled
    // by thread e % NT, VPT per thread per round (the first round's loads go
    // out before the weights, longer groups take further rounds after them);
    // a wave's 64 items share chunk and batch row.  Every item slot loads
    // (slots past the group re-read a live item's inputs and store them to the
    // sink).
    int items = gn * NB * kChunkCols;
    bool live[VPT];
    const FB_GLOBAL uint16_t *xrow[VPT];
    uint32_t ccl[VPT], gi[VPT];
    uint32_t cvl[VPT], xvl[VPT];  // 32-bit: the compiler would otherwise pack pairs, waiting early
    auto prep = [&](int base) {    // column scales of round `base`
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int e0 = base + i * NT + wave * 64;  // uniform
        const int eb = min(e0, items - 64);
        const int ch = eb / (NB * kChunkCols);
        const int b = (eb / kChunkCols) % NB;
        const bool brow = b < a.batch;  // uniform; batch rows past `batch` do not exist
        const uint32_t cc = (uint32_t)((c_lo + g0 + ch) * kChunkCols + (eb & (kChunkCols - 1)) + lane);
        live[i] = (e0 < items) & brow & (cc < (uint32_t)S.len);  // non-short-circuit: selects, not branches
        ccl[i] = live[i] ? cc : 0u;
        xrow[i] = ux + (int64_t)(brow ? b : 0) * a.k;
        cvl[i] = S.c[ccl[i]];
      }
    };
    auto load_x = [&]() {  // activations: global columns directly, salient ones through the gathered index
#pragma unroll
      for (int i = 0; i < VPT; ++i) xvl[i] = xrow[i][SAL ? gi[i] : ccl[i]];
    };
    auto load_idx = [&]() {
#pragma unroll
      for (int i = 0; i < VPT; ++i) gi[i] = (uint32_t)uidx[ccl[i]];
    };
    // Inputs to LDS.  No select or branch takes a loaded value as an operand
    // (the compiler would turn it into a branch around the load): unused slots
    // are zeroed by masking the fp16 bits and stored to the sink.
    auto stage = [&](int base) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t m = live[i] ? 0xffffu : 0u;
        float *dst = base + i * NT + wave * 64 < items ? s_v + base + i * NT + tid : s_sink + lane;
        *dst = h2f((uint16_t)(cvl[i] & m)) * h2f((uint16_t)(xvl[i] & m));
      }
    };
    // sched_barrier: the scheduler must not move work that waits for earlier
    // loads above the weight requests (that wait would hold them back).
    prep(0);
    if constexpr (!SAL) {
      load_x();
      __builtin_amdgcn_sched_barrier(0);
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
    } else {
      load_idx();
      __builtin_amdgcn_sched_barrier(0);
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
      load_x();
    }
    auto stage_rounds = [&]() {  // the group's further rounds (long groups only)
      for (int base = VPT * NT; base < items; base += VPT * NT) {  // uniform
        prep(base);
        if constexpr (SAL) load_idx();
        load_x();
        stage(base);
      }
    };
    stage(0);
    stage_rounds();
    __syncthreads();

    // Tables.  Entry p of a sub-vector is the sum, in this order, of
    // sgn_{G-1} v_{G-1}, sgn_0 v_0, sgn_1 v_1, ..., sgn_{G-2} v_{G-2}, with
    // sgn_t = +1 where bit t of p is set and -1 where it is clear.  A build
    // unit fixes the leading signs and branches on the rest as a tree, so its
    // entries round exactly like that sequence; the half with the top bit
    // clear is built from -v_{G-1} and is therefore the exact negation of
    // the other half (LUT[~p] = -LUT[p]).  The g = 8 unit is g8_unit_entries.
    // g = 4 build unit un of the sub-vector whose products start at v: unit
    // 1 gives entries 8..15, unit 0 entries 0..7
    auto g4_unit = [](const float *v, int un, float (&e)[8]) {
      const float4 vv = *reinterpret_cast<const float4 *>(v);
      const float top = un ? vv.w : -vv.w;
      const float l1[2] = {top - vv.x, top + vv.x};
      float l2[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) l2[i] = l1[i] - vv.y, l2[i + 2] = l1[i] + vv.y;
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = l2[i] - vv.z, e[i + 4] = l2[i] + vv.z;
    };
    auto build_tables = [&]() {
      constexpr int UPS = G == 4 ? 2 : 16;  // build units per sub-vector
      if constexpr (PAIRS) {
        // a unit builds one half of one sub-vector's entries for both rows of
        // a batch-row pair and stores them as 8 shared dwords
        const int units = gn * (NB / 2) * SUB * UPS;
        for (int t = tid; t < units; t += NT) {
          const int pu = t / UPS;  // (chunk * NB / 2 + pair) * SUB + sub-vector
          const int un = t - pu * UPS;
          const int j = pu % SUB;
          const int q = (pu / SUB) % (NB / 2);
          const int ch = pu / (SUB * (NB / 2));
          const int sv0 = (ch * NB + 2 * q) * SUB + j;
          float e0[8], e1[8];
          g4_unit(s_v + sv0 * G, un, e0);
          g4_unit(s_v + (sv0 + SUB) * G, un, e1);
          u32x4 h0, h1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h0[i] = (uint32_t)f2h(e0[i]) | ((uint32_t)f2h(e1[i]) << 16);
            h1[i] = (uint32_t)f2h(e0[i + 4]) | ((uint32_t)f2h(e1[i + 4]) << 16);
          }
          u32x4 *tb = reinterpret_cast<u32x4 *>(reinterpret_cast<uint32_t *>(s_tab) + ch * (CTB / 4) +
                                                pair_table_dword(q, j, un * 8));
          tb[0] = h0;
          tb[1] = h1;
        }
        return;
      }
      const int units = gn * NB * SUB * UPS;
      for (int t = tid; t < units; t += NT) {
        const int sv = t / UPS;  // (chunk * NB + batch row) * SUB + sub-vector
        const int un = t - sv * UPS;
        const float *v = s_v + sv * G;
        if constexpr (G == 4) {
          float e[8];
          g4_unit(v, un, e);
          if constexpr (TQ == 0) {
            float4 *tb = reinterpret_cast<float4 *>(s_tab + sv * TAB + un * 8);
            tb[0] = make_float4(e[0], e[1], e[2], e[3]);
            tb[1] = make_float4(e[4], e[5], e[6], e[7]);
          } else {
            u32x4 hp;
#pragma unroll
            for (int i = 0; i < 4; ++i) hp[i] = (uint32_t)f2h(e[2 * i]) | ((uint32_t)f2h(e[2 * i + 1]) << 16);
            *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(s_tab) + sv * TAB + un * 8) = hp;
          }
        } else {
          // unit = (top bit h, low three bits q3); its 16 entries vary bits 3..6
          float e[16];
          g8_unit_entries(v, un, e);
          const int h = un >> 3, q3 = un & 7;
          const int p0 = (h << 7) | q3;
          if constexpr (TQ == 0) {
            float *tb = s_tab + sv * TAB + p0;
#pragma unroll
            for (int m = 0; m < 16; ++m) tb[m * 8] = e[m];
          } else {
            uint16_t *tb = reinterpret_cast<uint16_t *>(s_tab) + sv * TAB + p0;
#pragma unroll
            for (int m = 0; m < 16; ++m) tb[m * 8] = f2h(e[m]);
          }
        }
      }
    };
    build_tables();
    __syncthreads();

    // Lookups, chunk by chunk, with D chunks of weights in flight: once a
    // chunk's slot is consumed the chunk D ahead is requested in its place.
    float acc0[NB], acc1[NB], part[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = part[b] = 0.0f;
    float(&accb)[NB] = TWO ? acc1 : acc0;
    auto consume = [&](const u32x4 w, int ch, int u) {
      const uint32_t base = tab_base + (uint32_t)(ch * CTB);
      if constexpr (RS == 1 && SAL) {
        // Block-wise salient chunk: the scale of each 8 columns.  E[j] holds
        // those of columns 16j..16j+7 (low half) and 16j+8..16j+15 (high
        // half): with 16 groups per chunk the loaded halves as they are, with
        // 8 groups half j of the first 16 bytes in both (v_perm duplicates
        // it).  The choice is a uniform bit mask, not a select of loaded values.
        const uint32_t M = 0u - (uint32_t)sal_hi;
        float sc[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t r16 = j < 4 ? rsa[u][j] : rsb[u][j - 4];
          const uint32_t s8 = rsa[u][j >> 1];
          const uint32_t d8 = __builtin_amdgcn_perm(s8, s8, (j & 1) ? 0x03020302u : 0x01000100u);
          const uint32_t e = (r16 & M) | (d8 & ~M);
          sc[2 * j] = h2f((uint16_t)(e & 0xffffu));
          sc[2 * j + 1] = h2f((uint16_t)(e >> 16));
        }
#pragma unroll
        for (int q = 0; q < WPL; ++q) {
          lookup_word_scaled<G, NB, EB>(w[q], base, part, q * (32 / G), sc[4 * q], sc[4 * q + 1], sc[4 * q + 2],
                                        sc[4 * q + 3]);
          if constexpr (NB >= 4) asm volatile("" ::: "memory");
        }
      } else {
#pragma unroll
        for (int q = 0; q < WPL; ++q) {
          lookup_word<G, NB, EB, PAIRS>(w[q], base, acc0, accb, q * (32 / G));
          // wider batches: one word's table reads at a time
          if constexpr (NB >= 4) asm volatile("" ::: "memory");
        }
        if constexpr (RS == 1) {
          // block-wise global chunk: one group, scaled once summed
          const float rc = h2f((uint16_t)rg[u]);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            part[b] = fmaf(rc, TWO ? acc0[b] + acc1[b] : acc0[b], part[b]);
            acc0[b] = acc1[b] = 0.0f;
          }
        }
      }
      // the next chunk's table reads stay behind this chunk's (registers)
      asm volatile("" ::: "memory");
    };
    if constexpr (NB == 1) {
      // one group: every chunk's tables are in LDS; this wave's part is
      // chunks [k0, k0 + nk) of the range
      int ch0 = 0;
      for (; ch0 + D < nk; ch0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
          // consumed before the refill is issued into the same registers: with
          // both alive the compiler would rotate registers with copies that wait
          consume(wb[u], k0 + ch0 + u, u);
          load_into(u);
          __builtin_amdgcn_sched_barrier(0);  // issue the refill here, not later
        }
      }
#pragma unroll
      for (int u = 0; u < D; ++u)
        if (ch0 + u < nk) consume(wb[u], k0 + ch0 + u, u);
    } else {
      for (;;) {  // uniform
        // group [g0, g0 + gn): g0 and, but for the last group, gn are multiples
        // of D, so chunk ch0 + u is in slot u; the loop is the one-group loop
        // above with the group's end as a second bound
        const int gend = g0 + gn;
        int ch0 = g0;
        for (; ch0 + D <= gend && ch0 + D < nch; ch0 += D) {
#pragma unroll
          for (int u = 0; u < D; ++u) {
            consume(wb[u], ch0 + u - g0, u);
            load_into(u);  // the chunk D ahead, across groups
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (gend >= nch) {
#pragma unroll
          for (int u = 0; u < D; ++u)
            if (ch0 + u < nch) consume(wb[u], ch0 + u - g0, u);
          break;
        }
        g0 = gend;
        gn = min(tbc, nch - g0);
        items = gn * NB * kChunkCols;
        __syncthreads();  // every wave is done with the group's tables
        prep(0);
        if constexpr (SAL) load_idx();
        load_x();
        stage(0);
        stage_rounds();
        __syncthreads();
        build_tables();
        __syncthreads();
      }
    }
    if constexpr (RS == 0) {
      // the row scale, once, after the range's accumulation
      const float rv = h2f(rr16);
#pragma unroll
      for (int b = 0; b < NB; ++b) part[b] = rv * (TWO ? acc0[b] + acc1[b] : acc0[b]);
    }

    if constexpr (KS > 1) {
      // the other waves of the tile hand their row-scaled partials to the first
      if (kh > 0) s_red[((kh - 1) * TW + wt) * 64 + lane] = part[0];
      __syncthreads();
      if (kh > 0) return;
#pragma unroll
      for (int h = 1; h < KS; ++h) part[0] += s_red[((h - 1) * TW + wt) * 64 + lane];
    }
    finish_rows<NB>(a, row, row_ok, part);
  };
  if (sg < a.kb) {
    body(BoolTag<false>{});
  } else {
    body(BoolTag<true>{});
  }
}

template <int G, int NB, int WAVES, int PF, int RS, int TQ>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(lut_waves_per_eu<G, NB, WAVES, PF, RS, TQ>())))
void lut_gemv_kernel(const GemvArgs a) {
  lut_gemv_body<G, NB, WAVES, PF, RS, TQ, 1>(a);
}

// Two waves per row tile (one batch row): WAVES / 2 row tiles.
template <int G, int WAVES, int PF, int RS, int TQ>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(lut_waves_per_eu<G, 1, WAVES, PF, RS, TQ>())))
void lut_gemv_ks2_kernel(const GemvArgs a) {
  lut_gemv_body<G, 1, WAVES, PF, RS, TQ, 2>(a);
}

// Four waves per row tile (one batch row): WAVES / 4 row tiles.
template <int G, int WAVES, int PF, int RS, int TQ>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(lut_waves_per_eu<G, 1, WAVES, PF, RS, TQ>())))
void lut_gemv_ks4_kernel(const GemvArgs a) {
  lut_gemv_body<G, 1, WAVES, PF, RS, TQ, 4>(a);
}

// Instance for (batch width, waves, prefetch depth) at table width G,
// row-scale format RS and table entry type TQ, or nullptr.
template <int G, int NB, int W, int RS, int TQ>
gemv_fn gemv_pick_pf(int pf) {
  if constexpr (G == 4 && NB == 1 && RS == 0) {
    if (pf == 3) return lut_gemv_kernel<G, NB, W, 3, RS, TQ>;
  }
  return pf == 8 ? lut_gemv_kernel<G, NB, W, 8, RS, TQ>
         : pf == 4 ? lut_gemv_kernel<G, NB, W, 4, RS, TQ>
         : pf == 2 ? lut_gemv_kernel<G, NB, W, 2, RS, TQ>
                   : nullptr;
}

template <int G, int NB, int RS, int TQ>
gemv_fn gemv_pick_waves(int waves, int pf) {
  return waves == 8 ? gemv_pick_pf<G, NB, 8, RS, TQ>(pf) : waves == 4 ? gemv_pick_pf<G, NB, 4, RS, TQ>(pf) : nullptr;
}

template <int G, int RS, int TQ>
gemv_fn gemv_pick(int nb, int waves, int pf) {
  switch (nb) {
    case 1: return gemv_pick_waves<G, 1, RS, TQ>(waves, pf);
    case 2: return gemv_pick_waves<G, 2, RS, TQ>(waves, pf);
    case 4: return gemv_pick_waves<G, 4, RS, TQ>(waves, pf);
  }
  if constexpr (G == 4) {
    if (nb == 8) return gemv_pick_waves<G, 8, RS, TQ>(waves, pf);
  }
  return nullptr;
}

}  // namespace fluxbin
