// gemv_kernel.hpp -- the LUT GEMV kernel template (gfx950 / CDNA4).  Included
// by the translation units that instantiate it (one per table width and
// row-scale format), so that the instances compile in parallel.
#pragma once

#include "common.hpp"

namespace fluxbin {

// RS selects the row-scale format: 0 = one scale per row per basis, applied
// when a segment's accumulation ends; 1 = block-wise, one scale per row per
// basis per 128-column group (FluxBin summary, appendix C.2), streamed with
// the weights from the tiled scale layout.  In the block-wise format a global
// chunk is one group, scaled once its lookups are summed; a salient chunk
// holds 16 groups of 8 or 8 groups of 16 compact columns, each sum of 8
// columns (one byte of a sign word) is scaled as it is formed.
//
// TQ selects the table entries: 0 = fp32; 1 = fp16 (quantised tables, LUT
// Tensor Core notes, section 3.1.3): each entry is summed in fp32 as before
// and rounded to fp16 once, halving the tables' LDS; lookups add the fp16
// entry into the fp32 accumulator with one v_fma_mix_f32.
//
//
// Block-wise single-row g = 4 instances of prefetch depth 2 and 4 (the decode
// plans) are held to 6 waves per SIMD (at most 80 VGPRs): left alone the
// compiler keeps the salient lookup loop's 32-byte scale slots and expanded
// scales live at once, 83-111 VGPRs, which caps every workgroup of the call,
// global or salient, at 4-5 waves.  So are the per-row g = 4 instances of 4
// batch rows and depth 4 or 8 (115-121 VGPRs left alone).  These instances
// need no spills for it; the others would spill and are left alone.
template <int G, int NB, int WAVES, int PF, int RS, int TQ>
constexpr int lut_waves_per_eu() {
  if (G != 4) return 1;
  if (RS == 1) return NB == 1 && PF <= 4 ? 6 : 1;
  return NB == 4 && PF >= 4 ? 6 : 1;
}

template <int G, int NB, int WAVES, int PF, int RS, int TQ>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(lut_waves_per_eu<G, NB, WAVES, PF, RS, TQ>())))
void lut_gemv_kernel(const GemvArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int SUB = kChunkCols / G;      // sub-vectors per chunk
  constexpr int TAB = 1 << G;              // full table entries
  constexpr int HALF = TAB / 2;
  constexpr int WPL = kChunkCols / 32;     // words per lane per chunk (4)
  constexpr int EB = TQ ? 2 : 4;           // bytes per table entry
  constexpr int CTB = NB * SUB * TAB * EB; // table bytes of one chunk (all batch rows)
  static_assert(CTB % 256 == 0 && (G == 4 || CTB % 512 == 0), "chunk table blocks must stay aligned");
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
  int c0, nch;
  if constexpr (RS == 0) {
    c0 = sp * cpb;
    nch = min(cpb, a.total_chunks - c0);
  } else {
    const bool gpart = sp < a.gsplits;
    c0 = gpart ? sp * cpb : a.gchunks + (sp - a.gsplits) * cpb;
    nch = min(cpb, (gpart ? a.gchunks : a.total_chunks) - c0);
  }

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
    // per-row format: the row scales of the segments this workgroup touches
    // (s0 .. s_last, consecutive)
    uint16_t rr0 = 0, rr1 = 0, rr2 = 0, rr3 = 0, rr4 = 0, rr5 = 0;
    if constexpr (RS == 0) {
      auto rptr = [&](int j) { return gemv_segment(a.seg, L.kb, min(s0 + j, s_last)).r + rrow; };
      rr0 = *rptr(0), rr1 = *rptr(1), rr2 = *rptr(2), rr3 = *rptr(3), rr4 = *rptr(4), rr5 = *rptr(5);
    }

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
    int ps = s0, pcis = cis0, pidx = 0;  // next chunk to load and its index in the range
    auto load_into = [&](int u) {
      const SegRef S = gemv_segment(a.seg, L.kb, ps);
      const int64_t te = ((int64_t)ltile * S.nchunks + pcis) * kTileRows + lane;  // this lane's element
      wb[u] = __builtin_nontemporal_load(S.bits + te);
      if constexpr (RS == 1 && !SAL) rg[u] = __builtin_nontemporal_load(S.r + te);
      if constexpr (RS == 1 && SAL) {
        const FB_GLOBAL u32x4 *rp = reinterpret_cast<const FB_GLOBAL u32x4 *>(S.r) + te * (1 + sal_hi);
        rsa[u] = __builtin_nontemporal_load(rp);
        rsb[u] = __builtin_nontemporal_load(rp + sal_hi);
      }
      const int step = (int)((uint32_t)(pidx - nch + 1) >> 31);  // 1 while pidx < nch - 1: past
      next_chunk(L, ps, pcis, step);                               // the last chunk it is read again
      pidx += step;
    };
    auto issue_weights = [&]() {
#pragma unroll
      for (int u = 0; u < D; ++u) load_into(u);
    };

    // Table-build items (chunk, batch row, column) of the range: item e is
    // handled by thread e % NT; a wave's 64 items share chunk and batch row.
    // Every item slot loads (items past the range re-read the last chunk's
    // inputs and are dropped).
    constexpr int CMAX = cpb_for_depth(PF, cpb_cap(G, NB, WAVES, EB));  // chunks, at most
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
      if constexpr (RS == 0)
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
        if constexpr (TQ == 0) {
          float *tb = &s_tab[(cb * SUB + j) * TAB];
          tb[q | HALF] = t;
          tb[(HALF - 1) ^ q] = -t;
        } else {
          uint16_t *tb = reinterpret_cast<uint16_t *>(s_tab) + (cb * SUB + j) * TAB;
          const uint16_t h = f2h(t);  // nearest even; the negation is exact
          tb[q | HALF] = h;
          tb[(HALF - 1) ^ q] = h ^ 0x8000u;
        }
      }
    }
    __syncthreads();

    // Lookups, chunk by chunk, with D chunks of weights in flight: once a
    // chunk's slot is consumed the chunk D ahead is requested in its place.
    float part[NB], acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) part[b] = acc[b] = 0.0f;
    int cur = s0;              // segment being accumulated
    int ls = s0, lcis = cis0;  // chunk being looked up
    // After each chunk, if the next one starts another segment, the finished
    // segment is folded in with its row scale.  Branch-free (selects), so a
    // chunk's table reads and the adds that consume them share one block.
    auto consume = [&](int ch, const u32x4 w, int u) {
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
          lookup_word<G, NB, EB>(w[q], base, acc, q * (32 / G));
          // wider batches: one word's table reads at a time
          if constexpr (NB >= 4) asm volatile("" ::: "memory");
        }
      }
      if constexpr (RS == 0) {
        next_chunk(L, ls, lcis);
        const bool fold = ls != cur;  // uniform
        const float rc = pick6(cur - s0, rv0, rv1, rv2, rv3, rv4, rv5);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          part[b] = fold ? fmaf(rc, acc[b], part[b]) : part[b];
          acc[b] = fold ? 0.0f : acc[b];
        }
        cur = ls;
      } else if constexpr (!SAL) {
        // block-wise global chunk: one group, scaled once summed
        const float rc = h2f((uint16_t)rg[u]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          part[b] = fmaf(rc, acc[b], part[b]);
          acc[b] = 0.0f;
        }
      }
      // the next chunk's table reads stay behind this chunk's (registers)
      asm volatile("" ::: "memory");
    };
    int ch0 = 0;
    for (; ch0 + D < nch; ch0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        // consumed before the refill is issued into the same registers: with
        // both alive the compiler would rotate registers with copies that wait
        consume(ch0 + u, wb[u], u);
        load_into(u);
        __builtin_amdgcn_sched_barrier(0);  // issue the refill here, not later
      }
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (ch0 + u < nch) consume(ch0 + u, wb[u], u);
    if constexpr (RS == 0) {
      if (cur <= s_last) {  // the range ended inside a segment: fold its remainder
        const float rc = pick6(cur - s0, rv0, rv1, rv2, rv3, rv4, rv5);
#pragma unroll
        for (int b = 0; b < NB; ++b) part[b] = fmaf(rc, acc[b], part[b]);
      }
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
    //
    // With several batch rows, all NB atomics are issued before any result
    // is examined, so that their round trips overlap instead of queueing one
    // behind the other.
    if constexpr (NB == 1) {
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
    } else if (row_ok) {
      uint64_t contrib[NB], old[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float scaled = fminf(fmaxf(part[b] * kFixScale, -kFixClamp), kFixClamp);
        contrib[b] = (uint64_t)(__float2ll_rn(scaled) + kFixBias);
        old[b] = 0;
        if (b < a.batch)
          old[b] = __hip_atomic_fetch_add(a.acc + (int64_t)b * a.n_pad + row, contrib[b] + kOneArrival,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b < a.batch && (int)(old[b] >> kCountShift) == a.splits - 1) {
          const int64_t total = (int64_t)((old[b] & kValueMask) + contrib[b]) - (int64_t)a.splits * kFixBias;
          a.y[(int64_t)b * L.n + row] = f2h(__ll2float_rn(total) * kFixInv);
          __hip_atomic_store(a.acc + (int64_t)b * a.n_pad + row, (uint64_t)0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
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

// Instance for (batch width, waves, prefetch depth) at table width G,
// row-scale format RS and table entry type TQ, or nullptr.
template <int G, int NB, int W, int RS, int TQ>
gemv_fn gemv_pick_pf(int pf) {
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
    switch (nb) {
      case 8: return gemv_pick_waves<G, 8, RS, TQ>(waves, pf);
      case 16: return gemv_pick_waves<G, 16, RS, TQ>(waves, pf);
    }
  }
  return nullptr;
}

}  // namespace fluxbin
