// gemv_banked.hpp -- the LUT GEMV kernel for g = 8 with bank-private tables
// (gfx950 / CDNA4): one batch row, per-row scales, fp32 table entries.
//
// The problem it solves.  With lane = row, every lane of a wave looks up the
// same 256-entry table at each step, at its own random pattern: 32 lanes land
// on about 32 random dwords of one 1 KiB table and collide in the LDS banks
// (the LUT Tensor Core notes, section 2.3 and Figure 4, on where large tables
// should live; FluxBin summary, appendix E.2, on the 8-wide sub-vectors).  On
// the LLaMA-2-7B g = 8 gate+up shape such stalls were two thirds of the
// LDS-active cycles.
//
// The layout.  A region of R chunks (R = 2 or 4) of a workgroup's column
// range has 16 R tables, table T = 16 c + t for sub-vector t (8 columns) of
// chunk c of the region; a range is one region, or two 2-chunk regions whose
// tables are built and looked up in turn in the same LDS.  Entry p of table
// T is the dword p * 16R + T: each table is a
// column of the LDS, one bank (dword address mod 32, or mod 64 for R = 4)
// holding all of it.  A lane is a (chunk c, row) pair, 16 rows per chunk:
// at step i (0..15) the lane with row index r (0..15 in its group of 16)
// looks up sub-vector t = i XOR r of its chunk.  In any half wave the 32
// lanes then read 32 different tables, so 32 different banks, whatever their
// patterns: the table reads never conflict.
//
// What that takes per lane: its 16 bytes of sign words hold sub-vectors
// 0..15 in order (byte t mod 4 of word t / 4), so it reads word q XOR (r / 4)
// at step group q (the 4 words permuted once per load, 8 selects) and byte
// kk XOR (r mod 4) of it; one v_perm_b32 with a per-lane selector picks that
// byte and merges it with the table's column, which makes the LDS address.
// A lane keeps its chunk position c in every region, so its sums run on
// across regions.  After the range, the partial sums of one row are spread
// over the R chunk lanes that share it and are added with R = 4: two, R = 2:
// one cross-lane exchange, after which each lane owns one row of the 64-row
// tile.
#pragma once

#include "common.hpp"

namespace fluxbin {

// One lane's view of a banked region of R chunks: lane (c, r) of chunk c
// looks up, at step (q, kk) of a 16-byte group of sign words, sub-vector
// t = (4 q + kk) XOR r, table T = 16 c + t.  slot[q] holds in byte kk the
// byte SLOT * T, sel[kk] is the v_perm_b32 selector that puts that byte into
// bits 0-7 of the address and byte kk XOR (r mod 4) of the reordered word
// into bits 8-15 (the pattern p), giving p * 256 + 4 T (R = 4), or
// p * 256 + 8 T, halved to p * 128 + 4 T (R = 2).
template <int R>
struct BankedLane {
  static constexpr uint32_t SLOT = R == 4 ? 4 : 8;
  uint32_t slot[4], sel[4];
  bool b0, b1;

  __device__ __forceinline__ BankedLane(int c, int r) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t sv = 0;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sv |= (SLOT * (uint32_t)(16 * c + ((4 * q + kk) ^ r))) << (8 * kk);
      slot[q] = sv;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) sel[kk] = 0x0c0c0000u | ((uint32_t)(kk ^ (r & 3)) << 8) | (uint32_t)(4 + kk);
    b0 = (r >> 2) & 1;
    b1 = (r >> 3) & 1;
  }

  // the lane's four words in step order: word q is word q XOR (r / 4)
  __device__ __forceinline__ void order(const u32x4 w, uint32_t (&ew)[4]) const {
    const uint32_t f0 = b0 ? w[1] : w[0], f1 = b0 ? w[0] : w[1];
    const uint32_t f2 = b0 ? w[3] : w[2], f3 = b0 ? w[2] : w[3];
    ew[0] = b1 ? f2 : f0;
    ew[1] = b1 ? f3 : f1;
    ew[2] = b1 ? f0 : f2;
    ew[3] = b1 ? f1 : f3;
  }

  // the table entry of step (q, kk) for the reordered words ew (the region
  // starts at LDS address 0)
  __device__ __forceinline__ float entry(const uint32_t (&ew)[4], int q, int kk) const {
    uint32_t ad = __builtin_amdgcn_perm(slot[q], ew[q], sel[kk]);
    if constexpr (R == 2) ad >>= 1;
    return lds_f32(ad);
  }
};

// R = 2 layouts take 33 KiB: four workgroups of 8 waves fit a CU, and the
// registers are held to 64 for 8 waves per SIMD.  R = 4 layouts take 66 KiB:
// two workgroups per CU, so they run 16 waves (1024 rows) to fill it.
template <int R, int WAVES>
constexpr int banked_waves_per_eu() {
  return (R == 2 || WAVES == 16) ? 8 : 1;
}

// A column range of up to NREG regions of R chunks: the inputs of all of
// them are staged and all of their sign words requested at once; the regions'
// tables are then built and looked up one after the other in the same LDS.
template <int R, int WAVES, int NREG>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(banked_waves_per_eu<R, WAVES>())))
void lut_gemv_g8_banked_kernel(const GemvArgs a) {
  static_assert(R == 2 || R == 4, "region of 2 or 4 chunks");
  static_assert(NREG == 1 || NREG == 2, "one or two regions per range");
  constexpr int NT = WAVES * 64;
  constexpr int NTAB = 16 * R;        // tables of the region
  constexpr int ITEMS = R * kChunkCols * NREG;
  constexpr int VPT = ITEMS >= NT ? ITEMS / NT : 1;
  constexpr int GR = 64 / R;          // rows of one row group: 16 rows per chunk lane group x R chunks = 64 lanes
  constexpr int NG = R;               // row groups of the wave's 64-row tile
  static_assert(ITEMS % NT == 0 || NT % ITEMS == 0, "staging rounds");
  extern __shared__ __align__(1024) float smem[];
  float *s_tab = smem;
  float *s_v = smem + NTAB * 256;
  // The kernel has no static LDS, so its dynamic LDS, and the table region
  // with it, starts at LDS address 0: table addresses carry no base.  (Were
  // that ever not so, the kernel would write nothing, not wrong numbers.)
  if (lds_addr(s_tab) != 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = blockIdx.x;  // row block
  const int sp = blockIdx.y;  // column range
  const int tile = rb * WAVES + wave;

  // lane roles: r = row within a group of 16 (and the rotation of the lane's
  // sub-vector order), c = chunk of the range, h = which 16 rows of a 32-row
  // group (R = 2)
  const int r = lane & 15;
  const int cq = lane >> 4;
  const int c = cq % R;
  const int h = cq / R;
  // the row this lane owns after the cross-lane sum: group c of the tile
  const int orow = c * GR + h * 16 + r;
  const int row = tile * kTileRows + orow;
  const bool row_ok = tile < a.row_tiles && row < a.n;

  const ColRange cr = column_range(a, sp);
  const SegRef S = cr.S;
  const int c_lo = cr.c_lo, nch = cr.nch;
  // this lane's 16 bytes of row group g of region q: element
  // ((tile * nchunks + c_lo + q R + c) * 64 + g * GR + h * 16 + r); waves past
  // the last tile read the last one and store nothing; lanes whose chunk does
  // not exist (ranges may be shorter than NREG R) load nothing
  const int ltile = min(tile, a.row_tiles - 1);
  const FB_GLOBAL u32x4 *wp = S.bits + ((int64_t)ltile * S.nchunks + c_lo) * kTileRows + h * 16 + r;

  auto body = [&](auto sal_tag) {
    constexpr bool SAL = decltype(sal_tag)::value;
    const FB_GLOBAL int32_t *uidx = uni(a.idx_or_dummy);
    const FB_GLOBAL uint16_t *ux = uni(a.x);
    const uint16_t rr16 = S.r[row_ok ? row : 0];

    // Staged inputs: item e = (chunk e / 128, column e % 128) of the region,
    // zero where the chunk or column does not exist, so that missing chunks
    // get all-zero tables and their lanes add nothing.
    const bool stager = ITEMS >= NT || tid < ITEMS;  // uniform per wave
    bool live[VPT];
    uint32_t ccl[VPT], gi[VPT], cvl[VPT], xvl[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = tid + i * NT;
      const int ch = e >> 7;
      const uint32_t cc = (uint32_t)((c_lo + ch) * kChunkCols + (e & (kChunkCols - 1)));
      live[i] = stager & (ch < nch) & (cc < (uint32_t)S.len);
      ccl[i] = live[i] ? cc : 0u;
      cvl[i] = S.c[ccl[i]];
    }
    u32x4 wb[NREG][NG];
    auto issue_weights = [&]() {
#pragma unroll
      for (int q = 0; q < NREG; ++q) {
        const int ch = q * R + c;
        const bool cl = ch < nch;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          wb[q][g] = u32x4{0u, 0u, 0u, 0u};
          if (cl) wb[q][g] = __builtin_nontemporal_load(wp + (cl ? ch : 0) * kTileRows + g * GR);
        }
      }
    };
    if constexpr (!SAL) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) xvl[i] = ux[ccl[i]];
      __builtin_amdgcn_sched_barrier(0);
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) gi[i] = (uint32_t)uidx[ccl[i]];
      __builtin_amdgcn_sched_barrier(0);
      issue_weights();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < VPT; ++i) xvl[i] = ux[gi[i]];
    }
    if (stager) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t m = live[i] ? 0xffffu : 0u;
        s_v[tid + i * NT] = h2f((uint16_t)(cvl[i] & m)) * h2f((uint16_t)(xvl[i] & m));
      }
    }
    __syncthreads();

    const BankedLane<R> L(c, r);
    float acc[NG][2];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
    for (int rq = 0; rq < NREG; ++rq) {
      if (rq * R >= nch) break;  // uniform: the range ends before this region
      if (rq > 0) __syncthreads();  // every wave is done with the previous region's tables
      // Tables: unit u = (combo, T), T fastest, so that the 64 lanes of a
      // store write 64 consecutive dwords (one row p of the layout, or two).
      for (int u = tid; u < NTAB * 16; u += NT) {
        const int T = u & (NTAB - 1);
        const int un = u / NTAB;
        float e[16];
        g8_unit_entries(s_v + rq * R * kChunkCols + 8 * T, un, e);
        const int p0 = ((un >> 3) << 7) | (un & 7);
        float *tb = s_tab + p0 * NTAB + T;
#pragma unroll
        for (int m = 0; m < 16; ++m) tb[m * 8 * NTAB] = e[m];
      }
      __syncthreads();

      uint32_t ew[NG][4];
#pragma unroll
      for (int g = 0; g < NG; ++g) L.order(wb[rq][g], ew[g]);
      // the row groups' lookups of one step go out together (independent reads)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int g = 0; g < NG; ++g) acc[g][kk & 1] += L.entry(ew[g], q, kk);
        }
      }
    }

    // Sum each row over the R chunk lanes that hold it; lane (c, ...) keeps
    // row group c.
    float own;
    if constexpr (R == 4) {
      const bool x0 = c & 1, x1 = (c >> 1) & 1;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = acc[j][0] + acc[j][1];
      // exchange with chunk c ^ 1: keep the groups of c's parity
      const float send0 = x0 ? v[0] : v[1], send1 = x0 ? v[2] : v[3];
      const float keep0 = x0 ? v[1] : v[0], keep1 = x0 ? v[3] : v[2];
      const float e0 = keep0 + __shfl_xor(send0, 16);
      const float e1 = keep1 + __shfl_xor(send1, 16);
      // exchange with chunk c ^ 2: keep group c
      const float send = x1 ? e0 : e1, keep = x1 ? e1 : e0;
      own = keep + __shfl_xor(send, 32);
    } else {
      const bool x0 = c & 1;
      const float v0 = acc[0][0] + acc[0][1], v1 = acc[1][0] + acc[1][1];
      own = (x0 ? v1 : v0) + __shfl_xor(x0 ? v0 : v1, 16);
    }
    const float part[1] = {h2f(rr16) * own};
    finish_rows<1>(a, row, row_ok, part);
  };
  if (cr.sg < a.kb) {
    body(BoolTag<false>{});
  } else {
    body(BoolTag<true>{});
  }
}

template <int R, int NREG>
gemv_fn gemv_pick_banked_waves(int waves) {
  return waves == 16  ? lut_gemv_g8_banked_kernel<R, 16, NREG>
         : waves == 8 ? lut_gemv_g8_banked_kernel<R, 8, NREG>
         : waves == 4 ? lut_gemv_g8_banked_kernel<R, 4, NREG>
                      : nullptr;
}

}  // namespace fluxbin
