// gemm_mfma.hpp -- the layer product for prefill-size batches on the matrix
// cores (gfx950 MFMA).
//
// The same product as the LUT GEMV, y[b] = sum over segments of
// r (.) (B (c (.) x[b])) (FluxBin summary, section 3 "Quantization" and
// "Salient-Aware Hybrid Bases"; x[S] gathered for the salient bases, section
// 3 "Virtual Columnar Mapping"), evaluated as a dense contraction: with a
// batch of tens of rows the table build and lookups of the LUT route cost
// per batch row, while a matrix-core product costs per weight bit.
//
// Operands of v_mfma_f32_32x32x16_f16 (D[m][n] = sum_k A[m][k] B[k][n] + C):
//   A = 32 batch rows x 16 columns of x, fp16 as given (staged in LDS);
//   B = 16 columns x 32 weight rows of the basis, expanded in registers from
//       the sign bits to +-c_j (fp16: only the sign bit of c_j changes, so
//       the expansion is exact).
// Every product c_j * x_bj is exact in the matrix core's fp32 arithmetic, so
// only the fp32 accumulation rounds.  Lane l supplies row (l mod 32) of A and
// column (l mod 32) of B for the 8 columns 8 * (l / 32) .. + 7 of the k-step;
// the instruction pairs A and B slot by slot, so any column order that both
// operands share gives the same sum.  D: lane l holds weight row (l mod 32)
// and the 16 batch rows 8 * (v / 4) + 4 * (l / 32) + (v mod 4), v < 16, so
// each lane scales its 16 sums by one row scale.
//
// Work division: a wave covers 32 * RB weight rows (RB = 2: one tile of the
// sign-word layout, so each x fragment read from LDS feeds two MFMAs; RB = 1:
// half a tile, twice the workgroups) x 32 * NBT batch rows, each expanded
// sign operand feeding NBT MFMAs.  A workgroup of 4 waves (WB along the
// batch, 4 / WB along the rows) covers (4 / WB) * 32 * RB rows x 32 * NBT * WB
// batch rows x a range of at most cpb 128-column chunks of ONE segment.  Per
// chunk the workgroup stages the chunk's columns of x (gathered through S for
// a salient segment), its column scales and its sign words in LDS, zero past
// the segment's end.  Ranges that cover the same rows add their scaled
// partials in fp32, summed in range order by a second kernel (plain stores
// and loads: no atomics, a fixed order of addition).
//
// Row scales: per row (RS = 0), applied once to the range's sum; block-wise
// (RS = 1), per 128-column group for the global bases (after every chunk)
// and per sal_group compact columns for the salient ones (after every k-step,
// or, with 8-column groups, after each half of it: the k-step runs as two
// MFMAs whose B operand keeps one 8-column half each).
#pragma once

#include "common.hpp"

namespace fluxbin {

constexpr int kMfmaWaves = 4;
constexpr int kMfmaMaxBlocks = 4;               // 32-row batch blocks of a call, at most (batch <= 128)
constexpr int kMfmaRowsPerBlock = 256;          // weight rows per workgroup of the instance in use
constexpr int kMfmaXStride = kChunkCols + 8;    // halfs per staged batch row: 272 B, conflict-free 16-B reads

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct MfmaArgs {
  LayerArgs L;
  const int32_t *idx_or_dummy;  // sal_idx, or a valid one-element array when ks == 0
  const uint16_t *x;            // fp16 [batch][k]
  uint16_t *y;                  // fp16 [batch][n]
  float *part;                  // [splits][batch][n_pad] fp32 partial sums (splits > 1)
  int64_t n_pad;
  int64_t rstride_g;            // row-scale elements per global / salient basis: n (per row), or the
  int64_t rstride_s;            // basis' block of the tiled scale layout (block-wise)
  int32_t cpb;                  // chunks per range
  int32_t ranges_g;             // ranges per global segment: ceil(nc_g / cpb)
  int32_t ranges_s;             // ranges per salient segment: ceil(nc_s / cpb)
  int32_t row_tiles;            // ceil(n / 64)
  int32_t row_blocks;           // ceil(n / 128)
  int32_t splits;               // kb * ranges_g + ks * ranges_s
  int32_t batch;
  int32_t xvec;                 // k % 8 == 0 and x, c_global 16-byte aligned: full global chunks
                                // are staged with 16-byte loads
  int32_t sal_group;            // block-wise salient columns per group (8 or 16)
};

typedef void (*mfma_fn)(const MfmaArgs);

// A kernel instance: NBT 32-row batch blocks and RB 32-row blocks of weight
// rows per wave, WB waves along the batch (the other 4 / WB along the rows).
struct MfmaInstance {
  mfma_fn fn;
  int nbt, wb, rb;
};

// The instance for a call of `batch` rows (1..128) with row-scale format rs
// (0 per row, 1 block-wise); fn is nullptr outside that range.  The same
// instance serves every batch (NBT = WB = 1, RB = 2: kMfmaRowsPerBlock
// weight rows by 32 batch rows per workgroup).
MfmaInstance mfma_instance(int64_t batch, int rs);

// Static LDS of an instance: two buffers of x ([32 * nbt * wb][kMfmaXStride]
// fp16), c (128 fp16) and the sign words of its (4 / wb) * 32 * rb rows.
constexpr int mfma_lds_bytes(int nbt, int wb, int rb) {
  return 2 * (32 * nbt * wb * kMfmaXStride * 2 + kChunkCols * 2 + (kMfmaWaves / wb) * 32 * rb * 16);
}

// Automatic chunks per range for a layer of row_blocks 128-row blocks, kb / ks
// segments of nc_g / nc_s chunks, and calls of at most max_batch rows.
int32_t mfma_auto_cpb(int32_t row_blocks, int32_t kb, int32_t nc_g, int32_t ks, int32_t nc_s, int64_t max_batch);


// B operand of one k-step: the 8 column scales c8 with the sign of each
// flipped where its weight bit is clear.  `neg` holds the 8 inverted bits
// (bit e set = column e is -1); E = neg | neg << 15 puts bit 2d at 2d and bit
// 2d + 1 at 2d + 16, so E << (15 - 2d) lands them on the sign bits 15 and 31
// of dword d (the fp16 pair of columns 2d, 2d + 1).
// (The shifts are written as instructions: left to itself the compiler folds
// E's two shifted copies into one quarter-rate integer multiply per dword.)
template <int SH>
__device__ __forceinline__ uint32_t shl(uint32_t v) {
  uint32_t r;
  asm("v_lshlrev_b32 %0, %1, %2" : "=v"(r) : "n"(SH), "v"(v));
  return r;
}

__device__ __forceinline__ half8_t signed_scales(uint32_t neg, u32x4 c8) {
  const uint32_t e = neg | (neg << 15);
  u32x4 v;
  v[0] = c8[0] ^ (shl<15>(e) & 0x80008000u);
  v[1] = c8[1] ^ (shl<13>(e) & 0x80008000u);
  v[2] = c8[2] ^ (shl<11>(e) & 0x80008000u);
  v[3] = c8[3] ^ (shl<9>(e) & 0x80008000u);
  return __builtin_bit_cast(half8_t, v);
}

// Waves per SIMD the register allocation must leave room for: two for the
// block-wise instances (one batch block per wave; their second accumulator
// set would otherwise take them to one wave per SIMD), no constraint else.
template <int NBT, int WB, int RB, int RS>
struct MfmaWavesPerEu {
  static constexpr int value = RS == 1 ? 2 : 1;
};

template <int NBT, int WB, int RB, int RS>
__global__ __launch_bounds__(kMfmaWaves * 64)
__attribute__((amdgpu_waves_per_eu(MfmaWavesPerEu<NBT, WB, RB, RS>::value))) void gemm_mfma_kernel(const MfmaArgs a) {
  static_assert(RB == 1 || RB == 2, "a wave covers 32 or 64 weight rows");
  constexpr int WR = kMfmaWaves / WB;           // waves along the rows
  constexpr int kWaveRows = 32 * RB;            // weight rows per wave
  constexpr int kRows = WR * kWaveRows;         // weight rows of the workgroup
  constexpr int kBatchRows = 32 * NBT * WB;     // staged batch rows
  constexpr int kPieces = kBatchRows / 16;      // 16-byte pieces of x per thread per chunk
  constexpr int kXHalfs = kBatchRows * kMfmaXStride;
  // Two LDS buffers of one chunk each: x [kBatchRows][kMfmaXStride], c [128], sign words [kRows]
  static_assert(2 * (kXHalfs * 2 + kChunkCols * 2 + kRows * 16) == mfma_lds_bytes(NBT, WB, RB), "LDS plan");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kXHalfs];
  __shared__ __attribute__((aligned(16))) uint16_t cs[2][kChunkCols];
  __shared__ __attribute__((aligned(16))) u32x4 ws[2][kRows];

  const ULayer L = uniform_layer(a.L);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave % WR, wb = wave / WR;
  const int m = lane & 31, kq = lane >> 5;
  const int rb = blockIdx.x % a.row_blocks;
  const int sp = blockIdx.x / a.row_blocks;
  const int b0 = blockIdx.y * kBatchRows;       // first batch row of the workgroup
  const int batch = a.batch;

  // the range: one segment, chunks [c0, c0 + nch)
  int sg, c0;
  {
    const int gr = L.kb * a.ranges_g;
    if (sp < gr) {
      sg = sp / a.ranges_g;
      c0 = (sp - sg * a.ranges_g) * a.cpb;
    } else {
      const int q = sp - gr;
      const int b = q / a.ranges_s;
      sg = L.kb + b;
      c0 = (q - b * a.ranges_s) * a.cpb;
    }
  }
  sg = __builtin_amdgcn_readfirstlane(sg);
  c0 = __builtin_amdgcn_readfirstlane(c0);
  const SegRef S = segment(L, sg);
  const FB_GLOBAL uint16_t *rbase =
      S.salient ? L.r_s + (sg - L.kb) * uni(a.rstride_s) : L.r_g + sg * uni(a.rstride_g);
  const int nch = min(a.cpb, S.nchunks - c0);
  const int len = (int)S.len;
  const int nc = S.nchunks;

  const FB_GLOBAL int32_t *idx = uni(a.idx_or_dummy);
  const FB_GLOBAL uint16_t *xg = uni(a.x);
  const bool xvec = a.xvec != 0;
  const int gpc = S.salient ? kChunkCols / a.sal_group : 1;  // block-wise scales per row per chunk

  // Staging, per thread and chunk: pieces i of x = batch row (tid / 16 + 16 i),
  // columns 8 * (tid % 16) .. + 7 of the chunk; the same 8 columns of c; the
  // chunk's sign words of workgroup row `tid` (tid < kRows).  Rows past the
  // last tile read the last tile; batch rows past the batch read the last
  // batch row (rows of A only reach the same rows of D, which are not stored).
  // Offsets are loop invariant: per chunk only the uniform base moves.
  const int pcol = 8 * (tid & 15);
  int xoff[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) xoff[i] = min(b0 + (tid >> 4) + 16 * i, batch - 1) * (int)L.k + pcol;
  const int wrow = min(tid, kRows - 1);         // workgroup row whose sign words this thread stages
  const int wgrow = rb * kRows + wrow;          // its global row
  const int wtile = min(wgrow / kTileRows, a.row_tiles - 1);
  const int64_t woff = (int64_t)wtile * nc * kTileRows + (wgrow % kTileRows);

  // This wave's 32 * RB weight rows (a tile of the sign-word layout, or half
  // of one); the lane holds rows 32 i + m of them.
  const int row0 = (rb * WR + wr) * kWaveRows;
  const int tile = min(row0 / kTileRows, a.row_tiles - 1);
  const int trow0 = row0 % kTileRows;           // 0, or 32 for the second half of a tile
  const int wbat = b0 + wb * NBT * 32;          // first batch row of this wave
  const int64_t roff0 = ((int64_t)tile * nc * kTileRows + trow0 + m) * gpc;  // block-wise scales, chunk 0
  // per-row scales of the lane's two rows, loaded now so the epilogue does not wait for them
  float rrow[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) rrow[i] = 1.0f;
  if constexpr (RS == 0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int row = row0 + 32 * i + m;
      rrow[i] = h2f(rbase[min(row, (int)L.n - 1)]);
    }
  }

  struct Stage {
    u32x4 x[kPieces];
    u32x4 c, w, r0[RB], r1[RB];
  };
  // Loads of chunk cis.  A full chunk of a global segment (the common case)
  // takes 16-byte loads and no branch; one that reaches past the segment's
  // end, or of a salient segment (gathered through S), goes element by
  // element: clamped addresses, values past the end zeroed.
  auto stage = [&](int cis, Stage &st) {
    const int col0 = cis * kChunkCols;
    st.w = __builtin_nontemporal_load(S.bits + (woff + (int64_t)cis * kTileRows));
    if constexpr (RS == 1) {
      const FB_GLOBAL uint16_t *rp = rbase + roff0 + (int64_t)cis * kTileRows * gpc;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const FB_GLOBAL uint16_t *ri = rp + 32 * i * gpc;
        if (S.salient) {
          st.r0[i] = *(const FB_GLOBAL u32x4 *)ri;
          st.r1[i] = gpc == 16 ? *(const FB_GLOBAL u32x4 *)(ri + 8) : st.r0[i];
        } else {
          st.r0[i][0] = *ri;
        }
      }
    }
    if (!S.salient && xvec && col0 + kChunkCols <= len) {
      const FB_GLOBAL uint16_t *xc = xg + col0;
#pragma unroll
      for (int i = 0; i < kPieces; ++i) st.x[i] = *(const FB_GLOBAL u32x4 *)(xc + xoff[i]);
      st.c = *(const FB_GLOBAL u32x4 *)(S.c + col0 + pcol);
      return;
    }
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const FB_GLOBAL uint16_t *xr = xg + (xoff[i] - pcol);
      uint32_t h[8];
      if (S.salient) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = col0 + pcol + e;
          const uint32_t xv = xr[idx[min(col, len - 1)]];
          h[e] = col < len ? xv : 0u;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = col0 + pcol + e;
          const uint32_t xv = xr[min(col, len - 1)];
          h[e] = col < len ? xv : 0u;
        }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) st.x[i][d] = h[2 * d] | (h[2 * d + 1] << 16);
    }
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = col0 + pcol + e;
      h[e] = col < len ? (uint32_t)S.c[min(col, len - 1)] : 0u;
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) st.c[d] = h[2 * d] | (h[2 * d + 1] << 16);
  };
  // block-wise scales of the chunk being multiplied, per lane row: fp16 pairs,
  // scale q in half (q & 1) of word (q / 2) of rqa (q < 8) or rqb
  u32x4 rqa[RB], rqb[RB];
  auto publish = [&](const Stage &st, int buf) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) *(u32x4 *)&xs[buf][((tid >> 4) + 16 * i) * kMfmaXStride + pcol] = st.x[i];
    if (tid < kChunkCols / 8) *(u32x4 *)&cs[buf][pcol] = st.c;
    if (tid < kRows) ws[buf][tid] = st.w;
    if constexpr (RS == 1) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        rqa[i] = st.r0[i];
        rqb[i] = st.r1[i];
      }
    }
  };

  // acc[i][j]: rows (32 i + .) of the wave, batch block j.  Block-wise scales
  // fold each group's sum into out; per-row scales multiply acc once at the end.
  f32x16 acc[RB][NBT];
  f32x16 out[RB][RS == 1 ? NBT : 1];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
#pragma unroll
    for (int j = 0; j < NBT; ++j) acc[i][j] = f32x16{};
#pragma unroll
    for (int j = 0; j < (RS == 1 ? NBT : 1); ++j) out[i][j] = f32x16{};
  }
  auto fold = [&](int i, float r) {
    if constexpr (RS == 1) {
#pragma unroll
      for (int j = 0; j < NBT; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) out[i][j][v] = fmaf(r, acc[i][j][v], out[i][j][v]);
        acc[i][j] = f32x16{};
      }
    }
  };

  auto compute = [&](int cis, int buf) {
    u32x4 nw[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) nw[i] = ~ws[buf][wr * kWaveRows + 32 * i + m];
    // block-wise scale q of lane row i (q a compile-time index after unrolling)
    auto rscale = [&](int i, int q) {
      const uint32_t w = q < 8 ? rqa[i][(q >> 1) & 3] : rqb[i][(q >> 1) & 3];
      return h2f((uint16_t)(w >> (16 * (q & 1))));
    };
#pragma unroll
    for (int t = 0; t < kChunkCols / 16; ++t) {
      const int kc = 16 * t + 8 * kq;  // this lane's 8 columns of the k-step
      const u32x4 c8 = *(const u32x4 *)&cs[buf][kc];
      half8_t aop[NBT];
#pragma unroll
      for (int j = 0; j < NBT; ++j)
        aop[j] = *(const half8_t *)&xs[buf][((wb * NBT + j) * 32 + m) * kMfmaXStride + kc];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint32_t neg = (nw[i][t >> 1] >> (16 * (t & 1) + 8 * kq)) & 0xffu;
        const half8_t bop = signed_scales(neg, c8);
        if (RS == 1 && S.salient && gpc == 16) {
          // 8-column groups: each half of the k-step is its own group
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const half8_t bh = kq == h ? bop : half8_t{};
#pragma unroll
            for (int j = 0; j < NBT; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[j], bh, acc[i][j], 0, 0, 0);
            fold(i, cis * kChunkCols + 16 * t + 8 * h < len ? rscale(i, 2 * t + h) : 0.0f);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NBT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop[j], bop, acc[i][j], 0, 0, 0);
          // 16-column groups: one per k-step (groups past the segment's end may hold any scale)
          if (RS == 1 && S.salient) fold(i, cis * kChunkCols + 16 * t < len ? rscale(i, t) : 0.0f);
        }
      }
    }
    if (RS == 1 && !S.salient) {
#pragma unroll
      for (int i = 0; i < RB; ++i) fold(i, rscale(i, 0));
    }
  };

  // Pipeline: chunk u is multiplied from LDS buffer u % 2 while the loads of
  // chunk u + 1 are in flight; they are published to the other buffer after
  // the multiply, then one barrier, then the loads of chunk u + 2 start.  (A
  // second register set in flight cost the widest instance its second wave
  // per SIMD, and was measured slower.)
  Stage st;
  stage(c0, st);
  publish(st, 0);
  __syncthreads();
  if (nch > 1) stage(c0 + 1, st);
  for (int u = 0; u < nch; ++u) {
    compute(c0 + u, u & 1);
    if (u + 1 < nch) {
      publish(st, (u + 1) & 1);
      __syncthreads();
      if (u + 2 < nch) stage(c0 + u + 2, st);
    }
  }

  // out[i][j][v] is (batch row wbat + 32 j + 8 (v / 4) + 4 kq + v % 4, weight row row0 + 32 i + m).
  // One range per row: y directly.  Several: this range's partial sums, fp32,
  // to part[range][batch row][n_pad], added in range order by the finalize
  // kernel (a fixed order, so repeated calls agree bit for bit).
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int row = row0 + 32 * i + m;
    if (row >= L.n) continue;
    const float r = rrow[i];  // per-row scale of the range's sum (1 when block-wise)
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int br = wbat + 32 * j + 8 * (v >> 2) + 4 * kq + (v & 3);
        if (br >= batch) continue;
        const float val = RS == 0 ? r * acc[i][j][v] : out[i][j][v];
        if (a.splits == 1)
          a.y[(int64_t)br * L.n + row] = f2h(val);
        else
          a.part[((int64_t)sp * batch + br) * a.n_pad + row] = val;
      }
    }
  }
}

// Sum of the ranges' partials of every output, in range order, to fp16.  The
// loads of eight ranges are issued together; the additions keep their order.
static __global__ __launch_bounds__(256) void mfma_finalize_kernel(const float *part, int32_t splits, int32_t batch,
                                                                   int64_t n, int64_t n_pad, uint16_t *y) {
  const int64_t total = (int64_t)batch * n;
  const int64_t stride = (int64_t)batch * n_pad;  // between ranges
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / n, row = i - b * n;
    const float *p = part + b * n_pad + row;
    float s = 0.0f;
    int r = 0;
    for (; r + 8 <= splits; r += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = p[(int64_t)(r + q) * stride];
#pragma unroll
      for (int q = 0; q < 8; ++q) s += v[q];
    }
    for (; r < splits; ++r) s += p[(int64_t)r * stride];
    y[i] = f2h(s);
  }
}

}  // namespace fluxbin
