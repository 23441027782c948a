// decomp_kernels.hpp -- the offline row-column binary decomposition on gfx950.
//
// W ~ sum_b diag(r_b) B_b diag(c_b) (FluxBin summary, section 3 bullets
// "Quantization" and "Parameter Optimization"; appendix A.1: closed-form
// least-squares row and column scales of one basis with the rest fixed;
// appendix A.2: exhaustive per-element search over the Kb signs, globally
// optimal for fixed scales).  Working scales are fp64.  Layouts: W fp16
// [n][k] row-major; sign words canonical [kb][n][ceil(k/32)] (column 32w+t of
// a row at bit t of word w, bit set = +1); r [kb][n], c [kb][k]; optional
// per-column weights d [k] of the weighted least squares.
//
// Every sum of one approximation W_hat_ij over the bases, and every sign
// decision, is evaluated in fp64 in basis order with each product rounded
// once (no fused multiply-add: contraction is switched off in these
// functions), so a decision depends only on its inputs.  Sums over a row or a
// column (the least-squares numerators, the error) are split over lanes and
// workgroups in a fixed order: deterministic, equal to the sequential sum up
// to rounding.
#pragma once

#include "common.hpp"

namespace fluxbin {

constexpr int kDecompRowChunk = 64;     // rows per partial of the column step
constexpr int kDecompErrBlocks = 1024;  // workgroups (partials) of the error reduction

__device__ __forceinline__ double sign_of_word(uint32_t word, int64_t j) { return ((word >> (j & 31)) & 1u) ? 1.0 : -1.0; }

// sum over bases l != skip of r_l,i B_l,ij c_l,j, in basis order (skip = -1: every basis)
__device__ __forceinline__ double decomp_approx(const uint32_t *bits, int64_t n, int64_t wpr, int64_t k, int kb,
                                                const double *r, const double *c, int64_t i, int64_t j, int skip) {
#pragma clang fp contract(off)
  double a = 0.0;
  for (int b = 0; b < kb; ++b) {
    if (b == skip) continue;
    const double s = sign_of_word(bits[((int64_t)b * n + i) * wpr + (j >> 5)], j);
    a += (r[(int64_t)b * n + i] * s) * c[(int64_t)b * k + j];
  }
  return a;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// out[0] = sum_t w_t * v_t^2 over t < len (w = NULL: 1), one workgroup of 1024
// threads: thread x adds t = x, x + 1024, ... in order, then the waves' sums
// are added in wave order.
constexpr int kSumsqThreads = 1024;
__global__ __launch_bounds__(kSumsqThreads) void decomp_sumsq_kernel(const double *__restrict__ v,
                                                                     const double *__restrict__ w, int64_t len,
                                                                     double *__restrict__ out) {
  __shared__ double part[kSumsqThreads / 64];
  double a = 0.0;
#pragma unroll 4
  for (int64_t t = threadIdx.x; t < len; t += kSumsqThreads) a += (w ? w[t] : 1.0) * v[t] * v[t];
  a = wave_sum(a);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int q = 0; q < kSumsqThreads / 64; ++q) s += part[q];
    out[0] = s;
  }
}

// Row step of basis `basis`: one wave per row.  The step reads the row scales
// of the other bases only, so r_out may be basis `basis`'s own row of r.
__global__ __launch_bounds__(256) void decomp_row_kernel(const uint16_t *w, int64_t n, int64_t k, int kb, int basis,
                                                         const uint32_t *bits, const double *r, const double *c,
                                                         const double *d, const double *den, double *r_out) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const int64_t wpr = (k + 31) / 32;
  const uint32_t *brow = bits + ((int64_t)basis * n + i) * wpr;
  const double *cb = c + (int64_t)basis * k;
  double num = 0.0;
  for (int64_t j = lane; j < k; j += 64) {
    const double res = (double)h2f(w[i * k + j]) - decomp_approx(bits, n, wpr, k, kb, r, c, i, j, basis);
    num += ((d ? d[j] : 1.0) * res * sign_of_word(brow[j >> 5], j)) * cb[j];
  }
  num = wave_sum(num);
  if (lane == 0) r_out[i] = den[0] > 0.0 ? num / den[0] : 0.0;
}

// Column step, first pass: partial[q][j] = sum over the rows of chunk q of R_ij B_ij r_i
// (reads the column scales of the other bases only).
__global__ __launch_bounds__(256) void decomp_col_partial_kernel(const uint16_t *w, int64_t n, int64_t k, int kb,
                                                                 int basis, const uint32_t *bits, const double *r,
                                                                 const double *c, double *partial) {
#pragma clang fp contract(off)
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t q = blockIdx.y;
  if (j >= k) return;
  const int64_t wpr = (k + 31) / 32;
  const double *rb = r + (int64_t)basis * n;
  double num = 0.0;
  const int64_t i1 = min(n, (q + 1) * kDecompRowChunk);
  for (int64_t i = q * kDecompRowChunk; i < i1; ++i) {
    const double res = (double)h2f(w[i * k + j]) - decomp_approx(bits, n, wpr, k, kb, r, c, i, j, basis);
    num += (res * sign_of_word(bits[((int64_t)basis * n + i) * wpr + (j >> 5)], j)) * rb[i];
  }
  partial[q * k + j] = num;
}

// Column step, second pass: c_out[j] = sum_q partial[q][j] / den, chunks in order.
__global__ __launch_bounds__(256) void decomp_col_finish_kernel(const double *partial, int64_t chunks, int64_t k,
                                                                const double *den, double *c_out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  double num = 0.0;
  for (int64_t q = 0; q < chunks; ++q) num += partial[q * k + j];
  c_out[j] = den[0] > 0.0 ? num / den[0] : 0.0;
}

// Sign words of one 64-column block of one row from a per-lane predicate: ballot
// bit l = column 64 * blk + l, i.e. canonical words 2 blk and 2 blk + 1.
__device__ __forceinline__ void store_ballot(uint32_t *row_words, int64_t wpr, int64_t blk, int lane, bool bit) {
  const uint64_t m = __ballot(bit);
  if (lane == 0) row_words[2 * blk] = (uint32_t)m;
  if (lane == 1 && 2 * blk + 1 < wpr) row_words[2 * blk + 1] = (uint32_t)(m >> 32);
}

// Sign step: one wave per (row, 64-column block); exhaustive search over the
// 2^KB combinations of each element, smallest combination index on ties.
template <int KB>
__global__ __launch_bounds__(256) void decomp_sign_kernel(const uint16_t *w, int64_t n, int64_t k,
                                                          const double *r, const double *c, uint32_t *bits_out) {
#pragma clang fp contract(off)
  const int64_t blocks = (k + 63) / 64;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= n * blocks) return;
  const int64_t i = wid / blocks, blk = wid - i * blocks;
  const int64_t j = blk * 64 + lane;
  const bool live = j < k;
  const int64_t jj = live ? j : k - 1;
  const double wv = (double)h2f(w[i * k + jj]);
  double p[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) p[b] = r[(int64_t)b * n + i] * c[(int64_t)b * k + jj];
  double best = __builtin_inf();
  int best_m = 0;
#pragma unroll
  for (int m = 0; m < (1 << KB); ++m) {
    double s = 0.0;
#pragma unroll
    for (int b = 0; b < KB; ++b) s = ((m >> b) & 1) ? s + p[b] : s - p[b];
    const double e = fabs(wv - s);
    if (e < best) {
      best = e;
      best_m = m;
    }
  }
  const int64_t wpr = (k + 31) / 32;
#pragma unroll
  for (int b = 0; b < KB; ++b)
    store_ballot(bits_out + ((int64_t)b * n + i) * wpr, wpr, blk, lane, live && ((best_m >> b) & 1));
}

// Initial signs of basis `basis`: +1 where the residual of the other bases is >= 0.
__global__ __launch_bounds__(256) void decomp_residual_sign_kernel(const uint16_t *w, int64_t n, int64_t k, int kb,
                                                                   int basis, const uint32_t *bits, const double *r,
                                                                   const double *c, uint32_t *basis_bits_out) {
#pragma clang fp contract(off)
  const int64_t blocks = (k + 63) / 64;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= n * blocks) return;
  const int64_t i = wid / blocks, blk = wid - i * blocks;
  const int64_t j = blk * 64 + lane;
  const bool live = j < k;
  const int64_t jj = live ? j : k - 1;
  const int64_t wpr = (k + 31) / 32;
  const double res = (double)h2f(w[i * k + jj]) - decomp_approx(bits, n, wpr, k, kb, r, c, i, jj, basis);
  store_ballot(basis_bits_out + i * wpr, wpr, blk, lane, live && res >= 0.0);
}

// Error, first pass: workgroup g sums d_j (W - W_hat)^2 over elements g*256 + t, step 256 * grid.
__global__ __launch_bounds__(256) void decomp_error_partial_kernel(const uint16_t *w, int64_t n, int64_t k, int kb,
                                                                   const uint32_t *bits, const double *r,
                                                                   const double *c, const double *d,
                                                                   double *partial) {
#pragma clang fp contract(off)
  __shared__ double part[4];
  const int64_t wpr = (k + 31) / 32;
  const int64_t total = n * k;
  double a = 0.0;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / k, j = e - i * k;
    const double res = (double)h2f(w[e]) - decomp_approx(bits, n, wpr, k, kb, r, c, i, j, -1);
    a += (d ? d[j] : 1.0) * res * res;
  }
  a = wave_sum(a);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = ((part[0] + part[1]) + part[2]) + part[3];
}

// Error, second pass: out[0] = sum of the partials in order (one thread).
__global__ void decomp_error_finish_kernel(const double *partial, int count, double *out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double a = 0.0;
  for (int t = 0; t < count; ++t) a += partial[t];
  out[0] = a;
}

// ---------------------------------------------------------------------------
// Tiled forms of the row, column and sign steps (k a multiple of 8, W 16-byte
// aligned).  A workgroup covers 512 columns x 64 rows: lane l of every wave
// owns columns 8l..8l+7 of the block (one 16-byte load of W per row, the fp64
// column scales of every basis held in registers for all rows), and wave w
// takes rows 16w..16w+15.  Each element is evaluated exactly as above.
// ---------------------------------------------------------------------------
constexpr int kDecompTileCols = 512;
constexpr int kDecompTileRows = 64;
constexpr int kDecompWaveRows = kDecompTileRows / 4;

// The 8 fp16 values of W at row i, columns j0..j0+7, as fp64.
__device__ __forceinline__ void load_w8(const uint16_t *w, int64_t k, int64_t i, int64_t j0, double (&wv)[8]) {
  const u32x4 q = *reinterpret_cast<const u32x4 *>(w + i * k + j0);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    wv[2 * t] = (double)h2f((uint16_t)(q[t] & 0xffffu));
    wv[2 * t + 1] = (double)h2f((uint16_t)(q[t] >> 16));
  }
}

// Sign bits of basis l, row i, columns j0..j0+7 (j0 a multiple of 8): one byte.
__device__ __forceinline__ uint32_t sign_byte(const uint32_t *bits, int64_t n, int64_t wpr, int l, int64_t i,
                                              int64_t j0) {
  return (bits[((int64_t)l * n + i) * wpr + (j0 >> 5)] >> (j0 & 31)) & 0xffu;
}

__device__ __forceinline__ double sgn_bit(uint32_t byte, int t) { return ((byte >> t) & 1u) ? 1.0 : -1.0; }

// Loads this lane's column scales (8 per basis; 0 past k).
template <int KB>
__device__ __forceinline__ void load_col_scales(const double *c, int64_t k, int64_t j0, bool live, double (&cl)[KB][8]) {
#pragma unroll
  for (int l = 0; l < KB; ++l)
#pragma unroll
    for (int t = 0; t < 8; ++t) cl[l][t] = live ? c[(int64_t)l * k + j0 + t] : 0.0;
}

// Row step, first pass: partial[cb][i] = sum over the 512 columns of block cb of d_j R_ij B_ij c_j.
// Each lane keeps one partial per row of its wave; the wave's 16 x 64 partials
// are then summed through LDS in a fixed order (lanes 4q..4q+3 each add 16
// lanes' values of row q in lane order, then the four sums pairwise).
template <int KB>
__global__ __launch_bounds__(256) void decomp_row_tiled_kernel(const uint16_t *__restrict__ w, int64_t n, int64_t k,
                                                               int basis, const uint32_t *__restrict__ bits,
                                                               const double *__restrict__ r,
                                                               const double *__restrict__ c,
                                                               const double *__restrict__ d,
                                                               double *__restrict__ partial) {
#pragma clang fp contract(off)
  __shared__ double red[4][kDecompWaveRows][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cb = blockIdx.x;
  const int64_t j0 = cb * kDecompTileCols + lane * 8;
  const bool live = j0 < k;
  const int64_t wpr = (k + 31) / 32;
  double cl[KB][8], dv[8];
  load_col_scales<KB>(c, k, j0, live, cl);
#pragma unroll
  for (int t = 0; t < 8; ++t) dv[t] = d && live ? d[j0 + t] : 1.0;
  const int64_t i0 = (int64_t)blockIdx.y * kDecompTileRows + wave * kDecompWaveRows;
#pragma unroll 4
  for (int row = 0; row < kDecompWaveRows; ++row) {
    const int64_t i = min(i0 + row, n - 1);  // rows past n repeat the last one; their sums are dropped
    double wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t sb[KB];
    double rs[KB];
#pragma unroll
    for (int l = 0; l < KB; ++l) {
      sb[l] = live ? sign_byte(bits, n, wpr, l, i, j0) : 0u;
      rs[l] = r[(int64_t)l * n + i];
    }
    if (live) load_w8(w, k, i, j0, wv);
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      double a = 0.0, sbb = 0.0, cbb = 0.0;
#pragma unroll
      for (int l = 0; l < KB; ++l) {
        if (l != basis) a += (rs[l] * sgn_bit(sb[l], t)) * cl[l][t];
        sbb = l == basis ? sgn_bit(sb[l], t) : sbb;
        cbb = l == basis ? cl[l][t] : cbb;
      }
      acc += ((dv[t] * (wv[t] - a)) * sbb) * cbb;
    }
    red[wave][row][lane] = acc;
  }
  __syncthreads();
  const int q = lane >> 2, part = lane & 3;
  double s = 0.0;
#pragma unroll
  for (int m = 0; m < 16; ++m) s += red[wave][q][part * 16 + m];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  const int64_t i = i0 + q;
  if (part == 0 && i < n) partial[cb * n + i] = s;
}

// Row step, second pass: r_out[i] = sum over column blocks (in order) / den.
__global__ __launch_bounds__(256) void decomp_row_finish_kernel(const double *partial, int64_t blocks, int64_t n,
                                                                const double *den, double *r_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double num = 0.0;
  for (int64_t q = 0; q < blocks; ++q) num += partial[q * n + i];
  r_out[i] = den[0] > 0.0 ? num / den[0] : 0.0;
}

// Column step, first pass: partial[q][j] = sum over the 64 rows of chunk q of R_ij B_ij r_i
// (the four waves' sums added in wave order).
template <int KB>
__global__ __launch_bounds__(256) void decomp_col_tiled_kernel(const uint16_t *__restrict__ w, int64_t n, int64_t k,
                                                               int basis, const uint32_t *__restrict__ bits,
                                                               const double *__restrict__ r,
                                                               const double *__restrict__ c,
                                                               double *__restrict__ partial) {
#pragma clang fp contract(off)
  static_assert(kDecompTileRows == kDecompRowChunk, "column partials are per 64-row chunk");
  __shared__ double red[4][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * kDecompTileCols + lane * 8;
  const bool live = j0 < k;
  const int64_t wpr = (k + 31) / 32;
  double cl[KB][8], num[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  load_col_scales<KB>(c, k, j0, live, cl);
  const int64_t i0 = (int64_t)blockIdx.y * kDecompTileRows + wave * kDecompWaveRows;
#pragma unroll 2
  for (int row = 0; row < kDecompWaveRows; ++row) {
    const int64_t i = min(i0 + row, n - 1);  // rows past n repeat the last one with a zero weight
    const double rowok = i0 + row < n ? 1.0 : 0.0;
    double wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t sb[KB];
    double rs[KB];
#pragma unroll
    for (int l = 0; l < KB; ++l) {
      sb[l] = live ? sign_byte(bits, n, wpr, l, i, j0) : 0u;
      rs[l] = r[(int64_t)l * n + i];
    }
    if (live) load_w8(w, k, i, j0, wv);
    double rb = 0.0;
#pragma unroll
    for (int l = 0; l < KB; ++l) rb = l == basis ? rs[l] * rowok : rb;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      double a = 0.0, sbb = 0.0;
#pragma unroll
      for (int l = 0; l < KB; ++l) {
        if (l != basis) a += (rs[l] * sgn_bit(sb[l], t)) * cl[l][t];
        sbb = l == basis ? sgn_bit(sb[l], t) : sbb;
      }
      num[t] += ((wv[t] - a) * sbb) * rb;
    }
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) red[wave][t][lane] = num[t];
  __syncthreads();
  if (wave == 0 && live) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      partial[(int64_t)blockIdx.y * k + j0 + t] = ((red[0][t][lane] + red[1][t][lane]) + red[2][t][lane]) + red[3][t][lane];
  }
}

// Sign step (all bases) or, with RESIDUAL, the initial signs of basis `basis`
// (+1 where W minus the other bases is >= 0).  Each lane writes one byte of
// sign bits per basis and row; bytes past k inside the last word are zero.
template <int KB, bool RESIDUAL>
__global__ __launch_bounds__(256) void decomp_sign_tiled_kernel(const uint16_t *__restrict__ w, int64_t n, int64_t k,
                                                                int basis, const uint32_t *__restrict__ bits,
                                                                const double *__restrict__ r,
                                                                const double *__restrict__ c,
                                                                uint32_t *__restrict__ bits_out) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = (int64_t)blockIdx.x * kDecompTileCols + lane * 8;
  const int64_t wpr = (k + 31) / 32;
  const bool live = j0 < k, pad = !live && j0 < wpr * 32;
  double cl[KB][8];
  load_col_scales<KB>(c, k, j0, live, cl);
  uint8_t *out8 = reinterpret_cast<uint8_t *>(bits_out);
  const int64_t i0 = (int64_t)blockIdx.y * kDecompTileRows + wave * kDecompWaveRows;
#pragma unroll 2
  for (int row = 0; row < kDecompWaveRows; ++row) {
    const int64_t i = min(i0 + row, n - 1);  // rows past n repeat the last one and store nothing
    const bool rowok = i0 + row < n;
    double wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    double rs[KB];
#pragma unroll
    for (int l = 0; l < KB; ++l) rs[l] = r[(int64_t)l * n + i];
    if (live) load_w8(w, k, i, j0, wv);
    if constexpr (RESIDUAL) {
      uint32_t sb[KB];
#pragma unroll
      for (int l = 0; l < KB; ++l) sb[l] = live && l != basis ? sign_byte(bits, n, wpr, l, i, j0) : 0u;
      uint32_t byte = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        double a = 0.0;
#pragma unroll
        for (int l = 0; l < KB; ++l)
          if (l != basis) a += (rs[l] * sgn_bit(sb[l], t)) * cl[l][t];
        byte |= (wv[t] - a >= 0.0 ? 1u : 0u) << t;
      }
      if (rowok && (live || pad)) out8[i * wpr * 4 + (j0 >> 3)] = (uint8_t)(live ? byte : 0u);
    } else {
      uint32_t byte[KB];
#pragma unroll
      for (int l = 0; l < KB; ++l) byte[l] = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        double p[KB];
#pragma unroll
        for (int l = 0; l < KB; ++l) p[l] = rs[l] * cl[l][t];
        double best = __builtin_inf();
        int best_m = 0;
#pragma unroll
        for (int m = 0; m < (1 << KB); ++m) {
          double sum = 0.0;
#pragma unroll
          for (int l = 0; l < KB; ++l) sum = ((m >> l) & 1) ? sum + p[l] : sum - p[l];
          const double e = fabs(wv[t] - sum);
          if (e < best) {
            best = e;
            best_m = m;
          }
        }
#pragma unroll
        for (int l = 0; l < KB; ++l) byte[l] |= (uint32_t)((best_m >> l) & 1) << t;
      }
      if (rowok && (live || pad)) {
#pragma unroll
        for (int l = 0; l < KB; ++l) out8[((int64_t)l * n + i) * wpr * 4 + (j0 >> 3)] = (uint8_t)(live ? byte[l] : 0u);
      }
    }
  }
}

// IEEE binary64 -> binary16, round to nearest even, from the formats'
// definitions (no detour through binary32, which could round twice).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int e = (int)((u >> 52) & 0x7ff);
  const uint64_t m = u & ((1ull << 52) - 1);
  if (e == 0x7ff) return sign | (m ? 0x7e00 : 0x7c00);
  if (e == 0) return sign;  // binary64 subnormals are far below half the smallest binary16 subnormal
  const int E = e - 1023;   // |v| in [2^E, 2^(E+1))
  if (E > 15) return sign | 0x7c00;
  const uint64_t sig = m | (1ull << 52);
  const int shift = E >= -14 ? 42 : 42 + (-14 - E);  // low bits dropped: keep 11 (normal) or fewer
  if (shift > 53) return sign;                        // below half the smallest subnormal
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (E >= -14) {
    int he = E + 15;
    if (q == 2048) {
      q = 1024;
      ++he;
    }
    if (he >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(he << 10) | (uint16_t)(q - 1024);
  }
  return sign | (uint16_t)q;  // subnormal (q = 1024 is the smallest normal)
}

// v16[t] = fp16(v[t]) (nearest even); vr[t] = the rounded value, exactly.
__global__ __launch_bounds__(256) void decomp_round_kernel(const double *v, int64_t len, uint16_t *v16, double *vr) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= len) return;
  const uint16_t h = f64_to_f16_rne(v[t]);
  v16[t] = h;
  vr[t] = (double)h2f(h);
}

__global__ __launch_bounds__(256) void decomp_fill_kernel(double *v, int64_t len, double value) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < len) v[t] = value;
}

__global__ __launch_bounds__(256) void decomp_zero_words_kernel(uint32_t *v, int64_t len) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < len) v[t] = 0u;
}

}  // namespace fluxbin
