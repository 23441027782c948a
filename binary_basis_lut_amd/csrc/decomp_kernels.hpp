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

// out[0] = sum_t w_t * v_t^2 over t < len (w = NULL: 1), one workgroup of 256 threads.
__global__ __launch_bounds__(256) void decomp_sumsq_kernel(const double *v, const double *w, int64_t len,
                                                           double *out) {
  __shared__ double part[4];
  double a = 0.0;
  for (int64_t t = threadIdx.x; t < len; t += 256) a += (w ? w[t] : 1.0) * v[t] * v[t];
  a = wave_sum(a);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = ((part[0] + part[1]) + part[2]) + part[3];
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
