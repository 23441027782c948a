/*
 * fluxbin_oracle.c -- plain, slow, fp64 CPU oracle for the FluxBin LUT GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and this file includes nothing from the GPU
 * library: every format below is re-derived here from its written definition.
 *
 * What is computed (FluxBin, paperlayer.ai summary, section 3 "Methodology",
 * bullets "Quantization", "Salient-Aware Hybrid Bases", "Virtual Columnar
 * Mapping"; same page, appendix C.1 "Compute Complexity Analysis"):
 *
 *   W_hat = sum_{k<Kb} diag(r_k) B_k diag(c_k)
 *         + sum_{s<Ks} diag(r_s) B_s diag(c_s) P_S          (P_S x = x[S])
 *   y[b]  = W_hat x[b]
 *
 * B are +-1 matrices stored as packed sign bits.  The salient bases act on
 * the salient columns only and are added on top of the global bases: a
 * second correction of the same columns, not a replacement of them.  The LUT form of the same
 * product (sub-vectors of g inputs, a table of all 2^g signed sums of the
 * scale-fused inputs, indexed by the weight bit pattern) reaches the same y
 * up to rounding order; orc_gemv_lut() evaluates it step by step in fp64 so
 * that the two routes can be compared.
 *
 * Readings taken where the pages are silent (each is documented in the
 * design notes of the repository):
 *   - bit value 1 means +1 and 0 means -1 (LUT Tensor Core page, section
 *     3.1.2: binary digits reinterpreted as {-1,+1});
 *   - bits are packed along the input dimension, least significant bit first:
 *     word w of a row holds column 32w+t at bit t; padding bits are 0;
 *   - the row scale is one fp16 value per output row per basis, or, in the
 *     block-wise format, one per output row per basis per group of
 *     `row_group` input columns (FluxBin summary, appendix C.2: the global
 *     part keeps block-wise row scales; a salient column takes the scale of
 *     the group its original column falls in);
 *   - the salient column scale c_s is stored in compact (VCM) order;
 *   - fp16 inputs, fp64 arithmetic, results returned in fp64.
 *
 * Parity status: the dense product is pinned by closed forms (popcount
 * identity, one-hot column selection, the LUT Tensor Core page's 1x4 times
 * 4xN worked shape with dyadic inputs), exact integer brute force on tiny
 * problems, and agreement with the separately written LUT route.  The
 * block-wise row scales are pinned by reduction to the per-row product (all
 * group scales of a row equal; a single non-zero group on activations
 * zeroed outside it) and by exact integer brute force.  The offline
 * decomposition's steps are pinned by the properties the pages assign them:
 * each scale step lands on the vertex of its least-squares quadratic, the
 * sign step is the exhaustive per-element optimum, the error never rises
 * over the steps, and a matrix that is one scaled binary basis is recovered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary64, written from the format definition.     */
/* ---------------------------------------------------------------------- */

ORC_EXPORT double orc_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* zero or subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* Round to nearest, ties to even (the default rounding mode of rint()). */
ORC_EXPORT uint16_t orc_double_to_half(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7e00;
  if (a >= 65520.0) return sign | 0x7c00; /* halfway above 65504 rounds to inf */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: quantum 2^-24; rounding may reach 1024 = min normal */
    double q = rint(ldexp(a, 24));
    return sign | (uint16_t)q;
  }
  int E;
  frexp(a, &E);                   /* a in [2^(E-1), 2^E) */
  int e = E - 1;                  /* unbiased exponent */
  double q = rint(ldexp(a, 10 - e)); /* significand in units of 2^(e-10) */
  if (q == 2048.0) {
    q = 1024.0;
    e += 1;
  }
  return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

ORC_EXPORT void orc_half_array_to_double(const uint16_t *h, int64_t count, double *out) {
  for (int64_t i = 0; i < count; ++i) out[i] = orc_half_to_double(h[i]);
}

ORC_EXPORT void orc_double_array_to_half(const double *v, int64_t count, uint16_t *out) {
  for (int64_t i = 0; i < count; ++i) out[i] = orc_double_to_half(v[i]);
}

/* ---------------------------------------------------------------------- */
/* Sign bits                                                                */
/* ---------------------------------------------------------------------- */

static inline int64_t words_per_row(int64_t cols) { return (cols + 31) / 32; }

/* Sign of column `col` of a canonical row: +1 when the bit is set, else -1. */
static inline double sign_at(const uint32_t *row_words, int64_t col) {
  uint32_t w = row_words[col >> 5];
  return ((w >> (col & 31)) & 1u) ? 1.0 : -1.0;
}

/* Pack int8 signs [rows][ld] (first `cols` used) into canonical words
 * [rows][ceil(cols/32)].  +1 sets the bit, -1 clears it; any other value is
 * counted as invalid and stored as a cleared bit.  Returns the invalid count. */
ORC_EXPORT int64_t orc_pack_rowmajor(const int8_t *signs, int64_t rows, int64_t cols, int64_t ld,
                                     uint32_t *out) {
  int64_t wpr = words_per_row(cols);
  int64_t bad = 0;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t w = 0; w < wpr; ++w) {
      uint32_t word = 0;
      for (int t = 0; t < 32; ++t) {
        int64_t col = 32 * w + t;
        if (col >= cols) break;
        int8_t s = signs[r * ld + col];
        if (s == 1) {
          word |= (1u << t);
        } else if (s != -1) {
          ++bad;
        }
      }
      out[r * wpr + w] = word;
    }
  }
  return bad;
}

/* Inverse of orc_pack_rowmajor for valid words: +1 / -1 as int8. */
ORC_EXPORT void orc_unpack_rowmajor(const uint32_t *words, int64_t rows, int64_t cols, int8_t *signs) {
  int64_t wpr = words_per_row(cols);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t col = 0; col < cols; ++col)
      signs[r * cols + col] = (int8_t)sign_at(words + r * wpr, col);
}

/* Tiled device layout.  Rows are padded to a multiple of 64 and columns to a
 * multiple of 128 (4 words).  The word holding canonical (row r, word w) is
 * stored at index ((floor(r/64) * NC + floor(w/4)) * 64 + r mod 64) * 4 + w mod 4,
 * NC = ceil(cols/128).  Padding words are zero.  The bits inside a word are
 * not permuted. */
ORC_EXPORT int64_t orc_tiled_words(int64_t rows, int64_t cols) {
  int64_t rt = (rows + 63) / 64;
  int64_t nc = (cols + 127) / 128;
  return rt * nc * 64 * 4;
}

ORC_EXPORT void orc_tile_words(const uint32_t *canon, int64_t rows, int64_t cols, uint32_t *tiled) {
  int64_t wpr = words_per_row(cols);
  int64_t nc = (cols + 127) / 128;
  memset(tiled, 0, (size_t)orc_tiled_words(rows, cols) * sizeof(uint32_t));
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t w = 0; w < wpr; ++w) {
      int64_t dst = (((r / 64) * nc + w / 4) * 64 + (r % 64)) * 4 + (w % 4);
      tiled[dst] = canon[r * wpr + w];
    }
  }
}

/* Tiled row-scale layout of the block-wise format: a [rows][groups] fp16
 * matrix whose groups fall `m` to a 128-column chunk.  Rows are padded to a
 * multiple of 64 and groups to a multiple of m; element (row r, group q) is
 * stored at ((floor(r/64) * NC + floor(q/m)) * 64 + r mod 64) * m + q mod m,
 * NC = ceil(groups/m), so that a row's scales for one chunk are contiguous
 * and a 64-row tile's scales for one chunk form one block.  Padding is 0. */
ORC_EXPORT int64_t orc_tiled_scale_elems(int64_t rows, int64_t groups, int64_t m) {
  return ((rows + 63) / 64) * ((groups + m - 1) / m) * 64 * m;
}

ORC_EXPORT void orc_tile_scales(const uint16_t *canon, int64_t rows, int64_t groups, int64_t m, uint16_t *tiled) {
  int64_t nc = (groups + m - 1) / m;
  memset(tiled, 0, (size_t)orc_tiled_scale_elems(rows, groups, m) * sizeof(uint16_t));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t q = 0; q < groups; ++q)
      tiled[(((r / 64) * nc + q / m) * 64 + (r % 64)) * m + (q % m)] = canon[r * groups + q];
}

/* VCM on sign bits: compact column c of the destination is source column
 * idx[c].  src canonical [rows][ceil(k/32)], dst canonical [rows][ceil(s/32)]. */
ORC_EXPORT void orc_vcm_gather_bits(const uint32_t *src, int64_t rows, int64_t k, const int32_t *idx,
                                    int64_t s, uint32_t *dst) {
  int64_t wk = words_per_row(k), ws = words_per_row(s);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t w = 0; w < ws; ++w) dst[r * ws + w] = 0;
    for (int64_t c = 0; c < s; ++c) {
      if (sign_at(src + r * wk, idx[c]) > 0) dst[r * ws + c / 32] |= (1u << (c % 32));
    }
  }
}

/* ---------------------------------------------------------------------- */
/* Dense reconstruction and product                                         */
/* ---------------------------------------------------------------------- */

typedef struct {
  int64_t n, k, s;
  int32_t kb, ks;
  int64_t row_group;      /* 0: one row scale per row; else columns per row-scale group */
  int64_t ngroups;        /* row scales per row per basis: 1, or ceil(k / row_group) */
  const uint32_t *bits_g; /* [kb][n][ceil(k/32)] */
  const uint16_t *r_g;    /* [kb][n][ngroups] */
  const uint16_t *c_g;    /* [kb][k] */
  const uint32_t *bits_s; /* [ks][n][ceil(s/32)] */
  const uint16_t *r_s;    /* [ks][n][ngroups] */
  const uint16_t *c_s;    /* [ks][s], compact order */
  const int32_t *idx;     /* [s], salient column of compact column c */
} orc_layer;

/* Row-scale group of input column j (0 when there is one scale per row). */
static inline int64_t group_of(int64_t row_group, int64_t j) { return row_group ? j / row_group : 0; }

static inline int64_t group_count(int64_t row_group, int64_t k) {
  return row_group ? (k + row_group - 1) / row_group : 1;
}

static double *halves(const uint16_t *h, int64_t count) {
  double *d = (double *)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
  orc_half_array_to_double(h, count, d);
  return d;
}

/* Row i of W_hat in fp64, written out from its definition. */
static void reconstruct_row(const orc_layer *L, const double *cg, const double *cs, int64_t i,
                            double *wrow) {
  int64_t wk = words_per_row(L->k), ws = words_per_row(L->s);
  for (int64_t j = 0; j < L->k; ++j) wrow[j] = 0.0;
  for (int32_t b = 0; b < L->kb; ++b) {
    const uint32_t *row = L->bits_g + ((int64_t)b * L->n + i) * wk;
    const uint16_t *rrow = L->r_g + ((int64_t)b * L->n + i) * L->ngroups;
    for (int64_t j = 0; j < L->k; ++j) {
      double r = orc_half_to_double(rrow[group_of(L->row_group, j)]);
      wrow[j] += r * sign_at(row, j) * cg[(int64_t)b * L->k + j];
    }
  }
  for (int32_t b = 0; b < L->ks; ++b) {
    const uint32_t *row = L->bits_s + ((int64_t)b * L->n + i) * ws;
    const uint16_t *rrow = L->r_s + ((int64_t)b * L->n + i) * L->ngroups;
    for (int64_t c = 0; c < L->s; ++c) {
      double r = orc_half_to_double(rrow[group_of(L->row_group, L->idx[c])]);
      wrow[L->idx[c]] += r * sign_at(row, c) * cs[(int64_t)b * L->s + c];
    }
  }
}

/* y[b][t] = sum_j W_hat[rows[t]][j] * x[b][j] and mag[b][t] = sum_j |W_hat x|
 * for each listed row t (all n rows when rows == NULL; then nrows must be n).
 * y and mag are [batch][nrows].  nthreads <= 0 uses the OpenMP default.
 * row_group = 0: r_g [kb][n], r_s [ks][n]; row_group > 0: r_g [kb][n][G],
 * r_s [ks][n][G] with G = ceil(k / row_group), and the salient scale of
 * compact column c is that of group floor(idx[c] / row_group).
 * Returns 1 for a row index out of range, 2 for a negative row_group. */
ORC_EXPORT int orc_gemv_dense(int64_t n, int64_t k, int64_t s, int32_t kb, int32_t ks, int64_t row_group,
                              const uint32_t *bits_g, const uint16_t *r_g, const uint16_t *c_g,
                              const uint32_t *bits_s, const uint16_t *r_s, const uint16_t *c_s,
                              const int32_t *idx, const uint16_t *x, int64_t batch,
                              const int64_t *rows, int64_t nrows, double *y, double *mag,
                              int32_t nthreads) {
  if (row_group < 0) return 2;
  orc_layer L = {n, k, s, kb, ks, row_group, group_count(row_group, k), bits_g, r_g, c_g, bits_s, r_s, c_s, idx};
  double *cg = halves(c_g, (int64_t)kb * k);
  double *cs = halves(c_s, (int64_t)ks * s);
  double *xd = halves(x, batch * k);
  int err = 0;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    double *wrow = (double *)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
    for (int64_t t = 0; t < nrows; ++t) {
      int64_t i = rows ? rows[t] : t;
      if (i < 0 || i >= n) {
        err = 1;
        continue;
      }
      reconstruct_row(&L, cg, cs, i, wrow);
      for (int64_t b = 0; b < batch; ++b) {
        double acc = 0.0, am = 0.0;
        const double *xb = xd + b * k;
        for (int64_t j = 0; j < k; ++j) {
          double p = wrow[j] * xb[j];
          acc += p;
          am += fabs(p);
        }
        y[b * nrows + t] = acc;
        if (mag) mag[b * nrows + t] = am;
      }
    }
    free(wrow);
  }
  free(cg);
  free(cs);
  free(xd);
  return err;
}

/* ---------------------------------------------------------------------- */
/* LUT route, step by step (scale-fused table, pattern lookup, row scale)   */
/* ---------------------------------------------------------------------- */

/* Full table of one sub-vector: LUT[p] = sum_t (2*bit_t(p) - 1) * v_t for all
 * p < 2^g, each entry enumerated directly (LUT Tensor Core page, section 2.2
 * Figure 3: one entry per sign pattern of a g-element activation group). */
ORC_EXPORT void orc_lut_explicit(int32_t g, const double *v, double *lut) {
  for (int64_t p = 0; p < ((int64_t)1 << g); ++p) {
    double acc = 0.0;
    for (int32_t t = 0; t < g; ++t) acc += (((p >> t) & 1) ? 1.0 : -1.0) * v[t];
    lut[p] = acc;
  }
}

/* Scale-fused inputs of sub-vector j of one segment: v_t = c[jg+t] * x[jg+t]
 * (global) or c[jg+t] * x[idx[jg+t]] (salient, VCM gather); zero past L. */
static void fused_inputs(int32_t g, int64_t j, int64_t len, const double *c, const double *xb,
                         const int32_t *gather, double *v) {
  for (int32_t t = 0; t < g; ++t) {
    int64_t col = j * g + t;
    if (col >= len) {
      v[t] = 0.0;
    } else {
      double xv = gather ? xb[gather[col]] : xb[col];
      v[t] = c[col] * xv;
    }
  }
}

/* Sign pattern of sub-vector j of a canonical row (g divides 32). */
static inline uint32_t pattern_at(const uint32_t *row_words, int32_t g, int64_t j) {
  int64_t bit = j * g;
  return (row_words[bit >> 5] >> (bit & 31)) & ((1u << g) - 1u);
}

/* y via the LUT route in fp64: per segment and batch row, build every
 * sub-vector's 2^g table from the scale-fused inputs, look each row's bit
 * pattern up and accumulate per row-scale group, then apply each group's row
 * scale to its partial sum and add the groups (with row_group = 0 there is
 * one group: the row scale is applied once, after accumulation).
 * y is [batch][nrows] like orc_gemv_dense, scales laid out as there.
 * Returns 1 for an unsupported g, 2 when a sub-vector's columns fall in two
 * row-scale groups (the block-wise format then has no per-group sum). */
/* Quantised tables (LUT Tensor Core notes, section 3.1.3: the precomputed
 * table entries stored in a lower, uniform precision).  table_fmt 0: exact
 * fp64 entries (the plain LUT route).  table_fmt 1: fp16 entries taken in
 * the precision the GPU kernel takes them -- the half-table entry
 * v_{g-1} + sum_{t<g-1} (+-v_t) summed in fp32 in that order (each v_t =
 * c_t x_t is exact in fp32), rounded to fp16 (nearest even); the other half
 * is its negation.  Returns 0 and writes lut (2^g entries).
 * table_fmt 1 mirrors the kernel's entry arithmetic on purpose, so it is a
 * diagnostic (it localises a failure to the table build or to the
 * accumulation), not a reference: the fp16-table contract is the bound
 * against the exact product (format 0 / orc_gemv_dense). */
static void quantised_table(int32_t g, const double *v, int32_t table_fmt, double *lut) {
  int64_t tsize = (int64_t)1 << g, half = tsize / 2;
  if (table_fmt == 0) {
    orc_lut_explicit(g, v, lut);
    return;
  }
  for (int64_t q = 0; q < half; ++q) {
    float t = (float)v[g - 1];
    for (int32_t i = 0; i < g - 1; ++i) {
      float vi = (float)v[i];
      t = ((q >> i) & 1) ? t + vi : t - vi;
    }
    double h = orc_half_to_double(orc_double_to_half((double)t));
    lut[q | half] = h;
    lut[(half - 1) ^ q] = -h;
  }
}

ORC_EXPORT int orc_gemv_lut_tables(int64_t n, int64_t k, int64_t s, int32_t kb, int32_t ks, int64_t row_group,
                                   int32_t g, int32_t table_fmt, const uint32_t *bits_g, const uint16_t *r_g,
                                   const uint16_t *c_g, const uint32_t *bits_s, const uint16_t *r_s,
                                   const uint16_t *c_s, const int32_t *idx, const uint16_t *x, int64_t batch,
                                   const int64_t *rows, int64_t nrows, double *y);

/* The full 2^g table of one sub-vector in format table_fmt (exported for the pins). */
ORC_EXPORT void orc_quantised_table(int32_t g, const double *v, int32_t table_fmt, double *lut) {
  quantised_table(g, v, table_fmt, lut);
}

ORC_EXPORT int orc_gemv_lut(int64_t n, int64_t k, int64_t s, int32_t kb, int32_t ks, int64_t row_group, int32_t g,
                            const uint32_t *bits_g, const uint16_t *r_g, const uint16_t *c_g,
                            const uint32_t *bits_s, const uint16_t *r_s, const uint16_t *c_s,
                            const int32_t *idx, const uint16_t *x, int64_t batch,
                            const int64_t *rows, int64_t nrows, double *y) {
  return orc_gemv_lut_tables(n, k, s, kb, ks, row_group, g, 0, bits_g, r_g, c_g, bits_s, r_s, c_s, idx, x, batch,
                             rows, nrows, y);
}

/* The LUT route with tables in format table_fmt (see quantised_table); y as
 * orc_gemv_lut.  Returns 1 for an unsupported g or format. */
ORC_EXPORT int orc_gemv_lut_tables(int64_t n, int64_t k, int64_t s, int32_t kb, int32_t ks, int64_t row_group,
                                   int32_t g, int32_t table_fmt, const uint32_t *bits_g, const uint16_t *r_g,
                                   const uint16_t *c_g, const uint32_t *bits_s, const uint16_t *r_s,
                                   const uint16_t *c_s, const int32_t *idx, const uint16_t *x, int64_t batch,
                                   const int64_t *rows, int64_t nrows, double *y) {
  if (g <= 0 || g > 16 || 32 % g) return 1;
  if (table_fmt != 0 && table_fmt != 1) return 1;
  if (row_group < 0) return 2;
  const int64_t ng = group_count(row_group, k);
  int err = 0;
  double *cg = halves(c_g, (int64_t)kb * k);
  double *cs = halves(c_s, (int64_t)ks * s);
  double *xd = halves(x, batch * k);
  int64_t tsize = (int64_t)1 << g;
  double v[16];
  double *partial = (double *)malloc((size_t)ng * sizeof(double));
  for (int64_t i = 0; i < batch * nrows; ++i) y[i] = 0.0;
  for (int32_t seg = 0; seg < kb + ks && !err; ++seg) {
    int salient = seg >= kb;
    int32_t sb = salient ? seg - kb : seg;
    int64_t len = salient ? s : k;
    int64_t nsub = (len + g - 1) / g;
    int64_t wpr = words_per_row(len);
    const double *c = salient ? cs + (int64_t)sb * s : cg + (int64_t)sb * k;
    const uint32_t *bits = salient ? bits_s + (int64_t)sb * n * wpr : bits_g + (int64_t)sb * n * wpr;
    const uint16_t *r = salient ? r_s + (int64_t)sb * n * ng : r_g + (int64_t)sb * n * ng;
    /* row-scale group of every sub-vector: that of its columns' original positions */
    int64_t *sub_group = (int64_t *)malloc((size_t)(nsub > 0 ? nsub : 1) * sizeof(int64_t));
    for (int64_t j = 0; j < nsub; ++j) {
      for (int32_t t = 0; t < g; ++t) {
        int64_t col = j * g + t;
        if (col >= len) break;
        int64_t grp = group_of(row_group, salient ? idx[col] : col);
        if (t == 0) sub_group[j] = grp;
        else if (grp != sub_group[j]) err = 2;
      }
    }
    double *tables = (double *)malloc((size_t)(nsub > 0 ? nsub : 1) * tsize * sizeof(double));
    for (int64_t b = 0; b < batch && !err; ++b) {
      const double *xb = xd + b * k;
      for (int64_t j = 0; j < nsub; ++j) {
        fused_inputs(g, j, len, c, xb, salient ? idx : NULL, v);
        quantised_table(g, v, table_fmt, tables + j * tsize);
      }
      for (int64_t t = 0; t < nrows; ++t) {
        int64_t i = rows ? rows[t] : t;
        const uint32_t *row = bits + i * wpr;
        for (int64_t q = 0; q < ng; ++q) partial[q] = 0.0;
        for (int64_t j = 0; j < nsub; ++j) partial[sub_group[j]] += tables[j * tsize + pattern_at(row, g, j)];
        double a = 0.0;
        for (int64_t q = 0; q < ng; ++q) a += orc_half_to_double(r[i * ng + q]) * partial[q];
        y[b * nrows + t] += a;
      }
    }
    free(tables);
    free(sub_group);
  }
  free(partial);
  free(cg);
  free(cs);
  free(xd);
  return err;
}

/* Half tables as exported by the GPU library's table builder:
 * out[b][seg][j][q] = LUT[q | 2^(g-1)] of sub-vector j (the half whose top
 * input carries sign +1; the other half follows from LUT[~p] = -LUT[p],
 * LUT Tensor Core page, section 3.1.2).  Segments are the kb global bases
 * then the ks salient bases; sub-vector counts are ceil(len/g).
 * absv[b][seg][j] = sum_t |v_t| (scale of the rounding bound). */
ORC_EXPORT int orc_half_luts(int64_t k, int64_t s, int32_t kb, int32_t ks, int32_t g,
                             const uint16_t *c_g, const uint16_t *c_s, const int32_t *idx,
                             const uint16_t *x, int64_t batch, double *out, double *absv) {
  if (g <= 0 || g > 16 || 32 % g) return 1;
  double *cg = halves(c_g, (int64_t)kb * k);
  double *cs = halves(c_s, (int64_t)ks * s);
  double *xd = halves(x, batch * k);
  int64_t tsize = (int64_t)1 << g, half = tsize / 2;
  double v[16];
  double *full = (double *)malloc((size_t)tsize * sizeof(double));
  int64_t o = 0, oa = 0;
  for (int64_t b = 0; b < batch; ++b) {
    for (int32_t seg = 0; seg < kb + ks; ++seg) {
      int salient = seg >= kb;
      int32_t sb = salient ? seg - kb : seg;
      int64_t len = salient ? s : k;
      int64_t nsub = (len + g - 1) / g;
      const double *c = salient ? cs + (int64_t)sb * s : cg + (int64_t)sb * k;
      for (int64_t j = 0; j < nsub; ++j) {
        fused_inputs(g, j, len, c, xd + b * k, salient ? idx : NULL, v);
        orc_lut_explicit(g, v, full);
        for (int64_t q = 0; q < half; ++q) out[o++] = full[q | half];
        double a = 0.0;
        for (int32_t t = 0; t < g; ++t) a += fabs(v[t]);
        absv[oa++] = a;
      }
    }
  }
  free(full);
  free(cg);
  free(cs);
  free(xd);
  return 0;
}

/* Dense fp16 matrix-vector product in fp64 (context kernel's reference):
 * y[b][i] = sum_j w[i][j] * x[b][j], w fp16 [n][k] row-major, x fp16 [batch][k]. */
ORC_EXPORT void orc_dense_f16_gemv(const uint16_t *w, int64_t n, int64_t k, const uint16_t *x,
                                   int64_t batch, double *y, double *mag) {
  double *xd = halves(x, batch * k);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t b = 0; b < batch; ++b) {
      double acc = 0.0, am = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        double p = orc_half_to_double(w[i * k + j]) * xd[b * k + j];
        acc += p;
        am += fabs(p);
      }
      y[b * n + i] = acc;
      if (mag) mag[b * n + i] = am;
    }
  }
  free(xd);
}

/* ---------------------------------------------------------------------- */
/* Offline decomposition W ~ sum_b diag(r_b) B_b diag(c_b)                  */
/* ---------------------------------------------------------------------- */
/* FluxBin summary, section 3 bullets "Quantization" (decoupled row-column
 * binary bases summed over decomposition orders) and "Parameter
 * Optimization" (alternating minimisation with weighted least squares; all
 * 2^Kb sign combinations evaluated jointly), appendix A.1 (with the binary
 * basis and the column scales fixed, each row scale is an independent scalar
 * least-squares problem with a closed form) and A.2 (with the scales fixed,
 * the error separates into independent per-element problems; exhaustive
 * search over the Kb signs of one element is globally optimal).
 *
 * Objective: E = sum_ij d_j (W_ij - W_hat_ij)^2, d_j > 0 per-column weights
 * (NULL: all 1).  Layouts: W fp16 [n][k]; bits canonical words
 * [kb][n][ceil(k/32)]; r fp64 [kb][n]; c fp64 [kb][k].  Readings where the
 * pages are silent (each is listed in the design notes):
 *   - the residual of basis b is R = W - sum_{l != b} diag(r_l) B_l diag(c_l);
 *   - row step:    r_b,i = sum_j d_j R_ij B_b,ij c_b,j / sum_j d_j c_b,j^2;
 *   - column step: c_b,j = sum_i R_ij B_b,ij r_b,i / sum_i r_b,i^2 (the
 *     weight d_j cancels); a zero denominator gives a zero scale;
 *   - sign step: for every element the combination m in [0, 2^kb) (bit b of
 *     m set = sign +1 on basis b) minimising |W_ij - s_m|, with
 *     s_m = sum_b (+-) r_b,i c_b,j accumulated in basis order from 0, each
 *     product rounded to fp64 once; ties go to the smallest m;
 *   - initialisation: bases in order; basis b takes the signs of the
 *     residual of the bases before it (R >= 0 gives +1), c_b = 1, then one row
 *     step and one column step;
 *   - one iteration: row then column step of every basis in order, then the
 *     sign step;
 *   - output: scales rounded to fp16 (nearest even), then one more sign step
 *     against the rounded scales. */

/* sum over bases l != skip of r_l,i B_l,ij c_l,j (skip = -1: every basis). */
static double approx_at(int64_t n, int64_t k, int32_t kb, const uint32_t *bits, const double *r, const double *c,
                        int64_t i, int64_t j, int32_t skip) {
  int64_t wpr = words_per_row(k);
  double a = 0.0;
  for (int32_t b = 0; b < kb; ++b) {
    if (b == skip) continue;
    a += r[(int64_t)b * n + i] * sign_at(bits + ((int64_t)b * n + i) * wpr, j) * c[(int64_t)b * k + j];
  }
  return a;
}

/* Row step of basis `basis`: r_out[i] for every row (other bases as given). */
ORC_EXPORT void orc_decomp_row_scales(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                      const uint32_t *bits, const double *r, const double *c, const double *d,
                                      double *r_out) {
  int64_t wpr = words_per_row(k);
  const double *cb = c + (int64_t)basis * k;
  double den = 0.0;
  for (int64_t j = 0; j < k; ++j) den += (d ? d[j] : 1.0) * cb[j] * cb[j];
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t *row = bits + ((int64_t)basis * n + i) * wpr;
    double num = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      double res = orc_half_to_double(w[i * k + j]) - approx_at(n, k, kb, bits, r, c, i, j, basis);
      num += (d ? d[j] : 1.0) * res * sign_at(row, j) * cb[j];
    }
    r_out[i] = den > 0.0 ? num / den : 0.0;
  }
}

/* Column step of basis `basis`: c_out[j] for every column. */
ORC_EXPORT void orc_decomp_col_scales(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                      const uint32_t *bits, const double *r, const double *c, double *c_out) {
  int64_t wpr = words_per_row(k);
  const double *rb = r + (int64_t)basis * n;
  double den = 0.0;
  for (int64_t i = 0; i < n; ++i) den += rb[i] * rb[i];
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t j = 0; j < k; ++j) {
    double num = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      const uint32_t *row = bits + ((int64_t)basis * n + i) * wpr;
      double res = orc_half_to_double(w[i * k + j]) - approx_at(n, k, kb, bits, r, c, i, j, basis);
      num += res * sign_at(row, j) * rb[i];
    }
    c_out[j] = den > 0.0 ? num / den : 0.0;
  }
}

/* Sign step: joint exhaustive search of every element; writes all kb bases. */
ORC_EXPORT void orc_decomp_signs(const uint16_t *w, int64_t n, int64_t k, int32_t kb, const double *r,
                                 const double *c, uint32_t *bits_out) {
  int64_t wpr = words_per_row(k);
  for (int64_t t = 0; t < (int64_t)kb * n * wpr; ++t) bits_out[t] = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t j = 0; j < k; ++j) {
      double wv = orc_half_to_double(w[i * k + j]);
      double best = INFINITY;
      int32_t best_m = 0;
      for (int32_t m = 0; m < (1 << kb); ++m) {
        double sum = 0.0;
        for (int32_t b = 0; b < kb; ++b) {
          double p = r[(int64_t)b * n + i] * c[(int64_t)b * k + j];
          sum = ((m >> b) & 1) ? sum + p : sum - p;
        }
        double e = fabs(wv - sum);
        if (e < best) {
          best = e;
          best_m = m;
        }
      }
      for (int32_t b = 0; b < kb; ++b)
        if ((best_m >> b) & 1) bits_out[((int64_t)b * n + i) * wpr + j / 32] |= 1u << (j % 32);
    }
  }
}

/* Initial signs of basis `basis`: +1 where the residual of the other bases is >= 0. */
ORC_EXPORT void orc_decomp_residual_signs(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                          const uint32_t *bits, const double *r, const double *c,
                                          uint32_t *basis_bits_out) {
  int64_t wpr = words_per_row(k);
  for (int64_t t = 0; t < n * wpr; ++t) basis_bits_out[t] = 0;
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      double res = orc_half_to_double(w[i * k + j]) - approx_at(n, k, kb, bits, r, c, i, j, basis);
      if (res >= 0.0) basis_bits_out[i * wpr + j / 32] |= 1u << (j % 32);
    }
}

/* E = sum_ij d_j (W_ij - W_hat_ij)^2. */
ORC_EXPORT double orc_decomp_error(const uint16_t *w, int64_t n, int64_t k, int32_t kb, const uint32_t *bits,
                                   const double *r, const double *c, const double *d) {
  double e = 0.0;
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < k; ++j) {
      double res = orc_half_to_double(w[i * k + j]) - approx_at(n, k, kb, bits, r, c, i, j, -1);
      e += (d ? d[j] : 1.0) * res * res;
    }
  return e;
}

/* The whole decomposition.  bits [kb][n][ceil(k/32)]; r16 [kb][n], c16 [kb][k]
 * fp16; r64, c64 (may be NULL) receive the fp64 scales before rounding.
 * trace (may be NULL) receives 2 + iters * (2 kb + 1) errors: after the
 * initialisation, after every row, column and sign step of every iteration,
 * and after the output rounding and its sign step. */
ORC_EXPORT int orc_decompose(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t iters, const double *d,
                             uint32_t *bits, uint16_t *r16, uint16_t *c16, double *r64, double *c64,
                             double *trace) {
  if (kb < 1 || kb > 4 || n < 1 || k < 1 || iters < 0) return 1;
  int64_t wpr = words_per_row(k);
  double *r = (double *)calloc((size_t)kb * n, sizeof(double));
  double *c = (double *)calloc((size_t)kb * k, sizeof(double));
  double *tmp = (double *)malloc((size_t)(n > k ? n : k) * sizeof(double));
  int64_t tr = 0;
  for (int64_t t = 0; t < (int64_t)kb * n * wpr; ++t) bits[t] = 0;
  for (int32_t b = 0; b < kb; ++b) {
    for (int64_t j = 0; j < k; ++j) c[(int64_t)b * k + j] = 1.0;
    orc_decomp_residual_signs(w, n, k, kb, b, bits, r, c, bits + (int64_t)b * n * wpr);
    orc_decomp_row_scales(w, n, k, kb, b, bits, r, c, d, tmp);
    memcpy(r + (int64_t)b * n, tmp, (size_t)n * sizeof(double));
    orc_decomp_col_scales(w, n, k, kb, b, bits, r, c, tmp);
    memcpy(c + (int64_t)b * k, tmp, (size_t)k * sizeof(double));
  }
  if (trace) trace[tr++] = orc_decomp_error(w, n, k, kb, bits, r, c, d);
  for (int32_t it = 0; it < iters; ++it) {
    for (int32_t b = 0; b < kb; ++b) {
      orc_decomp_row_scales(w, n, k, kb, b, bits, r, c, d, tmp);
      memcpy(r + (int64_t)b * n, tmp, (size_t)n * sizeof(double));
      if (trace) trace[tr++] = orc_decomp_error(w, n, k, kb, bits, r, c, d);
      orc_decomp_col_scales(w, n, k, kb, b, bits, r, c, tmp);
      memcpy(c + (int64_t)b * k, tmp, (size_t)k * sizeof(double));
      if (trace) trace[tr++] = orc_decomp_error(w, n, k, kb, bits, r, c, d);
    }
    orc_decomp_signs(w, n, k, kb, r, c, bits);
    if (trace) trace[tr++] = orc_decomp_error(w, n, k, kb, bits, r, c, d);
  }
  if (r64) memcpy(r64, r, (size_t)kb * n * sizeof(double));
  if (c64) memcpy(c64, c, (size_t)kb * k * sizeof(double));
  for (int64_t t = 0; t < (int64_t)kb * n; ++t) {
    r16[t] = orc_double_to_half(r[t]);
    r[t] = orc_half_to_double(r16[t]);
  }
  for (int64_t t = 0; t < (int64_t)kb * k; ++t) {
    c16[t] = orc_double_to_half(c[t]);
    c[t] = orc_half_to_double(c16[t]);
  }
  orc_decomp_signs(w, n, k, kb, r, c, bits);
  if (trace) trace[tr++] = orc_decomp_error(w, n, k, kb, bits, r, c, d);
  free(r);
  free(c);
  free(tmp);
  return 0;
}

ORC_EXPORT int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
