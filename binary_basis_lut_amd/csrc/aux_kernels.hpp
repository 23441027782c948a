// aux_kernels.hpp -- the kernels around the GEMV: table export, sign-word
// packing and relayout, VCM gather, and the dense fp16 context GEMV.
#pragma once

#include "common.hpp"

namespace fluxbin {

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

// Block-wise row scales, [rows][groups] fp16 <-> the tiled scale layout
// (m = groups per 128-column chunk): one thread per destination element.
__global__ __launch_bounds__(256) void relayout_scales_kernel(const uint16_t *src, int64_t rows, int64_t groups,
                                                              int64_t m, int32_t src_layout, int32_t dst_layout,
                                                              uint16_t *dst, int64_t total) {
  const int64_t nc = (groups + m - 1) / m;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    int64_t r, q;
    if (dst_layout == 0) {
      r = o / groups;
      q = o - r * groups;
    } else {
      const int64_t qm = o % m, lane = (o / m) % 64, tc = o / (m * 64);  // tc = tile * nc + chunk
      r = (tc / nc) * 64 + lane;
      q = (tc % nc) * m + qm;
    }
    uint16_t v = 0;
    if (r < rows && q < groups) {
      const int64_t si = src_layout == 0 ? r * groups + q : (((r / 64) * nc + q / m) * 64 + (r % 64)) * m + (q % m);
      v = src[si];
    }
    dst[o] = v;
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

// --------------------------------------------------------------------------
// Workspace reset: zero `words` 64-bit words (a kernel, not a memset, so that
// the call can be captured in a graph)
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_words_kernel(uint64_t *w, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    w[i] = 0;
}

}  // namespace fluxbin
