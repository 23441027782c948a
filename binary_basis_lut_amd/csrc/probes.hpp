// probes.hpp -- measurement kernels (not part of the method): the rooflines
// the GEMV is reported against, measured on the device it runs on.
//
//   * stream_read_kernel: the sustainable HBM read rate of the access pattern
//     the GEMV uses for its sign words (each wave reads contiguous 1 KiB
//     blocks with non-temporal 16-byte loads, D of them in flight);
//   * empty_kernel: the cost of a launch of a given grid (nothing but the
//     dispatch of its workgroups);
//   * lds_lookup_kernel: the rate of the GEMV's table lookups alone (LDS
//     reads plus their address and accumulate instructions) with weights held
//     in registers, for a table width and batch width: the roofline of the
//     batch path, which at several batch rows is bound by lookups, not HBM;
//   * lds_lookup_banked_kernel: the same for the g = 8 bank-private tables.
#pragma once

#include "common.hpp"
#include "gemv_banked.hpp"

namespace fluxbin {

// Wave w reads elements [w * per_wave, min((w + 1) * per_wave, n16)) of
// `buf` (16-byte elements), 64 consecutive elements (1 KiB) per load
// instruction, D instructions in flight.  The loaded words are folded into
// one value per lane that is stored only if it matches `never` (the caller
// passes a value no fold produces in practice), so that the loads are kept.
template <int D>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, int64_t n16, int64_t per_wave,
                                                          uint32_t never, uint32_t *sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t start = wave * per_wave;
  const int64_t end = min(start + per_wave, n16);
  const FB_GLOBAL u32x4 *g = (const FB_GLOBAL u32x4 *)(uintptr_t)buf;
  uint32_t acc = 0;
  for (int64_t i = start + lane; i < end; i += 64 * D) {
    u32x4 v[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int64_t e = i + 64 * u;
      v[u] = __builtin_nontemporal_load(g + min(e, end - 1));
    }
#pragma unroll
    for (int u = 0; u < D; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == never) sink[wave * 64 + lane] = acc;
}

__global__ void empty_kernel() {}

// Table lookups at the GEMV's instruction mix: every wave holds one chunk of
// sign words per lane (16 bytes, drawn from a per-lane hash) and looks them up
// `iters` times in NB batch rows' tables of width G, accumulating in fp32.
// The tables (LDS) are filled from the thread index.  The empty asm statements
// make the words opaque at every iteration, so that the address instructions
// are executed per lookup as in the GEMV instead of being hoisted out of the
// loop, and keep every iteration's table reads inside its iteration.
template <int G, int NB>
__global__ __launch_bounds__(256) void lds_lookup_kernel(int32_t iters, uint32_t seed, float never, float *sink) {
  constexpr int SUB = kChunkCols / G;
  constexpr int TAB = 1 << G;
  constexpr int CTB = NB * SUB * TAB * 4;
  extern __shared__ __align__(1024) float smem[];
  const int tid = threadIdx.x;
  for (int e = tid; e < CTB / 4; e += blockDim.x) smem[e] = (float)(e & 1023) * 0.001f;
  __syncthreads();
  uint32_t h = seed ^ (uint32_t)(blockIdx.x * 256 + tid) * 0x9e3779b9u;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    w[q] = h;
  }
  const uint32_t base = lds_addr(smem);
  float acc0[NB], acc1[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = 0.0f;
  float(&accb)[NB] = NB == 1 ? acc1 : acc0;  // the GEMV's chains: two for one batch row
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(w[q]));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lookup_word<G, NB, 4>(w[q], base, acc0, accb, q * (32 / G));
      if constexpr (NB >= 4) asm volatile("" ::: "memory");
    }
    asm volatile("" ::: "memory");
  }
  float s = 0.0f;
#pragma unroll
  for (int b = 0; b < NB; ++b) s += acc0[b] + acc1[b];
  if (s == never) sink[blockIdx.x * 256 + tid] = s;
}

// The banked g = 8 lookups of lut_gemv_g8_banked_kernel (BankedLane) on a
// region of R chunks, 8 waves per workgroup as in the GEMV: every lane holds
// R groups of 16 bytes of sign words (per-lane hash) and looks them up
// `iters` times, 16 R lookups per iteration.
template <int R>
__global__ __launch_bounds__(512) void lds_lookup_banked_kernel(int32_t iters, uint32_t seed, float never,
                                                               float *sink) {
  constexpr int NTAB = 16 * R;
  extern __shared__ __align__(1024) float smem[];
  const int tid = threadIdx.x;
  if (lds_addr(smem) != 0) return;  // the banked addresses carry no base (no static LDS here)
  for (int e = tid; e < NTAB * 256; e += blockDim.x) smem[e] = (float)(e & 1023) * 0.001f;
  __syncthreads();
  const int lane = tid & 63;
  const BankedLane<R> L((lane >> 4) % R, lane & 15);
  uint32_t h = seed ^ (uint32_t)(blockIdx.x * 512 + tid) * 0x9e3779b9u;
  u32x4 w[R];
#pragma unroll
  for (int g = 0; g < R; ++g) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h ^= h << 13;
      h ^= h >> 17;
      h ^= h << 5;
      w[g][q] = h;
    }
  }
  float acc[R][2];
#pragma unroll
  for (int g = 0; g < R; ++g) acc[g][0] = acc[g][1] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int g = 0; g < R; ++g) asm volatile("" : "+v"(w[g]));
    uint32_t ew[R][4];
#pragma unroll
    for (int g = 0; g < R; ++g) L.order(w[g], ew[g]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int g = 0; g < R; ++g) acc[g][kk & 1] += L.entry(ew[g], q, kk);
      }
    }
    asm volatile("" ::: "memory");
  }
  float s = 0.0f;
#pragma unroll
  for (int g = 0; g < R; ++g) s += acc[g][0] + acc[g][1];
  if (s == never) sink[blockIdx.x * 512 + tid] = s;
}

}  // namespace fluxbin
