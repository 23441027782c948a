// fluxbin.hip -- C ABI of libfluxbin.so (declared in include/fluxbin.h).
//
// Host side: argument validation (pure host work, before any HIP call),
// work planning, kernel launches.  The GEMV kernel instances live in the
// gemv_g*_rs*_t*.hip translation units (gemv_kernel.hpp), the other kernels in
// aux_kernels.hpp.
#include "fluxbin.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "aux_kernels.hpp"
#include "gemm_mfma.hpp"
#include "decomp_kernels.hpp"

using namespace fluxbin;

namespace {

thread_local char g_err[512] = "";

fluxbin_status fail(fluxbin_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

fluxbin_status hip_fail(hipError_t e, const char *what) {
  return fail(FLUXBIN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

fluxbin_status ok() {
  g_err[0] = '\0';
  return FLUXBIN_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kTargetBlocks = 1024;  // about four workgroups per CU
constexpr int64_t kWideWork = 32768;  // row tiles x chunks from which per-row layers take 8 waves

struct Plan {
  int32_t waves;       // waves per workgroup (64 rows each)
  int32_t nb;          // compiled batch width = batch rows per group (see batch_group)
  int32_t cpb;         // chunks per workgroup
  int32_t pf;          // chunks of weights in flight per wave (2 or 8)
  int32_t row_tiles;
  int32_t row_blocks;
  int32_t total_chunks;
  int32_t gchunks;     // chunks of the first range part (all chunks, or the global ones when block-wise)
  int32_t gsplits;     // workgroup ranges over the first part
  int32_t splits;
  int64_t n_pad;
  size_t acc_bytes;    // workspace (splits > 1): packed reduction words (LUT) or fp32 partials (MFMA)
  bool mfma;           // matrix-core route: ranges of one segment each
  int32_t ranges_g;    // matrix-core ranges per global / salient segment
  int32_t ranges_s;
};

constexpr int kMaxBatch = 128;

int32_t pow2_at_least(int64_t v) {
  int32_t p = 1;
  while (p < v) p <<= 1;
  return p;
}



fluxbin_status validate_shape(const fluxbin_layer_desc *d) {
  if (!d) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->abi_version != FLUXBIN_ABI_VERSION)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "abi_version %d, library %d", d->abi_version, FLUXBIN_ABI_VERSION);
  if (d->g != 4 && d->g != 8) return fail(FLUXBIN_ERR_UNSUPPORTED, "g = %d (supported: 4, 8)", d->g);
  if (d->kb < 1 || d->kb > 4) return fail(FLUXBIN_ERR_UNSUPPORTED, "kb = %d (supported: 1..4)", d->kb);
  if (d->ks < 0 || d->ks > 2) return fail(FLUXBIN_ERR_UNSUPPORTED, "ks = %d (supported: 0..2)", d->ks);
  if (d->n < 1 || d->k < 1) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "n = %lld, k = %lld (must be >= 1)",
                                        (long long)d->n, (long long)d->k);
  if (d->n > (int64_t)1 << 30 || d->k > (int64_t)1 << 30)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "n or k above 2^30");
  if (d->ks == 0 && d->s != 0) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "s = %lld with ks = 0", (long long)d->s);
  if (d->ks > 0 && (d->s < 1 || d->s > d->k))
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "s = %lld must be in [1, k] when ks > 0", (long long)d->s);
  if (d->max_batch < 1 || d->max_batch > kMaxBatch)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "max_batch = %lld (supported: 1..%d)", (long long)d->max_batch, kMaxBatch);
  if (d->chunks_per_block < 0 || d->chunks_per_block > kMaxCpb)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "chunks_per_block = %d (0 = automatic, else 1..%d)", d->chunks_per_block,
                kMaxCpb);
  if (d->waves_per_block != 0 && d->waves_per_block != 4 && d->waves_per_block != 8)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "waves_per_block = %d (0, 4 or 8)", d->waves_per_block);
  if (d->compute != FLUXBIN_COMPUTE_LUT && d->compute != FLUXBIN_COMPUTE_MFMA)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "compute = %d (0 = LUT, 1 = MFMA)", d->compute);
  if (d->compute == FLUXBIN_COMPUTE_MFMA && d->waves_per_block != 0 && d->waves_per_block != kMfmaWaves)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "waves_per_block = %d with compute MFMA (0 or %d)", d->waves_per_block,
                kMfmaWaves);
  if (d->table_precision != FLUXBIN_TABLE_F32 && d->table_precision != FLUXBIN_TABLE_F16)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "table_precision = %d (0 = fp32, 1 = fp16)", d->table_precision);
  if (d->row_group != 0 && d->row_group != kChunkCols)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "row_group = %d (supported: 0 = per row, 128 = block-wise)", d->row_group);
  if (d->row_group == 0 || d->ks == 0) {
    if (d->sal_group != 0)
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "sal_group = %d must be 0 without block-wise salient bases",
                  d->sal_group);
  } else {
    if (d->sal_group != 8 && d->sal_group != 16)
      return fail(FLUXBIN_ERR_UNSUPPORTED, "sal_group = %d (supported: 8, 16)", d->sal_group);
    if (d->sal_group % d->g)
      return fail(FLUXBIN_ERR_UNSUPPORTED, "sal_group = %d is not a multiple of g = %d", d->sal_group, d->g);
    const int64_t want = cdiv(d->k, d->row_group) * d->sal_group;
    if (d->s != want)
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "s = %lld, block-wise format needs sal_group * ceil(k / 128) = %lld",
                  (long long)d->s, (long long)want);
  }
  return FLUXBIN_OK;
}

// Chunks per workgroup: about kTargetBlocks workgroups' worth of work in all,
// a workgroup of nb batch rows counting nb times (measured on MI355X over
// 4096..57344-row layers: fewer, longer ranges amortise the table build, more
// workgroups hide latency; at 4 batch rows the 4096 -> 11008 projection ran
// 15.3 us with 4 chunks against 18.2 with 2), at least 2 chunks, a power of
// two up to 8 and a multiple of 8 above (the prefetch depths), within the
// LDS and register budget (cmax) and the split limit.
//
// Eight-wave g = 4 workgroups take at most 7 chunks: the depth-4 instance
// that serves them holds 58 VGPRs (8 waves per SIMD) against 78 (6 waves)
// for depth 8, and on the 70B gate+up projection (8192 -> 57344) 7-chunk
// ranges ran 34.7 us against 37.8 us for 8-chunk ones.
int32_t auto_cpb(int32_t g, int32_t nb, int32_t cmax, int32_t waves, int64_t row_tiles, int32_t total_chunks) {
  int64_t c = (int64_t)row_tiles * total_chunks * nb / ((int64_t)waves * kTargetBlocks);
  c = std::max<int64_t>(c, 2);
  if (g == 4 && waves == 8 && c > 7) {
    c = 7;
  } else if (c <= 8) {
    int64_t p = 1;
    while (p * 2 <= c) p *= 2;
    c = p;
  } else {
    c = c / 8 * 8;
  }
  c = std::max<int64_t>(c, cdiv(total_chunks, kMaxSplits));
  if (c > 8) c = cdiv(c, 8) * 8;
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(c, cmax));
}

// Batch rows one workgroup serves (the kernel's compiled width): the next
// power of two of max_batch, at most 16 (g = 4) or 4 (g = 8); wider batches
// run as several groups.
int32_t batch_group(int32_t g, int64_t max_batch) {
  const int64_t cap = g == 4 ? 16 : 4;
  return pow2_at_least(max_batch < cap ? max_batch : cap);
}

int entry_bytes(const fluxbin_layer_desc *d) { return d->table_precision == FLUXBIN_TABLE_F16 ? 2 : 4; }

// Matrix-core route: ranges of cpb chunks inside one segment (automatic cpb:
// mfma_auto_cpb, next to the kernel).
fluxbin_status make_mfma_plan(const fluxbin_layer_desc *d, Plan *p) {
  // x is addressed with 32-bit element offsets: batch row * k + column
  if (d->max_batch * d->k > (int64_t)INT32_MAX - kChunkCols)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "max_batch * k = %lld too large for compute MFMA (below 2^31)",
                (long long)(d->max_batch * d->k));
  p->mfma = true;
  p->nb = 0;
  p->pf = 0;
  p->waves = kMfmaWaves;
  p->row_blocks = (int32_t)cdiv(d->n, kMfmaRowsPerBlock);
  const int32_t nc_g = (int32_t)cdiv(d->k, kChunkCols), nc_s = d->ks > 0 ? (int32_t)cdiv(d->s, kChunkCols) : 0;
  auto splits_for = [&](int32_t c) { return d->kb * (int32_t)cdiv(nc_g, c) + d->ks * (int32_t)cdiv(nc_s, c); };
  int32_t cpb = d->chunks_per_block;
  if (!cpb) {
    cpb = mfma_auto_cpb((int32_t)cdiv(d->n, 2 * kTileRows), d->kb, nc_g, d->ks, nc_s, d->max_batch);
    while (splits_for(cpb) > kMaxSplits && cpb < kMaxCpb) ++cpb;
  }
  p->cpb = cpb;
  p->ranges_g = (int32_t)cdiv(nc_g, cpb);
  p->ranges_s = d->ks > 0 ? (int32_t)cdiv(nc_s, cpb) : 0;
  p->splits = splits_for(cpb);
  p->gsplits = d->kb * p->ranges_g;
  p->gchunks = d->kb * nc_g;
  if (p->splits > kMaxSplits)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "%d column ranges exceed %d (chunks_per_block %d)", p->splits, kMaxSplits,
                cpb);
  p->acc_bytes = p->splits > 1 ? (size_t)p->splits * d->max_batch * p->n_pad * sizeof(float) : 0;
  return FLUXBIN_OK;
}

fluxbin_status make_plan(const fluxbin_layer_desc *d, Plan *p) {
  p->row_tiles = (int32_t)cdiv(d->n, kTileRows);
  p->n_pad = (int64_t)p->row_tiles * kTileRows;
  p->total_chunks = (int32_t)(d->kb * cdiv(d->k, kChunkCols) + d->ks * cdiv(d->s, kChunkCols));
  p->mfma = false;
  p->ranges_g = p->ranges_s = 0;
  if (d->compute == FLUXBIN_COMPUTE_MFMA) return make_mfma_plan(d, p);
  p->nb = batch_group(d->g, d->max_batch);
  if (d->waves_per_block) {
    p->waves = d->waves_per_block;
  } else {
    // eight waves (512 rows) halve the per-row share of the table build: for
    // the large g = 8 tables, for very tall layers, and for large layers with
    // per-row scales (measured on MI355X: the 70B down projection, 128 row
    // tiles x 455 chunks, ran 20.4-21.5 us with 8 waves against 21.5-22.9
    // with 4, but 27.0 against 25.1-26.5 with block-wise scales; q_proj and
    // the 70B qkv / o shapes, 4 200 - 21 000 tile-chunks, are as fast or
    // faster with 4)
    const bool wide = !d->row_group && (int64_t)p->row_tiles * p->total_chunks >= kWideWork;
    p->waves = (d->g == 8 || p->row_tiles >= 512 || wide) ? 8 : 4;
  }
  const int32_t cmax = cpb_cap(d->g, p->nb, p->waves, entry_bytes(d));
  if (d->chunks_per_block > cmax)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "chunks_per_block = %d exceeds %d for g = %d, max_batch = %lld, %d waves",
                d->chunks_per_block, cmax, d->g, (long long)d->max_batch, p->waves);
  p->row_blocks = (int32_t)cdiv(p->row_tiles, p->waves);
  p->cpb = d->chunks_per_block ? d->chunks_per_block : auto_cpb(d->g, p->nb, cmax, p->waves, p->row_tiles, p->total_chunks);
  p->pf = prefetch_depth(p->cpb);
  if (d->row_group) {
    // block-wise: global and salient chunks take separate workgroup ranges
    p->gchunks = (int32_t)(d->kb * cdiv(d->k, kChunkCols));
    p->gsplits = (int32_t)cdiv(p->gchunks, p->cpb);
    p->splits = p->gsplits + (int32_t)cdiv(p->total_chunks - p->gchunks, p->cpb);
  } else {
    p->gchunks = p->total_chunks;
    p->splits = p->gsplits = (int32_t)cdiv(p->total_chunks, p->cpb);
  }
  if (p->splits > kMaxSplits)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "%d column splits exceed %d (too many 128-column chunks for chunks_per_block %d)",
                p->splits, kMaxSplits, p->cpb);
  p->acc_bytes = p->splits > 1 ? (size_t)d->max_batch * p->n_pad * sizeof(uint64_t) : 0;
  return FLUXBIN_OK;
}

}  // namespace

struct fluxbin_layer {
  fluxbin_layer_desc d;
  Plan plan;
  gemv_fn fn;                 // kernel instance for (g, row-scale format, batch width, waves, depth)
  size_t lds;                 // its dynamic LDS bytes
  const int32_t *idx_or_dummy;  // sal_idx, or the library's one-element zero array when ks == 0
  bool fault_launch;
};

// A valid index array for layers without salient bases: the GEMV reads its
// entry 0 (and ignores it) where a salient chunk would read its gather index.
__device__ int32_t g_zero_index[4];

// ---------------------------------------------------------------------------
// launch table for the GEMV kernel
// ---------------------------------------------------------------------------
namespace {

gemv_fn pick_gemv(int g, int rs, int tq, int nb, int waves, int pf) {
  if (g == 4 && tq == 0) return rs ? gemv_pick_g4_rs1_t32(nb, waves, pf) : gemv_pick_g4_rs0_t32(nb, waves, pf);
  if (g == 8 && tq == 0) return rs ? gemv_pick_g8_rs1_t32(nb, waves, pf) : gemv_pick_g8_rs0_t32(nb, waves, pf);
  if (g == 4 && tq == 1) return rs ? gemv_pick_g4_rs1_t16(nb, waves, pf) : gemv_pick_g4_rs0_t16(nb, waves, pf);
  if (g == 8 && tq == 1) return rs ? gemv_pick_g8_rs1_t16(nb, waves, pf) : gemv_pick_g8_rs0_t16(nb, waves, pf);
  return nullptr;
}

LayerArgs layer_args(const fluxbin_layer_desc &d) {
  LayerArgs L;
  L.bits_g = reinterpret_cast<const u32x4 *>(d.bits_global);
  L.bits_s = reinterpret_cast<const u32x4 *>(d.ks > 0 ? d.bits_sal : d.bits_global);
  L.c_g = d.c_global;
  L.c_s = d.ks > 0 ? d.c_sal : d.c_global;
  L.r_g = d.r_global;
  L.r_s = d.ks > 0 ? d.r_sal : d.r_global;
  L.sal_idx = d.ks > 0 ? d.sal_idx : nullptr;
  L.tv_g = fluxbin_tiled_words(d.n, d.k) / 4;
  L.tv_s = d.ks > 0 ? fluxbin_tiled_words(d.n, d.s) / 4 : 0;
  L.n = d.n;
  L.k = d.k;
  L.s = d.s;
  L.kb = d.kb;
  L.ks = d.ks;
  L.nc_g = (int32_t)cdiv(d.k, kChunkCols);
  L.nc_s = d.ks > 0 ? (int32_t)cdiv(d.s, kChunkCols) : 1;
  return L;
}

// Base pointers of every segment of a GEMV call (unused entries repeat the
// last segment, so that any index the kernel clamps to stays valid).
void gemv_segments(const fluxbin_layer_desc &d, SegDesc (&seg)[kMaxSeg]) {
  const int64_t tw_g = fluxbin_tiled_words(d.n, d.k), tw_s = d.ks > 0 ? fluxbin_tiled_words(d.n, d.s) : 0;
  const int32_t nc_g = (int32_t)cdiv(d.k, kChunkCols), nc_s = d.ks > 0 ? (int32_t)cdiv(d.s, kChunkCols) : 1;
  // row-scale elements per basis: n, or the tiled block-wise blocks
  const int64_t groups = d.row_group ? cdiv(d.k, d.row_group) : 0;
  const int64_t rs_g = d.row_group ? fluxbin_tiled_scale_elems(d.n, groups, 1) : d.n;
  const int64_t rs_s = d.row_group && d.ks > 0 ? fluxbin_tiled_scale_elems(d.n, groups, kChunkCols / d.sal_group) : d.n;
  int i = 0;
  for (int b = 0; b < d.kb; ++b, ++i) {
    seg[i].bits = reinterpret_cast<const u32x4 *>(d.bits_global) + b * tw_g / 4;
    seg[i].c = d.c_global + b * d.k;
    seg[i].r = d.r_global + b * rs_g;
    seg[i].len = (int32_t)d.k;
    seg[i].nchunks = nc_g;
  }
  for (int b = 0; b < d.ks; ++b, ++i) {
    seg[i].bits = reinterpret_cast<const u32x4 *>(d.bits_sal) + b * tw_s / 4;
    seg[i].c = d.c_sal + b * d.s;
    seg[i].r = d.r_sal + b * rs_s;
    seg[i].len = (int32_t)d.s;
    seg[i].nchunks = nc_s;
  }
  for (; i < kMaxSeg; ++i) seg[i] = seg[i - 1];
}

int grid_for(int64_t items, int per_thread_block = 256) {
  int64_t g = cdiv(items, per_thread_block);
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

}  // namespace

// ---------------------------------------------------------------------------
// offline decomposition: argument checks and launches
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kDecompMaxRows = (int64_t)1 << 22;  // column-step grid.y = rows / 64 <= 65535

fluxbin_status decomp_shape(int64_t n, int64_t k, int32_t kb) {
  if (n < 1 || k < 1) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "n = %lld, k = %lld (must be >= 1)", (long long)n,
                                  (long long)k);
  if (n > kDecompMaxRows || k > ((int64_t)1 << 30))
    return fail(FLUXBIN_ERR_UNSUPPORTED, "n above 2^22 or k above 2^30");
  if (kb < 1 || kb > 4) return fail(FLUXBIN_ERR_UNSUPPORTED, "kb = %d (supported: 1..4)", kb);
  return FLUXBIN_OK;
}

// Partials of the row and column steps: [ceil(n/64)][k] for the columns,
// [ceil(k/512)][n] for the rows (tiled form); the larger of the two.
int64_t decomp_partial_elems(int64_t n, int64_t k) {
  return std::max(cdiv(n, kDecompRowChunk) * k, cdiv(k, kDecompTileCols) * n);
}

size_t decomp_ws_bytes(int64_t n, int64_t k) {
  return sizeof(double) * (size_t)(decomp_partial_elems(n, k) + kDecompErrBlocks + 16 + 4 * (n + k));
}

// Workspace: the step partials, kDecompErrBlocks error partials, 16 scalars,
// then room for fp64 copies of the rounded scales (up to 4 bases).
struct DecompWs {
  double *partial, *errp, *scal, *rounded;
};

fluxbin_status decomp_ws(void *ws, size_t bytes, int64_t n, int64_t k, DecompWs *out) {
  const size_t need = decomp_ws_bytes(n, k);
  if (!ws || bytes < need)
    return fail(FLUXBIN_ERR_WORKSPACE, "decomposition workspace of %zu bytes needed, %zu given", need,
                ws ? bytes : (size_t)0);
  if (!aligned(ws, 256)) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  out->partial = static_cast<double *>(ws);
  out->errp = out->partial + decomp_partial_elems(n, k);
  out->scal = out->errp + kDecompErrBlocks;
  out->rounded = out->scal + 16;
  return FLUXBIN_OK;
}

dim3 grid1(int64_t items, int per = 256) { return dim3((unsigned)cdiv(items, per)); }

// The tiled kernels read W with 16-byte loads: rows must start 16-byte aligned.
bool decomp_tiled(const uint16_t *w, int64_t k) { return k % 8 == 0 && aligned(w, 16); }

dim3 decomp_tiles(int64_t n, int64_t k) {
  return dim3((unsigned)cdiv(k, kDecompTileCols), (unsigned)cdiv(n, kDecompTileRows));
}

// kernel<KB> for a run-time kb in 1..4
#define FB_KB_SWITCH(kb, KERNEL, ...)                                   \
  switch (kb) {                                                         \
    case 1: hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); break;          \
    case 2: hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); break;          \
    case 3: hipLaunchKernelGGL(KERNEL<3>, __VA_ARGS__); break;          \
    default: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;         \
  }

void run_row(hipStream_t st, const uint16_t *w, int64_t n, int64_t k, int kb, int basis, const uint32_t *bits,
             const double *r, const double *c, const double *d, double *r_out, const DecompWs &ws) {
  hipLaunchKernelGGL(decomp_sumsq_kernel, dim3(1), dim3(kSumsqThreads), 0, st, c + (int64_t)basis * k, d, k, ws.scal);
  if (decomp_tiled(w, k)) {
    FB_KB_SWITCH(kb, decomp_row_tiled_kernel, decomp_tiles(n, k), dim3(256), 0, st, w, n, k, basis, bits, r, c, d,
                 ws.partial)
    hipLaunchKernelGGL(decomp_row_finish_kernel, grid1(n), dim3(256), 0, st, ws.partial, cdiv(k, kDecompTileCols), n,
                       ws.scal, r_out);
  } else {
    hipLaunchKernelGGL(decomp_row_kernel, grid1(n, 4), dim3(256), 0, st, w, n, k, kb, basis, bits, r, c, d, ws.scal,
                       r_out);
  }
}

void run_col(hipStream_t st, const uint16_t *w, int64_t n, int64_t k, int kb, int basis, const uint32_t *bits,
             const double *r, const double *c, double *c_out, const DecompWs &ws) {
  const int64_t chunks = cdiv(n, kDecompRowChunk);
  hipLaunchKernelGGL(decomp_sumsq_kernel, dim3(1), dim3(kSumsqThreads), 0, st, r + (int64_t)basis * n, nullptr, n, ws.scal);
  if (decomp_tiled(w, k)) {
    FB_KB_SWITCH(kb, decomp_col_tiled_kernel, decomp_tiles(n, k), dim3(256), 0, st, w, n, k, basis, bits, r, c,
                 ws.partial)
  } else {
    hipLaunchKernelGGL(decomp_col_partial_kernel, dim3((unsigned)cdiv(k, 256), (unsigned)chunks), dim3(256), 0, st,
                       w, n, k, kb, basis, bits, r, c, ws.partial);
  }
  hipLaunchKernelGGL(decomp_col_finish_kernel, grid1(k), dim3(256), 0, st, ws.partial, chunks, k, ws.scal, c_out);
}

void run_signs(hipStream_t st, const uint16_t *w, int64_t n, int64_t k, int kb, const double *r, const double *c,
               uint32_t *bits) {
  if (decomp_tiled(w, k)) {
    switch (kb) {
      case 1: hipLaunchKernelGGL((decomp_sign_tiled_kernel<1, false>), decomp_tiles(n, k), dim3(256), 0, st, w, n, k,
                                 0, nullptr, r, c, bits); break;
      case 2: hipLaunchKernelGGL((decomp_sign_tiled_kernel<2, false>), decomp_tiles(n, k), dim3(256), 0, st, w, n, k,
                                 0, nullptr, r, c, bits); break;
      case 3: hipLaunchKernelGGL((decomp_sign_tiled_kernel<3, false>), decomp_tiles(n, k), dim3(256), 0, st, w, n, k,
                                 0, nullptr, r, c, bits); break;
      default: hipLaunchKernelGGL((decomp_sign_tiled_kernel<4, false>), decomp_tiles(n, k), dim3(256), 0, st, w, n,
                                  k, 0, nullptr, r, c, bits); break;
    }
    return;
  }
  const dim3 g = grid1(n * cdiv(k, 64), 4);
  switch (kb) {
    case 1: hipLaunchKernelGGL(decomp_sign_kernel<1>, g, dim3(256), 0, st, w, n, k, r, c, bits); break;
    case 2: hipLaunchKernelGGL(decomp_sign_kernel<2>, g, dim3(256), 0, st, w, n, k, r, c, bits); break;
    case 3: hipLaunchKernelGGL(decomp_sign_kernel<3>, g, dim3(256), 0, st, w, n, k, r, c, bits); break;
    default: hipLaunchKernelGGL(decomp_sign_kernel<4>, g, dim3(256), 0, st, w, n, k, r, c, bits); break;
  }
}

void run_residual_signs(hipStream_t st, const uint16_t *w, int64_t n, int64_t k, int kb, int basis,
                        const uint32_t *bits, const double *r, const double *c, uint32_t *out) {
  if (decomp_tiled(w, k)) {
    switch (kb) {
      case 1: hipLaunchKernelGGL((decomp_sign_tiled_kernel<1, true>), decomp_tiles(n, k), dim3(256), 0, st, w, n, k,
                                 basis, bits, r, c, out); break;
      case 2: hipLaunchKernelGGL((decomp_sign_tiled_kernel<2, true>), decomp_tiles(n, k), dim3(256), 0, st, w, n, k,
                                 basis, bits, r, c, out); break;
      case 3: hipLaunchKernelGGL((decomp_sign_tiled_kernel<3, true>), decomp_tiles(n, k), dim3(256), 0, st, w, n, k,
                                 basis, bits, r, c, out); break;
      default: hipLaunchKernelGGL((decomp_sign_tiled_kernel<4, true>), decomp_tiles(n, k), dim3(256), 0, st, w, n,
                                  k, basis, bits, r, c, out); break;
    }
    return;
  }
  hipLaunchKernelGGL(decomp_residual_sign_kernel, grid1(n * cdiv(k, 64), 4), dim3(256), 0, st, w, n, k, kb, basis,
                     bits, r, c, out);
}

void run_error(hipStream_t st, const uint16_t *w, int64_t n, int64_t k, int kb, const uint32_t *bits,
               const double *r, const double *c, const double *d, double *out, const DecompWs &ws) {
  hipLaunchKernelGGL(decomp_error_partial_kernel, dim3(kDecompErrBlocks), dim3(256), 0, st, w, n, k, kb, bits, r, c,
                     d, ws.errp);
  hipLaunchKernelGGL(decomp_error_finish_kernel, dim3(1), dim3(64), 0, st, ws.errp, kDecompErrBlocks, out);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int32_t fluxbin_abi_version(void) { return FLUXBIN_ABI_VERSION; }

const char *fluxbin_status_string(fluxbin_status s) {
  switch (s) {
    case FLUXBIN_OK: return "ok";
    case FLUXBIN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FLUXBIN_ERR_UNSUPPORTED: return "unsupported";
    case FLUXBIN_ERR_WORKSPACE: return "workspace missing or too small";
    case FLUXBIN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *fluxbin_last_error(void) { return g_err; }

int64_t fluxbin_tiled_words(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  return cdiv(rows, kTileRows) * cdiv(cols, kChunkCols) * kTileRows * 4;
}

int64_t fluxbin_tiled_scale_elems(int64_t rows, int64_t groups, int64_t groups_per_chunk) {
  if (rows <= 0 || groups <= 0 || groups_per_chunk < 1 || groups_per_chunk > kChunkCols) return 0;
  return cdiv(rows, kTileRows) * cdiv(groups, groups_per_chunk) * kTileRows * groups_per_chunk;
}

fluxbin_status fluxbin_relayout_scales(const uint16_t *src, int64_t rows, int64_t groups, int64_t groups_per_chunk,
                                       int32_t src_layout, int32_t dst_layout, uint16_t *dst, void *stream) {
  if (rows < 0 || groups < 0) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "negative size");
  if (groups_per_chunk < 1 || groups_per_chunk > kChunkCols)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "groups_per_chunk = %lld (1..%d)", (long long)groups_per_chunk,
                kChunkCols);
  for (int32_t l : {src_layout, dst_layout})
    if (l != FLUXBIN_LAYOUT_ROWMAJOR && l != FLUXBIN_LAYOUT_TILED)
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "layout = %d", l);
  if (rows == 0 || groups == 0) return ok();
  if (!src || !dst) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (src == dst) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "src and dst must not overlap");
  const int64_t elems = dst_layout == FLUXBIN_LAYOUT_ROWMAJOR ? rows * groups
                                                             : fluxbin_tiled_scale_elems(rows, groups, groups_per_chunk);
  hipLaunchKernelGGL(relayout_scales_kernel, dim3(grid_for(elems)), dim3(256), 0, (hipStream_t)stream, src, rows,
                     groups, groups_per_chunk, src_layout, dst_layout, dst, elems);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "relayout_scales launch");
  return ok();
}

fluxbin_status fluxbin_pack(const int8_t *signs, int64_t rows, int64_t cols, int64_t ld, int32_t layout,
                            uint32_t *packed, uint32_t *invalid_count, void *stream) {
  if (rows < 0 || cols < 0) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "negative size");
  if (layout != FLUXBIN_LAYOUT_ROWMAJOR && layout != FLUXBIN_LAYOUT_TILED)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "layout = %d", layout);
  if (rows == 0 || cols == 0) return ok();
  if (!signs || !packed) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (ld < cols) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "ld = %lld < cols = %lld", (long long)ld, (long long)cols);
  const int64_t words = layout == FLUXBIN_LAYOUT_ROWMAJOR ? rows * cdiv(cols, 32) : fluxbin_tiled_words(rows, cols);
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(words)), dim3(256), 0, (hipStream_t)stream, signs, rows, cols, ld,
                     layout, packed, invalid_count, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

fluxbin_status fluxbin_relayout(const uint32_t *src, int64_t rows, int64_t cols, int32_t src_layout,
                                int32_t dst_layout, uint32_t *dst, void *stream) {
  if (rows < 0 || cols < 0) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "negative size");
  for (int32_t l : {src_layout, dst_layout})
    if (l != FLUXBIN_LAYOUT_ROWMAJOR && l != FLUXBIN_LAYOUT_TILED)
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "layout = %d", l);
  if (rows == 0 || cols == 0) return ok();
  if (!src || !dst) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (src == dst) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "src and dst must not overlap");
  const int64_t words =
      dst_layout == FLUXBIN_LAYOUT_ROWMAJOR ? rows * cdiv(cols, 32) : fluxbin_tiled_words(rows, cols);
  hipLaunchKernelGGL(relayout_kernel, dim3(grid_for(words)), dim3(256), 0, (hipStream_t)stream, src, rows, cols,
                     src_layout, dst_layout, dst, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "relayout launch");
  return ok();
}

fluxbin_status fluxbin_vcm_gather(const int32_t *idx, int64_t s, const void *src, int64_t rows, int64_t cols,
                                  int32_t dtype, void *dst, void *stream) {
  if (s < 0 || rows < 0 || cols < 0) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "negative size");
  if (dtype != FLUXBIN_DT_I8 && dtype != FLUXBIN_DT_F16 && dtype != FLUXBIN_DT_BITS)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "dtype = %d", dtype);
  if (s == 0 || rows == 0) return ok();
  if (!idx || !src || !dst) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (cols < 1) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "cols = 0 with s > 0");
  hipStream_t st = (hipStream_t)stream;
  if (dtype == FLUXBIN_DT_I8) {
    hipLaunchKernelGGL(vcm_gather_values_kernel<int8_t>, dim3(grid_for(rows * s)), dim3(256), 0, st, idx, s,
                       (const int8_t *)src, rows, cols, (int8_t *)dst, (int8_t)-1);
  } else if (dtype == FLUXBIN_DT_F16) {
    hipLaunchKernelGGL(vcm_gather_values_kernel<uint16_t>, dim3(grid_for(rows * s)), dim3(256), 0, st, idx, s,
                       (const uint16_t *)src, rows, cols, (uint16_t *)dst, (uint16_t)0);
  } else {
    hipLaunchKernelGGL(vcm_gather_bits_kernel, dim3(grid_for(rows * cdiv(s, 32))), dim3(256), 0, st, idx, s,
                       (const uint32_t *)src, rows, cols, (uint32_t *)dst);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "vcm gather launch");
  return ok();
}

fluxbin_status fluxbin_workspace_size(const fluxbin_layer_desc *d, size_t *bytes) {
  fluxbin_status st = validate_shape(d);
  if (st) return st;
  if (!bytes) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan p;
  st = make_plan(d, &p);
  if (st) return st;
  *bytes = p.acc_bytes;
  return ok();
}

fluxbin_status fluxbin_create(const fluxbin_layer_desc *d, fluxbin_handle *out) {
  fluxbin_status st = validate_shape(d);
  if (st) return st;
  if (!out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!d->bits_global || !d->r_global || !d->c_global)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "global basis pointers must be non-NULL");
  if (!aligned(d->bits_global, 16)) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bits_global not 16-byte aligned");
  if (d->ks > 0) {
    if (!d->bits_sal || !d->r_sal || !d->c_sal || !d->sal_idx)
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "salient pointers must be non-NULL when ks > 0");
    if (!aligned(d->bits_sal, 16)) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bits_sal not 16-byte aligned");
    if (d->row_group && !aligned(d->r_sal, 16))
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "r_sal not 16-byte aligned (block-wise scales)");
  }
  Plan p;
  st = make_plan(d, &p);
  if (st) return st;
  const size_t need = p.acc_bytes;
  if (need > 0) {
    if (!d->workspace || d->workspace_bytes < need)
      return fail(FLUXBIN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  d->workspace ? d->workspace_bytes : (size_t)0);
    if (!aligned(d->workspace, 256)) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  }
  // salient index: strictly ascending, in [0, k)
  if (d->ks > 0) {
    std::vector<int32_t> idx((size_t)d->s);
    hipError_t e = hipMemcpy(idx.data(), d->sal_idx, (size_t)d->s * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "reading sal_idx");
    for (int64_t i = 0; i < d->s; ++i) {
      if (idx[i] < 0 || idx[i] >= d->k)
        return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "sal_idx[%lld] = %d outside [0, %lld)", (long long)i, idx[i],
                    (long long)d->k);
      if (i > 0 && idx[i] <= idx[i - 1])
        return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "sal_idx not strictly ascending at %lld", (long long)i);
      if (d->row_group && idx[i] / d->row_group != i / d->sal_group)
        return fail(FLUXBIN_ERR_INVALID_ARGUMENT,
                    "sal_idx[%lld] = %d is not in column group %lld (block-wise: %d salient columns per group)",
                    (long long)i, idx[i], (long long)(i / d->sal_group), d->sal_group);
    }
  }
  if (p.acc_bytes) {
    hipError_t e = hipMemset(d->workspace, 0, p.acc_bytes);
    if (e != hipSuccess) return hip_fail(e, "zeroing the split-reduction words");
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "synchronising after create");
  }
  gemv_fn fn = nullptr;
  size_t lds = 0;
  hipError_t e = hipSuccess;
  if (!p.mfma) {
    fn = pick_gemv(d->g, d->row_group ? 1 : 0, d->table_precision, p.nb, p.waves, p.pf);
    if (!fn) return fail(FLUXBIN_ERR_UNSUPPORTED, "no kernel for g = %d, batch width %d, %d waves", d->g, p.nb, p.waves);
    lds = (size_t)lds_bytes(d->g, p.nb, p.cpb, entry_bytes(d));
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e, "setting the kernel's dynamic LDS size");
  }
  const int32_t *idx = d->sal_idx;
  if (d->ks == 0) {
    void *z = nullptr;
    e = hipGetSymbolAddress(&z, HIP_SYMBOL(g_zero_index));
    if (e != hipSuccess) return hip_fail(e, "locating the zero index array");
    idx = static_cast<const int32_t *>(z);
  }
  fluxbin_layer *h = new (std::nothrow) fluxbin_layer;
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "out of host memory");
  h->fn = fn;
  h->lds = lds;
  h->idx_or_dummy = idx;
  h->d = *d;
  h->plan = p;
  const char *f = getenv("FLUXBIN_FAULT");
  h->fault_launch = f && strcmp(f, "launch") == 0;
  *out = h;
  return ok();
}

fluxbin_status fluxbin_destroy(fluxbin_handle h) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  delete h;
  return ok();
}

namespace {

void fill_plan(const fluxbin_layer_desc &d, const Plan &p, fluxbin_plan *plan) {
  plan->rows_per_block = p.mfma ? kMfmaRowsPerBlock : p.waves * kTileRows;
  plan->chunks_per_block = p.cpb;
  plan->row_blocks = p.row_blocks;
  plan->splits = p.splits;
  plan->total_chunks = p.total_chunks;
  plan->lds_bytes = p.mfma ? mfma_lds_bytes(1, 1, 2) : lds_bytes(d.g, p.nb, p.cpb, entry_bytes(&d));
  plan->grid = (int64_t)p.row_blocks * p.splits;
}

}  // namespace

fluxbin_status fluxbin_get_plan(fluxbin_handle h, fluxbin_plan *plan) {
  if (!h || !plan) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL argument");
  fill_plan(h->d, h->plan, plan);
  return ok();
}

fluxbin_status fluxbin_plan_of(const fluxbin_layer_desc *d, fluxbin_plan *plan) {
  fluxbin_status st = validate_shape(d);
  if (st) return st;
  if (!plan) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "plan is NULL");
  Plan p;
  st = make_plan(d, &p);
  if (st) return st;
  fill_plan(*d, p, plan);
  return ok();
}

fluxbin_status fluxbin_lut_size(fluxbin_handle h, int64_t batch, size_t *floats) {
  if (!h || !floats) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL argument");
  if (batch < 0) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "negative batch");
  const fluxbin_layer_desc &d = h->d;
  const int64_t subs = d.kb * cdiv(d.k, d.g) + d.ks * cdiv(d.s, d.g);
  *floats = (size_t)(batch * subs * ((int64_t)1 << (d.g - 1)));
  return ok();
}

fluxbin_status fluxbin_build_lut(fluxbin_handle h, const uint16_t *x, int64_t batch, float *lut, void *stream) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (batch < 0 || batch > h->d.max_batch)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "batch = %lld outside [0, %lld]", (long long)batch,
                (long long)h->d.max_batch);
  if (batch == 0) return ok();
  if (!x || !lut) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (h->fault_launch) return fail(FLUXBIN_ERR_HIP, "injected launch fault (FLUXBIN_FAULT=launch)");
  const fluxbin_layer_desc &d = h->d;
  LutArgs a;
  a.L = layer_args(d);
  a.g = d.g;
  a.batch = (int32_t)batch;
  a.sub_g = cdiv(d.k, d.g);
  a.sub_s = d.ks > 0 ? cdiv(d.s, d.g) : 1;
  const int64_t sub = d.kb * a.sub_g + (d.ks > 0 ? d.ks * a.sub_s : 0);
  a.subs_per_batch = sub;
  a.x = x;
  a.lut = lut;
  const int64_t total = batch * sub * ((int64_t)1 << (d.g - 1));
  if (d.g == 4)
    hipLaunchKernelGGL(build_lut_kernel<4>, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL(build_lut_kernel<8>, dim3(grid_for(total)), dim3(256), 0, (hipStream_t)stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "build_lut launch");
  return ok();
}

namespace {

// The matrix-core route (instance for the batch: mfma_instance, next to the
// kernel; the per-element arithmetic does not depend on it).
fluxbin_status mfma_gemv(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, hipStream_t stream) {
  const fluxbin_layer_desc &d = h->d;
  const Plan &p = h->plan;
  const MfmaInstance in = mfma_instance(batch, d.row_group ? 1 : 0);
  if (!in.fn) return fail(FLUXBIN_ERR_UNSUPPORTED, "no matrix-core kernel for batch %lld", (long long)batch);
  const int64_t rows_per_block = (int64_t)(kMfmaWaves / in.wb) * 32 * in.rb;
  MfmaArgs a;
  a.L = layer_args(d);
  a.idx_or_dummy = h->idx_or_dummy;
  a.x = x;
  a.y = y;
  a.part = p.splits > 1 ? reinterpret_cast<float *>(d.workspace) : nullptr;
  a.n_pad = p.n_pad;
  const int64_t groups = d.row_group ? cdiv(d.k, d.row_group) : 0;
  a.rstride_g = d.row_group ? fluxbin_tiled_scale_elems(d.n, groups, 1) : d.n;
  a.rstride_s = d.row_group && d.ks > 0 ? fluxbin_tiled_scale_elems(d.n, groups, kChunkCols / d.sal_group) : d.n;
  a.cpb = p.cpb;
  a.ranges_g = p.ranges_g;
  a.ranges_s = p.ranges_s;
  a.row_tiles = p.row_tiles;
  a.row_blocks = (int32_t)cdiv(d.n, rows_per_block);
  a.splits = p.splits;
  a.batch = (int32_t)batch;
  a.xvec = d.k % 8 == 0 && aligned(x, 16) && aligned(d.c_global, 16) ? 1 : 0;
  a.sal_group = d.row_group && d.ks > 0 ? d.sal_group : kChunkCols;
  const dim3 grid((unsigned)((int64_t)a.row_blocks * p.splits), (unsigned)cdiv(batch, 32 * in.nbt * in.wb));
  hipLaunchKernelGGL(in.fn, grid, dim3(kMfmaWaves * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "matrix-core gemv launch");
  if (p.splits > 1) {
    hipLaunchKernelGGL(mfma_finalize_kernel, dim3(grid_for(batch * d.n)), dim3(256), 0, stream, a.part, p.splits,
                       (int32_t)batch, d.n, p.n_pad, y);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "matrix-core finalize launch");
  }
  return ok();
}

}  // namespace

fluxbin_status fluxbin_gemv(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (batch < 0 || batch > h->d.max_batch)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "batch = %lld outside [0, %lld]", (long long)batch,
                (long long)h->d.max_batch);
  if (batch == 0) return ok();
  if (!x || !y) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (h->fault_launch) return fail(FLUXBIN_ERR_HIP, "injected launch fault (FLUXBIN_FAULT=launch)");
  const fluxbin_layer_desc &d = h->d;
  const Plan &p = h->plan;
  if (p.mfma) return mfma_gemv(h, x, y, batch, (hipStream_t)stream);
  GemvArgs a;
  a.L = layer_args(d);
  gemv_segments(d, a.seg);
  a.idx_or_dummy = h->idx_or_dummy;
  a.cpb = p.cpb;
  a.total_chunks = p.total_chunks;
  a.gsplits = p.gsplits;
  a.gchunks = p.gchunks;
  a.sal16 = d.row_group && d.ks > 0 && d.sal_group == 8 ? 1 : 0;
  a.row_tiles = p.row_tiles;
  a.row_blocks = p.row_blocks;
  a.splits = p.splits;
  a.n_pad = p.n_pad;
  uint64_t *acc = p.splits > 1 ? reinterpret_cast<uint64_t *>(d.workspace) : nullptr;
  const int64_t grid = (int64_t)p.row_blocks * p.splits;
  // one launch per group of p.nb batch rows (a prefill batch runs as several groups,
  // each building its own tables and streaming the weights again)
  for (int64_t b0 = 0; b0 < batch; b0 += p.nb) {
    a.batch = (int32_t)std::min<int64_t>(p.nb, batch - b0);
    a.x = x + b0 * d.k;
    a.y = y + b0 * d.n;
    a.acc = acc ? acc + b0 * p.n_pad : nullptr;
    hipLaunchKernelGGL(h->fn, dim3((unsigned)grid), dim3(p.waves * 64), h->lds, (hipStream_t)stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "gemv launch");
  }
  return ok();
}

fluxbin_status fluxbin_dense_gemv_f16(const uint16_t *w, int64_t n, int64_t k, const uint16_t *x, uint16_t *y,
                                      int64_t batch, void *stream) {
  if (n < 1 || k < 1) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "n, k must be >= 1");
  if (k % 8) return fail(FLUXBIN_ERR_UNSUPPORTED, "k = %lld not a multiple of 8", (long long)k);
  if (batch < 1 || batch > 16) return fail(FLUXBIN_ERR_UNSUPPORTED, "batch = %lld (1..16)", (long long)batch);
  if (!w || !x || !y) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!aligned(w, 16) || !aligned(x, 16)) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "w and x must be 16-B aligned");
  const int nb = pow2_at_least(batch);
  const dim3 grid((unsigned)cdiv(n, 4)), block(256);
  hipStream_t st = (hipStream_t)stream;
  switch (nb) {
    case 1: hipLaunchKernelGGL(dense_f16_gemv_kernel<1>, grid, block, 0, st, w, n, k, x, y, (int)batch); break;
    case 2: hipLaunchKernelGGL(dense_f16_gemv_kernel<2>, grid, block, 0, st, w, n, k, x, y, (int)batch); break;
    case 4: hipLaunchKernelGGL(dense_f16_gemv_kernel<4>, grid, block, 0, st, w, n, k, x, y, (int)batch); break;
    case 8: hipLaunchKernelGGL(dense_f16_gemv_kernel<8>, grid, block, 0, st, w, n, k, x, y, (int)batch); break;
    default: hipLaunchKernelGGL(dense_f16_gemv_kernel<16>, grid, block, 0, st, w, n, k, x, y, (int)batch); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "dense gemv launch");
  return ok();
}

// ---------------------------------------------------------------------------
// offline decomposition
// ---------------------------------------------------------------------------

fluxbin_status fluxbin_decomp_workspace_size(int64_t n, int64_t k, int32_t kb, size_t *bytes) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (!bytes) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = decomp_ws_bytes(n, k);
  return ok();
}

fluxbin_status fluxbin_decomp_row_scales(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                         const uint32_t *bits, const double *r, const double *c,
                                         const double *col_weight, double *r_out, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (basis < 0 || basis >= kb) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "basis = %d outside [0, %d)", basis, kb);
  if (!w || !bits || !r || !c || !r_out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  DecompWs ws;
  st = decomp_ws(workspace, workspace_bytes, n, k, &ws);
  if (st) return st;
  run_row((hipStream_t)stream, w, n, k, kb, basis, bits, r, c, col_weight, r_out, ws);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? hip_fail(e, "decomposition row step launch") : ok();
}

fluxbin_status fluxbin_decomp_col_scales(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                         const uint32_t *bits, const double *r, const double *c, double *c_out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (basis < 0 || basis >= kb) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "basis = %d outside [0, %d)", basis, kb);
  if (!w || !bits || !r || !c || !c_out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  DecompWs ws;
  st = decomp_ws(workspace, workspace_bytes, n, k, &ws);
  if (st) return st;
  run_col((hipStream_t)stream, w, n, k, kb, basis, bits, r, c, c_out, ws);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? hip_fail(e, "decomposition column step launch") : ok();
}

fluxbin_status fluxbin_decomp_signs(const uint16_t *w, int64_t n, int64_t k, int32_t kb, const double *r,
                                    const double *c, uint32_t *bits_out, void *stream) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (!w || !r || !c || !bits_out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  run_signs((hipStream_t)stream, w, n, k, kb, r, c, bits_out);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? hip_fail(e, "decomposition sign step launch") : ok();
}

fluxbin_status fluxbin_decomp_residual_signs(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                             const uint32_t *bits, const double *r, const double *c,
                                             uint32_t *basis_bits_out, void *stream) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (basis < 0 || basis >= kb) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "basis = %d outside [0, %d)", basis, kb);
  if (!w || !bits || !r || !c || !basis_bits_out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  run_residual_signs((hipStream_t)stream, w, n, k, kb, basis, bits, r, c, basis_bits_out);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? hip_fail(e, "decomposition residual-sign launch") : ok();
}

fluxbin_status fluxbin_decomp_error(const uint16_t *w, int64_t n, int64_t k, int32_t kb, const uint32_t *bits,
                                    const double *r, const double *c, const double *col_weight, double *err_out,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (!w || !bits || !r || !c || !err_out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  DecompWs ws;
  st = decomp_ws(workspace, workspace_bytes, n, k, &ws);
  if (st) return st;
  run_error((hipStream_t)stream, w, n, k, kb, bits, r, c, col_weight, err_out, ws);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? hip_fail(e, "decomposition error launch") : ok();
}

fluxbin_status fluxbin_decompose(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t iters,
                                 const double *col_weight, uint32_t *bits, uint16_t *r16, uint16_t *c16, double *r64,
                                 double *c64, double *trace, void *workspace, size_t workspace_bytes, void *stream) {
  fluxbin_status st = decomp_shape(n, k, kb);
  if (st) return st;
  if (iters < 0 || iters > 10000) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "iters = %d (0..10000)", iters);
  if (!w || !bits || !r16 || !c16 || !r64 || !c64) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  DecompWs ws;
  st = decomp_ws(workspace, workspace_bytes, n, k, &ws);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t wpr = cdiv(k, 32);
  int64_t tr = 0;
  hipLaunchKernelGGL(decomp_zero_words_kernel, grid1(kb * n * wpr), dim3(256), 0, s, bits, kb * n * wpr);
  hipLaunchKernelGGL(decomp_fill_kernel, grid1(kb * n), dim3(256), 0, s, r64, kb * n, 0.0);
  hipLaunchKernelGGL(decomp_fill_kernel, grid1(kb * k), dim3(256), 0, s, c64, kb * k, 0.0);
  // initialisation: basis b from the signs of the residual of bases 0..b-1
  for (int b = 0; b < kb; ++b) {
    double *rb = r64 + (int64_t)b * n, *cb = c64 + (int64_t)b * k;
    hipLaunchKernelGGL(decomp_fill_kernel, grid1(k), dim3(256), 0, s, cb, k, 1.0);
    run_residual_signs(s, w, n, k, kb, b, bits, r64, c64, bits + (int64_t)b * n * wpr);
    run_row(s, w, n, k, kb, b, bits, r64, c64, col_weight, rb, ws);
    run_col(s, w, n, k, kb, b, bits, r64, c64, cb, ws);
  }
  if (trace) run_error(s, w, n, k, kb, bits, r64, c64, col_weight, trace + tr++, ws);
  for (int it = 0; it < iters; ++it) {
    for (int b = 0; b < kb; ++b) {
      run_row(s, w, n, k, kb, b, bits, r64, c64, col_weight, r64 + (int64_t)b * n, ws);
      if (trace) run_error(s, w, n, k, kb, bits, r64, c64, col_weight, trace + tr++, ws);
      run_col(s, w, n, k, kb, b, bits, r64, c64, c64 + (int64_t)b * k, ws);
      if (trace) run_error(s, w, n, k, kb, bits, r64, c64, col_weight, trace + tr++, ws);
    }
    run_signs(s, w, n, k, kb, r64, c64, bits);
    if (trace) run_error(s, w, n, k, kb, bits, r64, c64, col_weight, trace + tr++, ws);
  }
  // output: fp16 scales and a last sign step against them
  double *rr = ws.rounded, *cr = ws.rounded + kb * n;
  hipLaunchKernelGGL(decomp_round_kernel, grid1(kb * n), dim3(256), 0, s, r64, kb * n, r16, rr);
  hipLaunchKernelGGL(decomp_round_kernel, grid1(kb * k), dim3(256), 0, s, c64, kb * k, c16, cr);
  run_signs(s, w, n, k, kb, rr, cr, bits);
  if (trace) run_error(s, w, n, k, kb, bits, rr, cr, col_weight, trace + tr++, ws);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? hip_fail(e, "decomposition launch") : ok();
}

}  // extern "C"
