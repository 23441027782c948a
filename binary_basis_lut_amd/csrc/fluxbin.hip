// fluxbin.hip -- C ABI of libfluxbin.so (declared in include/fluxbin.h).
//
// Host side: argument validation (pure host work, before any HIP call),
// work planning, kernel launches.  The GEMV kernel instances live in the
// gemv_g*_rs*_t*.hip translation units (gemv_kernel.hpp), the other kernels in
// aux_kernels.hpp.
#include "fluxbin.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "aux_kernels.hpp"
#include "probes.hpp"
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
constexpr int kCus = 256;            // compute units of an MI355X (8 XCDs of 32)

struct Plan {
  int32_t waves;       // waves per workgroup (64 rows each)
  int32_t nb;          // compiled batch width = batch rows per group (see batch_group)
  int32_t cpb;         // most chunks in one column range
  int32_t tb;          // chunks whose tables LDS holds at once (LDS is sized for it): cpb, or for
                       // several batch rows a multiple of pf below cpb (tables built in groups)
  int32_t pf;          // chunks of weights in flight per wave (2, 3 or 4)
  int32_t ks;          // waves per row tile (g = 4, one batch row: 1, or 2 over the two halves of a range)
  int32_t row_tiles;
  int32_t row_blocks;
  int32_t total_chunks;
  int32_t rpg, rps;    // column ranges per global / salient segment
  int32_t splits;      // kb * rpg + ks * rps
  int32_t banked;      // g = 8 bank-private tables over regions of this many chunks (2 or 4), else 0
  int32_t bregions;    // regions per column range of the banked kernel (1, or 2 with 2-chunk regions)
  int32_t lds;         // dynamic LDS bytes of one workgroup
  uint32_t range[kMaxSplits];  // range_word of every split: segment, first chunk, chunk count
  int64_t n_pad;
  size_t acc_bytes;    // workspace (splits > 1): packed reduction words
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

  if (d->layout != FLUXBIN_LAYOUT_ROWMAJOR && d->layout != FLUXBIN_LAYOUT_TILED)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "layout = %d (0 = row-major, 1 = tiled)", d->layout);
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

// Target chunks per column range: about target_blocks workgroups' worth of
// work in all (kTargetBlocks; half as many, of 8 waves, for the very wide
// single-row layers, so that the 70B down projection keeps 8-chunk ranges at 8
// waves), a workgroup of nb batch rows counting nb times, at least 2, a
// power of two, at most 8, and at most 4 for several batch rows, within cmax:
// the LDS budget, or for several batch rows at g = 4 the grouped-table limit
// (8 rows: 4-chunk ranges whose tables are built two chunks at a time, 24.3 /
// 25.0 us on the 4096 -> 11008 / 11008 -> 4096 projections against 30.4 / 32.7
// with 3-chunk ranges held whole; at g = 8 with 2 rows grouping lost, qkv
// 22.5 -> 24.3 us).  Every segment is then cut into ceil(chunks / target)
// ranges of equal length (within one chunk).  Measured on MI355X (graph of
// distinct resident weight sets, 8 / 4 waves): the 70B gate+up projection
// (8192 -> 57344, 8 waves) ran 31.2 / 29.1 / 27.2 / 28.8 / 31.5 us with 5 / 7 /
// 8 / 10 / 16-chunk ranges; the down projection (28672 -> 8192, 4 waves)
// 17.1 / 16.3 / 20.9 us with 4 / 8 / 16; the qkv projection 10.0 / 8.8 /
// 10.4 us with 2 / 4 / 8; the 4096 -> 11008 projection at 4 batch rows 15.2
// us with 4 chunks, 18.0 with 7.
int32_t auto_cpb(int32_t nb, int32_t cmax, int32_t waves, int64_t row_tiles, int32_t total_chunks, int32_t target_blocks) {
  int64_t c = (int64_t)row_tiles * total_chunks * nb / ((int64_t)waves * target_blocks);
  c = std::min<int64_t>(std::max<int64_t>(c, 2), nb > 1 ? 4 : 8);
  int64_t p = 1;
  while (p * 2 <= c) p *= 2;
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(p, cmax));
}

// Ranges of the banked g = 8 kernel (automatic plan): 2 chunks (one 2-chunk
// region, 33 KiB of LDS, four 8-wave workgroups per CU), or 4 chunks as two
// 2-chunk regions in turn (the same LDS and occupancy, half the split
// atomics) where 2-chunk ranges would make more than 64 column ranges or
// more than 1536 workgroups.  Measured on MI355X (graph of 32 distinct
// resident weight sets of the LLaMA-2-7B g = 8 layer, 8 waves, interleaved),
// one / two regions per range: gate+up (2107 workgroups) 13.09 / 12.44 us,
// down (130 ranges) 9.19 (4-chunk regions at 16 waves) / 8.81, qkv (1176)
// 9.14 / 9.21, o (392) 5.64 / 6.04.
int32_t banked_cpb(const fluxbin_layer_desc *d, int64_t row_tiles) {
  const int64_t ranges2 = d->kb * cdiv(cdiv(d->k, kChunkCols), 2) + d->ks * cdiv(cdiv(d->s, kChunkCols), 2);
  const int64_t blocks2 = cdiv(row_tiles, 8) * ranges2;
  return (ranges2 > 64 || blocks2 > 1536) ? 4 : 2;
}

// Batch rows one workgroup serves (the kernel's compiled width): the next
// power of two of max_batch, at most 16 (g = 4) or 4 (g = 8); wider batches
// run as several groups.
int32_t batch_group(int32_t g, int64_t max_batch) {
  const int64_t cap = g == 4 ? 8 : 4;
  return pow2_at_least(max_batch < cap ? max_batch : cap);
}

int entry_bytes(const fluxbin_layer_desc *d) { return d->table_precision == FLUXBIN_TABLE_F16 ? 2 : 4; }

fluxbin_status make_plan(const fluxbin_layer_desc *d, Plan *p) {
  p->row_tiles = (int32_t)cdiv(d->n, kTileRows);
  p->n_pad = (int64_t)p->row_tiles * kTileRows;
  p->total_chunks = (int32_t)(d->kb * cdiv(d->k, kChunkCols) + d->ks * cdiv(d->s, kChunkCols));
  p->nb = batch_group(d->g, d->max_batch);
  p->ks = 1;
  // one batch row at g = 4, per-row scales, over very many chunks (the 70B
  // down projection; its block-wise form is slower at 8 waves: 21.2 against
  // 20.3 us)
  const bool wide = d->g == 4 && p->nb == 1 && !d->row_group && p->total_chunks >= 256;
  if (d->waves_per_block) {
    p->waves = d->waves_per_block;
  } else {
    // eight waves (512 rows) halve the per-row share of the table build: for
    // the large g = 8 tables, for very tall layers (the 70B gate+up
    // projection, 896 row tiles: 27.2 us with 8 waves, 29.9 with 4) and, at
    // g = 4 with one batch row and per-row scales, for very wide ones (the
    // 70B down projection, 455 chunks: 15.5-15.8 us with 8 waves and 8-chunk
    // ranges, 15.9-16.0 with 4); the 70B qkv and o shapes (130 chunks, 128 -
    // 160 row tiles) are faster with 4 (qkv 8.74 against 8.91 us)
    p->waves = (d->g == 8 || p->row_tiles >= 512 || wide) ? 8 : 4;
  }
  const int32_t cmax = cpb_cap(d->g, p->nb, entry_bytes(d));
  // several batch rows build their tables in groups of chunks, so their ranges
  // may exceed what LDS holds at once (given room for two chunks)
  const bool grouped_ok = p->nb > 1 && cmax >= 2;
  if (d->chunks_per_block > (grouped_ok ? kMaxCpb : cmax))
    return fail(FLUXBIN_ERR_UNSUPPORTED, "chunks_per_block = %d exceeds %d for g = %d, max_batch = %lld, %d waves",
                d->chunks_per_block, grouped_ok ? kMaxCpb : cmax, d->g, (long long)d->max_batch, p->waves);
  // g = 8, one batch row, per-row scales, fp32 entries: bank-private tables
  const bool bank_ok = d->g == 8 && p->nb == 1 && !d->row_group && entry_bytes(d) == 4;
  int32_t target = d->chunks_per_block ? d->chunks_per_block
                   : bank_ok           ? banked_cpb(d, p->row_tiles)
                                       : auto_cpb(p->nb, grouped_ok && d->g == 4 ? kMaxCpb : cmax, p->waves, p->row_tiles,
                                              p->total_chunks, wide ? kTargetBlocks / 2 : kTargetBlocks);
  // Several waves per row tile where one wave per tile would take 2-chunk
  // ranges over more workgroups than the chip has CUs (g = 4, one batch row,
  // per-row scales, fp32 entries, 4-wave layers, automatic plan): 8-wave
  // workgroups whose ks waves per tile each look up 2 chunks of a 2 ks-chunk
  // range, so 1 / ks of the ranges, and so of the split atomics, for the same
  // waves.  Two waves per tile (256 rows, 4-chunk ranges); four (128 rows,
  // 8-chunk ranges) where the two-wave grid is a single round (at most two
  // workgroups per CU) and the four-wave one still has a workgroup for every
  // CU.  Measured on MI355X (256 resident weight sets, one graph, the
  // libraries interleaved), one / two / four waves per tile: q_proj 5.13 /
  // 5.02 / 4.92 us, the 7B 11008 -> 4096 projection at one batch row 7.65 /
  // 6.47 / 6.50, 4096 -> 11008 6.53 / 6.45 / 6.54; slower where the one-wave
  // plan has few workgroups (512 x 512: 3.50 / 3.86 with two, 8 workgroups)
  // or longer ranges (with two: the 70B qkv 8.67 / 9.45, gate+up 26.3 / 29.4).
  if (!d->chunks_per_block && !d->waves_per_block && d->g == 4 && p->nb == 1 && !d->row_group &&
      entry_bytes(d) == 4 && p->waves == 4 && target == 2 && cmax >= 8 &&
      cdiv(p->row_tiles, 4) * cdiv(p->total_chunks, 2) > kCus) {
    const bool four = cdiv(p->row_tiles, 4) * cdiv(p->total_chunks, 4) <= 2 * kCus &&
                      cdiv(p->row_tiles, 2) * cdiv(p->total_chunks, 8) >= kCus;
    p->ks = four ? 4 : 2;
    p->waves = 8;
    target = 2 * p->ks;
  }
  const int32_t nc_g = (int32_t)cdiv(d->k, kChunkCols), nc_s = d->ks > 0 ? (int32_t)cdiv(d->s, kChunkCols) : 0;
  for (;;) {
    p->rpg = (int32_t)cdiv(nc_g, target);
    p->rps = d->ks > 0 ? (int32_t)cdiv(nc_s, target) : 0;
    p->splits = d->kb * p->rpg + d->ks * p->rps;
    if (p->splits <= kMaxSplits || d->chunks_per_block || target >= (grouped_ok ? kMaxCpb : cmax)) break;
    ++target;  // automatic plan: longer ranges until the splits fit the reduction word
  }
  if (p->splits > kMaxSplits)
    return fail(FLUXBIN_ERR_UNSUPPORTED, "%d column ranges exceed %d (too many 128-column chunks for chunks_per_block %d)",
                p->splits, kMaxSplits, target);
  // the longest range (balanced cut: ceil(chunks / ranges))
  p->cpb = (int32_t)std::max<int64_t>(cdiv(nc_g, p->rpg), d->ks > 0 ? cdiv(nc_s, p->rps) : 0);
  // at g = 4 with one batch row, two chunks in flight per wave, three for
  // 4-wave workgroups over 4-chunk or longer ranges with per-row scales: with
  // 8 waves per SIMD the HBM serves fewer, earlier requests better (70B
  // gate+up 26.3 against 27.6 us with four, down at 8 waves 15.5-15.8 against
  // 16.4-16.7, the block-wise gate+up 32.5 against 33.2; one chunk is slower
  // everywhere, gate+up 27.9 against 26.4), while the 4-wave qkv and o take
  // three (8.59 / 7.78 us against 8.69 / 8.03 with two and 8.76 / 7.97 with
  // four; interleaved on one MI355X, the same order on another); two waves
  // per row tile take two at any range length
  if (d->g == 4 && p->nb == 1)
    p->pf = (p->ks == 1 && p->waves == 4 && p->cpb >= 4 && !d->row_group) ? 3 : 2;
  else
    p->pf = prefetch_depth(p->cpb);
  p->tb = p->cpb;
  if (p->cpb > cmax) {  // grouped tables: groups of tb chunks, tb a multiple of the prefetch depth
    p->pf = cmax >= 4 ? 4 : 2;
    p->tb = cmax - cmax % p->pf;
  }
  // split sp < kb * rpg is range sp % rpg of global segment sp / rpg, the rest
  // follow the same rule over the salient segments; range rr of a segment of
  // nc chunks is chunks [rr * nc / nr, (rr + 1) * nc / nr)
  for (int32_t sp = 0; sp < p->splits; ++sp) {
    const bool gpart = sp < d->kb * p->rpg;
    const int32_t rel = gpart ? sp : sp - d->kb * p->rpg;
    const int32_t nr = gpart ? p->rpg : p->rps;
    const int32_t nc = gpart ? nc_g : nc_s;
    const int32_t sg = (gpart ? 0 : d->kb) + rel / nr, rr = rel % nr;
    const int32_t lo = (int32_t)((int64_t)rr * nc / nr), hi = (int32_t)((int64_t)(rr + 1) * nc / nr);
    p->range[sp] = range_word(sg, lo, hi - lo);
  }
  // banked tables (cpb_cap keeps g = 8 fp32 ranges at <= 4 chunks): the
  // automatic plan takes 2-chunk regions, one per range or, for 3- or 4-chunk
  // ranges, two in turn; a given chunks_per_block takes one region of 2 or 4
  // chunks that holds the whole range
  p->banked = bank_ok ? (p->cpb <= 2 || !d->chunks_per_block ? 2 : 4) : 0;
  p->bregions = p->banked && p->cpb > p->banked ? 2 : 1;
  if (p->banked) p->tb = p->banked;
  // 4-chunk regions (66 KiB of LDS, two workgroups per CU) take 16 waves, so
  // that the CU still holds 32: the 7B g = 8 down projection 10.29 -> 9.00 us
  // (2-chunk regions stay at 8 waves, four workgroups per CU: qkv / o /
  // gate+up 9.07 / 5.65 / 13.04 us against 9.78 / 5.81 / 13.64 at 16)
  if (p->banked == 4 && !d->waves_per_block) p->waves = 16;
  p->row_blocks = (int32_t)cdiv(p->row_tiles, p->waves / p->ks);
  p->lds = p->banked ? banked_lds_bytes(p->banked, p->bregions) : lds_bytes(d->g, p->nb, p->tb, entry_bytes(d));
  if (p->ks > 1) p->lds += (p->ks - 1) * (p->waves / p->ks) * kTileRows * 4;  // the other waves' partials
  p->acc_bytes = p->splits > 1 ? (size_t)d->max_batch * p->n_pad * sizeof(uint64_t) : 0;
  return FLUXBIN_OK;
}

// Regions of a handle's workspace (byte offsets, each 256-B aligned): the
// split-reduction words, then, for row-major inputs, the tiled copies made by
// fluxbin_create.
struct WsLayout {
  size_t acc, bits_g, bits_s, r_g, r_s, total;
};

WsLayout ws_layout(const fluxbin_layer_desc *d, const Plan &p) {
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.acc = take(p.acc_bytes);
  if (d->layout == FLUXBIN_LAYOUT_ROWMAJOR) {
    w.bits_g = take((size_t)d->kb * fluxbin_tiled_words(d->n, d->k) * 4);
    if (d->ks > 0) w.bits_s = take((size_t)d->ks * fluxbin_tiled_words(d->n, d->s) * 4);
    if (d->row_group) {
      const int64_t groups = cdiv(d->k, d->row_group);
      w.r_g = take((size_t)d->kb * fluxbin_tiled_scale_elems(d->n, groups, 1) * 2);
      if (d->ks > 0)
        w.r_s = take((size_t)d->ks * fluxbin_tiled_scale_elems(d->n, groups, kChunkCols / d->sal_group) * 2);
    }
  }
  w.total = off;
  return w;
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

// Split-reduction words of fluxbin_gemv_static: a file-scope device array (8
// MiB), one copy per GPU the library runs on, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name
// is a stand-in, not a device address): the address each device gives for it
// (hipGetSymbolAddress, taken once per device with that device current) is
// kept in g_scratch_ptr and used instead.
constexpr int64_t kScratchWords = 1 << 20;
static __device__ __align__(256) uint64_t scratch[kScratchWords];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint64_t *g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use on that device).
fluxbin_status scratch_words(uint64_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FLUXBIN_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "locating the static scratch array");
    g_scratch_ptr[dev] = static_cast<uint64_t *>(p);
  }
  *out = g_scratch_ptr[dev];
  return FLUXBIN_OK;
}

}  // namespace

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
namespace {

template <int G, int NB>
hipError_t launch_lookup_probe(int64_t workgroups, int32_t iters, float never, float *sink, hipStream_t st) {
  constexpr int lds = NB * (kChunkCols / G) * (1 << G) * 4;
  hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void *>(lds_lookup_kernel<G, NB>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((lds_lookup_kernel<G, NB>), dim3((unsigned)workgroups), dim3(256), lds, st, iters, 0x2545f491u,
                     never, sink);
  return hipGetLastError();
}

}  // namespace

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
  *bytes = ws_layout(d, p).total;
  return ok();
}

fluxbin_status fluxbin_create(const fluxbin_layer_desc *d, fluxbin_handle *out) {
  fluxbin_status st = validate_shape(d);
  if (st) return st;
  if (!out) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!d->bits_global || !d->r_global || !d->c_global)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "global basis pointers must be non-NULL");
  const bool tiled = d->layout == FLUXBIN_LAYOUT_TILED;
  if (!aligned(d->bits_global, tiled ? 16 : 4))
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bits_global not %d-byte aligned", tiled ? 16 : 4);
  if (d->ks > 0) {
    if (!d->bits_sal || !d->r_sal || !d->c_sal || !d->sal_idx)
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "salient pointers must be non-NULL when ks > 0");
    if (!aligned(d->bits_sal, tiled ? 16 : 4))
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bits_sal not %d-byte aligned", tiled ? 16 : 4);
    if (d->row_group && tiled && !aligned(d->r_sal, 16))
      return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "r_sal not 16-byte aligned (block-wise scales)");
  }
  Plan p;
  st = make_plan(d, &p);
  if (st) return st;
  const WsLayout wl = ws_layout(d, p);
  // a tiled layer may be created without a workspace (NULL, 0 bytes): its split
  // reduction then runs only through fluxbin_gemv_static
  const bool no_ws = tiled && !d->workspace && d->workspace_bytes == 0;
  if (wl.total > 0 && !no_ws) {
    if (!d->workspace || d->workspace_bytes < wl.total)
      return fail(FLUXBIN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.total,
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
  // the description the handle keeps: row-major inputs are replaced by their
  // tiled copies in the workspace
  fluxbin_layer_desc hd = *d;
  char *ws = static_cast<char *>(d->workspace);
  if (!tiled) {
    const int64_t wpr_g = cdiv(d->k, 32), wpr_s = cdiv(d->s, 32);
    const int64_t tw_g = fluxbin_tiled_words(d->n, d->k), tw_s = d->ks > 0 ? fluxbin_tiled_words(d->n, d->s) : 0;
    uint32_t *bg = reinterpret_cast<uint32_t *>(ws + wl.bits_g);
    for (int b = 0; b < d->kb && !st; ++b)
      st = fluxbin_relayout(d->bits_global + b * d->n * wpr_g, d->n, d->k, FLUXBIN_LAYOUT_ROWMAJOR,
                            FLUXBIN_LAYOUT_TILED, bg + b * tw_g, nullptr);
    hd.bits_global = bg;
    if (d->ks > 0) {
      uint32_t *bs = reinterpret_cast<uint32_t *>(ws + wl.bits_s);
      for (int b = 0; b < d->ks && !st; ++b)
        st = fluxbin_relayout(d->bits_sal + b * d->n * wpr_s, d->n, d->s, FLUXBIN_LAYOUT_ROWMAJOR,
                              FLUXBIN_LAYOUT_TILED, bs + b * tw_s, nullptr);
      hd.bits_sal = bs;
    }
    if (d->row_group) {
      const int64_t groups = cdiv(d->k, d->row_group), m = kChunkCols / (d->ks > 0 ? d->sal_group : kChunkCols);
      const int64_t te_g = fluxbin_tiled_scale_elems(d->n, groups, 1);
      uint16_t *rg = reinterpret_cast<uint16_t *>(ws + wl.r_g);
      for (int b = 0; b < d->kb && !st; ++b)
        st = fluxbin_relayout_scales(d->r_global + b * d->n * groups, d->n, groups, 1, FLUXBIN_LAYOUT_ROWMAJOR,
                                     FLUXBIN_LAYOUT_TILED, rg + b * te_g, nullptr);
      hd.r_global = rg;
      if (d->ks > 0) {
        const int64_t te_s = fluxbin_tiled_scale_elems(d->n, groups, m);
        uint16_t *rs = reinterpret_cast<uint16_t *>(ws + wl.r_s);
        for (int b = 0; b < d->ks && !st; ++b)
          st = fluxbin_relayout_scales(d->r_sal + b * d->n * groups, d->n, groups, m, FLUXBIN_LAYOUT_ROWMAJOR,
                                       FLUXBIN_LAYOUT_TILED, rs + b * te_s, nullptr);
        hd.r_sal = rs;
      }
    }
    if (st) return st;
    hd.layout = FLUXBIN_LAYOUT_TILED;
  }
  if ((p.acc_bytes && !no_ws) || !tiled) {
    if (p.acc_bytes && !no_ws) {
      hipError_t e = hipMemset(ws + wl.acc, 0, p.acc_bytes);
      if (e != hipSuccess) return hip_fail(e, "zeroing the split-reduction words");
    }
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "synchronising after create");
  }
  gemv_fn fn = p.ks > 1 ? gemv_pick_g4_ks(p.ks, p.waves, p.pf)
               : p.banked ? gemv_pick_g8_banked(p.banked, p.bregions, p.waves)
                        : pick_gemv(d->g, d->row_group ? 1 : 0, d->table_precision, p.nb, p.waves, p.pf);
  if (!fn) return fail(FLUXBIN_ERR_UNSUPPORTED, "no kernel for g = %d, batch width %d, %d waves", d->g, p.nb, p.waves);
  const size_t lds = (size_t)p.lds;
  hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return hip_fail(e, "setting the kernel's dynamic LDS size");
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
  h->d = hd;
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
  plan->rows_per_block = p.waves / p.ks * kTileRows;
  plan->chunks_per_block = p.cpb;
  plan->row_blocks = p.row_blocks;
  plan->splits = p.splits;
  plan->total_chunks = p.total_chunks;
  plan->lds_bytes = p.lds;
  plan->grid = (int64_t)p.row_blocks * p.splits;
  plan->banked_tables = p.banked;
  plan->table_chunks = p.tb;
  plan->threads_per_block = p.waves * 64;
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

// The GEMV's launches; with events, start_event is recorded when the first
// launch begins and stop_event when the last one ends (hipExtLaunchKernel).
fluxbin_status gemv_launch(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream,
                           hipEvent_t start_event, hipEvent_t stop_event, uint64_t *words) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (batch < 0 || batch > h->d.max_batch)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "batch = %lld outside [0, %lld]", (long long)batch,
                (long long)h->d.max_batch);
  if (batch == 0) return ok();
  if (!x || !y) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (h->fault_launch) return fail(FLUXBIN_ERR_HIP, "injected launch fault (FLUXBIN_FAULT=launch)");
  const fluxbin_layer_desc &d = h->d;
  const Plan &p = h->plan;
  GemvArgs a;
  gemv_segments(d, a.seg);
  a.idx_or_dummy = h->idx_or_dummy;
  a.n = d.n;
  a.k = d.k;
  a.n_pad = p.n_pad;
  a.kb = d.kb;
  a.ks = d.ks;
  a.cpb = p.cpb;
  a.tb = p.tb;
  a.row_tiles = p.row_tiles;
  a.splits = p.splits;
  a.sal16 = d.row_group && d.ks > 0 && d.sal_group == 8 ? 1 : 0;
  memcpy(a.range, p.range, sizeof(uint32_t) * (size_t)p.splits);
  uint64_t *acc = p.splits > 1 ? words : nullptr;
  const dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);  // x: row block, y: column range
  // one launch per group of p.nb batch rows (a prefill batch runs as several groups,
  // each building its own tables and streaming the weights again)
  for (int64_t b0 = 0; b0 < batch; b0 += p.nb) {
    a.batch = (int32_t)std::min<int64_t>(p.nb, batch - b0);
    a.x = x + b0 * d.k;
    a.y = y + b0 * d.n;
    a.acc = acc ? acc + b0 * p.n_pad : nullptr;
    if (start_event || stop_event) {
      void *args[] = {&a};
      hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void *>(h->fn), grid,
                                        dim3(p.waves * 64), args, h->lds, (hipStream_t)stream,
                                        b0 == 0 ? start_event : nullptr, b0 + p.nb >= batch ? stop_event : nullptr, 0);
      if (e != hipSuccess) return hip_fail(e, "gemv launch");
    } else {
      hipLaunchKernelGGL(h->fn, grid, dim3(p.waves * 64), h->lds, (hipStream_t)stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "gemv launch");
  }
  return ok();
}

// The handle's own reduction words (its workspace), or an error when the plan
// needs them and the handle was created without a workspace.
fluxbin_status handle_words(fluxbin_handle h, uint64_t **words) {
  *words = reinterpret_cast<uint64_t *>(h->d.workspace);
  if (h->plan.splits > 1 && !*words)
    return fail(FLUXBIN_ERR_WORKSPACE,
                "the handle has no workspace (created without one): use fluxbin_gemv_static, or create it with "
                "fluxbin_workspace_size() bytes");
  return FLUXBIN_OK;
}

}  // namespace

fluxbin_status fluxbin_gemv(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  uint64_t *words;
  fluxbin_status st = handle_words(h, &words);
  if (st) return st;
  return gemv_launch(h, x, y, batch, stream, nullptr, nullptr, words);
}

fluxbin_status fluxbin_gemv_timed(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream,
                                  void *start_event, void *stop_event) {
  if (!start_event || !stop_event) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "events must be non-NULL");
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  uint64_t *words;
  fluxbin_status st = handle_words(h, &words);
  if (st) return st;
  return gemv_launch(h, x, y, batch, stream, static_cast<hipEvent_t>(start_event),
                     static_cast<hipEvent_t>(stop_event), words);
}

fluxbin_status fluxbin_gemv_static(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (batch < 0 || batch > h->d.max_batch)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "batch = %lld outside [0, %lld]", (long long)batch,
                (long long)h->d.max_batch);
  const int64_t words = h->plan.splits > 1 ? batch * h->plan.n_pad : 0;
  if (words > kScratchWords)
    return fail(FLUXBIN_ERR_UNSUPPORTED,
                "batch %lld x %lld padded rows = %lld split-reduction words exceed the %lld of the static scratch "
                "array (use fluxbin_gemv with a workspace)",
                (long long)batch, (long long)h->plan.n_pad, (long long)words, (long long)kScratchWords);
  if (batch == 0) return ok();
  if (!x || !y) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (h->fault_launch) return fail(FLUXBIN_ERR_HIP, "injected launch fault (FLUXBIN_FAULT=launch)");
  uint64_t *sw = nullptr;
  fluxbin_status st = scratch_words(&sw);
  if (st) return st;
  if (words) {
    // the array keeps the last call's contents: the words this call uses start at zero
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(words)), dim3(256), 0, (hipStream_t)stream, sw, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
  }
  return gemv_launch(h, x, y, batch, stream, nullptr, nullptr, sw);
}

fluxbin_status fluxbin_reset_workspace(fluxbin_handle h, void *stream) {
  if (!h) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (h->fault_launch) return fail(FLUXBIN_ERR_HIP, "injected launch fault (FLUXBIN_FAULT=launch)");
  const Plan &p = h->plan;
  if (!p.acc_bytes || !h->d.workspace) return ok();
  const int64_t words = (int64_t)(p.acc_bytes / sizeof(uint64_t));
  hipLaunchKernelGGL(zero_words_kernel, dim3(grid_for(words)), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<uint64_t *>(h->d.workspace), words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "workspace reset launch");
  return ok();
}

fluxbin_status fluxbin_probe_stream_read(const void *buf, int64_t bytes, int32_t depth, int64_t workgroups,
                                         uint32_t never, uint32_t *sink, void *stream) {
  if (!buf || !sink) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (bytes < 1024 || bytes % 16) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "bytes = %lld (a multiple of 16, >= 1024)",
                                              (long long)bytes);
  if (!aligned(buf, 16)) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "buf not 16-byte aligned");
  if (workgroups < 1 || workgroups > 65536)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "workgroups = %lld (1..65536)", (long long)workgroups);
  const int64_t n16 = bytes / 16, waves = workgroups * 4;
  const int64_t per_wave = cdiv(cdiv(n16, waves), 64) * 64;  // whole 1 KiB blocks per wave
  const u32x4 *b = static_cast<const u32x4 *>(buf);
  const dim3 grid((unsigned)workgroups), block(256);
  hipStream_t st = (hipStream_t)stream;
  switch (depth) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, st, b, n16, per_wave, never, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, st, b, n16, per_wave, never, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, st, b, n16, per_wave, never, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, st, b, n16, per_wave, never, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, st, b, n16, per_wave, never, sink); break;
    default: return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "depth = %d (1, 2, 4, 8 or 16)", depth);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "stream probe launch");
  return ok();
}

fluxbin_status fluxbin_probe_empty(int64_t workgroups, int32_t threads, void *stream) {
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "workgroups = %lld (1..2^20)", (long long)workgroups);
  if (threads < 1 || threads > 1024) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "threads = %d (1..1024)", threads);
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3(threads), 0, (hipStream_t)stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "empty probe launch");
  return ok();
}

fluxbin_status fluxbin_probe_lds_lookup(int32_t g, int32_t nb, int64_t workgroups, int32_t iters, float never,
                                        float *sink, void *stream) {
  if (!sink) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "sink is NULL");
  if (workgroups < 1 || workgroups > 65536 || iters < 1)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "workgroups = %lld (1..65536), iters = %d (>= 1)", (long long)workgroups,
                iters);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (g == 4 && nb == 1) e = launch_lookup_probe<4, 1>(workgroups, iters, never, sink, st);
  else if (g == 4 && nb == 2) e = launch_lookup_probe<4, 2>(workgroups, iters, never, sink, st);
  else if (g == 4 && nb == 4) e = launch_lookup_probe<4, 4>(workgroups, iters, never, sink, st);
  else if (g == 4 && nb == 8) e = launch_lookup_probe<4, 8>(workgroups, iters, never, sink, st);
  else if (g == 4 && nb == 16) e = launch_lookup_probe<4, 16>(workgroups, iters, never, sink, st);
  else if (g == 8 && nb == 1) e = launch_lookup_probe<8, 1>(workgroups, iters, never, sink, st);
  else if (g == 8 && nb == 2) e = launch_lookup_probe<8, 2>(workgroups, iters, never, sink, st);
  else if (g == 8 && nb == 4) e = launch_lookup_probe<8, 4>(workgroups, iters, never, sink, st);
  else return fail(FLUXBIN_ERR_UNSUPPORTED, "g = %d, nb = %d (g 4: nb 1, 2, 4, 8, 16; g 8: nb 1, 2, 4)", g, nb);
  if (e != hipSuccess) return hip_fail(e, "lookup probe launch");
  return ok();
}

fluxbin_status fluxbin_probe_lds_lookup_banked(int32_t region, int64_t workgroups, int32_t iters, float never,
                                               float *sink, void *stream) {
  if (!sink) return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "sink is NULL");
  if (workgroups < 1 || workgroups > 65536 || iters < 1)
    return fail(FLUXBIN_ERR_INVALID_ARGUMENT, "workgroups = %lld (1..65536), iters = %d (>= 1)", (long long)workgroups,
                iters);
  if (region != 2 && region != 4) return fail(FLUXBIN_ERR_UNSUPPORTED, "region = %d (2 or 4)", region);
  const void *fn = region == 4 ? reinterpret_cast<const void *>(lds_lookup_banked_kernel<4>)
                               : reinterpret_cast<const void *>(lds_lookup_banked_kernel<2>);
  const int lds = region * 16 * 256 * 4;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return hip_fail(e, "setting the probe's dynamic LDS size");
  const uint32_t seed = 0x2545F491u;
  if (region == 4)
    hipLaunchKernelGGL(lds_lookup_banked_kernel<4>, dim3((unsigned)workgroups), dim3(512), lds, (hipStream_t)stream,
                       iters, seed, never, sink);
  else
    hipLaunchKernelGGL(lds_lookup_banked_kernel<2>, dim3((unsigned)workgroups), dim3(512), lds, (hipStream_t)stream,
                       iters, seed, never, sink);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "banked lookup probe launch");
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
