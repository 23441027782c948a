/*
 * fluxbin.h -- C ABI of libfluxbin.so: the FluxBin LUT GEMV on MI355X (gfx950).
 *
 * The library computes, for fp16 activations x[b] (b < batch),
 *
 *   y[b] = sum_{k<Kb} r_k (.) (B_k (c_k (.) x[b]))
 *        + sum_{s<Ks} r_s (.) (B_s (c_s (.) x[b][S]))
 *
 * where (.) is the element-wise product, every B is a +-1 matrix stored as
 * packed sign bits, r are per-row and c per-column fp16 scales, and S is the
 * ordered list of salient columns.  In the block-wise format (desc.row_group
 * = 128) each r holds one scale per row per 128-column group of x, and a
 * salient column takes the scale of the group its original column lies in
 * (the storage of the FluxBin summary, appendix C.2: dense global bits with
 * column scales and block-wise row scales, plus a few salient columns per
 * group).  This is the inference form of the
 * decoupled row-column binary decomposition with salient-aware hybrid bases
 * (FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by
 * Algorithm-Kernel Synergy, paperlayer.ai summary, section 3 "Methodology",
 * bullets "Quantization" and "Salient-Aware Hybrid Bases").
 *
 * The product is evaluated without reconstructing any floating-point weight:
 * for every g-column sub-vector (g = 4 or 8) the kernel builds a table of the
 * 2^g signed sums of the scale-fused inputs c (.) x, with the column scale
 * folded into the table build; the g-bit pattern of a packed weight row is
 * the table index; lookups accumulate in fp32 registers and the row scale is
 * applied after accumulation (same summary, section 3 bullet "LUT-Based GEMV
 * Kernel" and appendix C.1; the ainews.surl.tw article on FluxBin, paragraph
 * on the execution layer).  The salient bases use the same kernel on the
 * compact columns S, with x[S] gathered at run time (Virtual Columnar
 * Mapping, same summary, section 3 bullet "Virtual Columnar Mapping").
 *
 * Conventions of every entry point
 *   - All pointers to array data are DEVICE pointers (hipMalloc or torch
 *     CUDA tensors), unless the comment says otherwise.  The caller owns all
 *     memory.  Nothing is freed by the library except handle metadata.
 *   - fp16 values are IEEE binary16 passed as raw uint16_t bits.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Launching calls
 *     are asynchronous: they enqueue work and return.
 *   - Every call returns fluxbin_status.  On an error nothing is launched,
 *     outputs are left untouched and fluxbin_last_error() holds a
 *     thread-local message.  Device faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this boundary.
 *   - fluxbin_build_lut and fluxbin_reset_workspace launch one kernel and
 *     fluxbin_gemv one kernel per group of batch rows (8 at g = 4, 4 at
 *     g = 8; one launch up to that batch); none of them ever allocates,
 *     copies, sets memory or synchronises, so they may be captured in a HIP
 *     graph.  fluxbin_create does synchronise.
 */
#ifndef FLUXBIN_H
#define FLUXBIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLUXBIN_ABI_VERSION 8

typedef enum {
  FLUXBIN_OK = 0,
  FLUXBIN_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, alignment or index list */
  FLUXBIN_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement */
  FLUXBIN_ERR_WORKSPACE = 3,        /* workspace missing or too small */
  FLUXBIN_ERR_HIP = 4               /* a HIP runtime call failed */
} fluxbin_status;

/* Sign-word layouts.
 *
 * FLUXBIN_LAYOUT_ROWMAJOR (canonical): a +-1 matrix of `rows` x `cols` is
 *   stored as uint32 words [rows][ceil(cols/32)].  Word w of row r holds
 *   column 32w+t at bit t (least significant bit first).  Bit 1 means +1 and
 *   bit 0 means -1 (the LUT Tensor Core notes, section 3.1.2, read weight
 *   bits as {-1,+1}).  Padding bits past `cols` are 0.
 *
 * FLUXBIN_LAYOUT_TILED (what fluxbin_gemv streams): rows are padded to a
 *   multiple of 64 and columns to a multiple of 128.  The canonical word
 *   (row r, word w) is stored at index
 *       ((floor(r/64) * NC + floor(w/4)) * 64 + (r mod 64)) * 4 + (w mod 4),
 *   NC = ceil(cols/128); bits inside a word keep their canonical order and
 *   padding words are 0.  One 64-row x 128-column tile is therefore 1 KiB of
 *   contiguous memory in which lane l of a wave finds the 16 bytes of row l.
 *   Size in words: fluxbin_tiled_words(rows, cols). */
typedef enum { FLUXBIN_LAYOUT_ROWMAJOR = 0, FLUXBIN_LAYOUT_TILED = 1 } fluxbin_layout;

/* Table entry types of the GEMV (fluxbin_layer_desc.table_precision). */
typedef enum {
  FLUXBIN_TABLE_F32 = 0, /* fp32 entries (the default) */
  FLUXBIN_TABLE_F16 = 1  /* fp16 entries: each entry summed in fp32, rounded to fp16 (nearest even) */
} fluxbin_table_precision;

/* Element kinds for fluxbin_vcm_gather. */
typedef enum {
  FLUXBIN_DT_I8 = 0,  /* int8 elements, [rows][cols] */
  FLUXBIN_DT_F16 = 1, /* fp16 elements, [rows][cols] */
  FLUXBIN_DT_BITS = 2 /* canonical sign words [rows][ceil(cols/32)] */
} fluxbin_dtype;

typedef struct fluxbin_layer *fluxbin_handle; /* opaque, immutable after create */

/* Description of one linear layer.  The handle keeps the pointers (it does
 * not copy the tensors): they must stay valid and unchanged for the handle's
 * lifetime.  Segments are numbered: global bases 0..kb-1, then salient bases
 * kb..kb+ks-1. */
typedef struct {
  int32_t abi_version;   /* must equal FLUXBIN_ABI_VERSION */
  int32_t g;             /* table sub-vector length: 4 or 8 */
  int32_t kb;            /* global bases, 1..4 */
  int32_t ks;            /* salient bases, 0..2 */
  int64_t n;             /* output rows, >= 1 */
  int64_t k;             /* input columns, >= 1 */
  int64_t s;             /* salient columns |S|: 0 when ks == 0, else 1..k */
  int64_t max_batch;     /* largest batch a call may pass: 1..128.  A workgroup serves up to 8 batch
                            rows (g = 8: 4); wider batches run as groups of that many rows, each
                            building its own tables and streaming the weights again */
  const uint32_t *bits_global; /* kb blocks of sign words in `layout`: TILED, fluxbin_tiled_words(n, k)
                                  words each, 16-B aligned; or ROWMAJOR, n * ceil(k/32) words each */
  const uint16_t *r_global;    /* fp16 row scales: [kb][n], or block-wise (see row_group) */
  const uint16_t *c_global;    /* fp16 [kb][k] column scales */
  const uint32_t *bits_sal;    /* ks blocks over the s compact columns, in `layout` like bits_global */
  const uint16_t *r_sal;       /* fp16 [ks][n], or block-wise (see row_group) */
  const uint16_t *c_sal;       /* fp16 [ks][s], compact order (entry c belongs to column sal_idx[c]) */
  const int32_t *sal_idx;      /* [s] salient columns, strictly ascending, in [0, k) */
  void *workspace;             /* >= fluxbin_workspace_size() bytes, 256-B aligned, caller-owned; may be NULL
                                  if that size is 0.  A TILED layer may also be created with NULL and
                                  workspace_bytes 0 whatever its size: its split reduction then runs only
                                  through fluxbin_gemv_static (fluxbin_gemv fails with
                                  FLUXBIN_ERR_WORKSPACE when the plan splits the columns) */
  size_t workspace_bytes;
  int32_t chunks_per_block;    /* tuning: 0 = automatic, else 1..32: the longest column range of one
                                  workgroup, in 128-column chunks (each segment is cut into equal ranges no
                                  longer than this).  With one batch row the range's tables must fit 80 KiB
                                  of LDS (FLUXBIN_ERR_UNSUPPORTED beyond it); with several, ranges longer
                                  than that build their tables in groups (table_chunks of the plan) */
  int32_t waves_per_block;     /* tuning: 0 = automatic, else 4 or 8 (64 output rows per wave) */
  int32_t row_group;           /* row-scale format.  0: one scale per row per basis, r_global fp16 [kb][n],
                                  r_sal fp16 [ks][n].  128: block-wise, one scale per row per basis per group
                                  of 128 columns of x; with G = ceil(k/128), r_global holds kb and r_sal ks
                                  [n][G] fp16 matrices in `layout`: TILED, blocks of
                                  fluxbin_tiled_scale_elems(n, G, 1) (global) and of
                                  fluxbin_tiled_scale_elems(n, G, 128/sal_group) (salient, 16-B aligned), see
                                  fluxbin_relayout_scales; or ROWMAJOR, n * G each.  Other values:
                                  FLUXBIN_ERR_UNSUPPORTED */
  int32_t sal_group;           /* block-wise with ks > 0: salient columns per 128-column group, 8 or 16 (a
                                  multiple of g).  S must take exactly sal_group columns from every group:
                                  s == sal_group * G and sal_idx[c] / 128 == c / sal_group (checked by
                                  fluxbin_create).  Must be 0 otherwise. */
  int32_t table_precision;     /* fluxbin_table_precision of the GEMV's tables.  FLUXBIN_TABLE_F16 stores
                                  the scale-fused tables in fp16 (quantised tables, LUT Tensor Core notes,
                                  section 3.1.3): half the LDS per table; each entry adds one fp16
                                  rounding, |error| <= 2^-11 |entry| (accumulation stays fp32) */
  int32_t layout;              /* fluxbin_layout of the sign words and of block-wise row scales.  TILED:
                                  streamed as given.  ROWMAJOR (the canonical words): fluxbin_create converts
                                  them into the workspace (fluxbin_workspace_size counts that copy), and the
                                  caller's buffers are not read again after it returns */
} fluxbin_layer_desc;

/* How a handle splits the work (read-only introspection). */
typedef struct {
  int32_t rows_per_block;   /* output rows per workgroup (64 per wave) */
  int32_t chunks_per_block; /* most 128-column chunks in one workgroup's column range */
  int32_t row_blocks;       /* workgroups along the rows */
  int32_t splits;           /* column ranges: every segment is cut into ranges of consecutive chunks of
                               equal length (within one chunk), none longer than chunks_per_block */
  int32_t total_chunks;     /* sum over segments of ceil(len/128) */
  int32_t lds_bytes;        /* LDS per workgroup at max_batch */
  int64_t grid;             /* workgroups per fluxbin_gemv launch (per group of batch rows) */
  int32_t banked_tables;    /* 0: each sub-vector's table in consecutive dwords, one row per lane; 2 or 4
                               (g = 8, one batch row, per-row scales, fp32 entries): bank-private tables,
                               each a column of the LDS, over regions of that many chunks (a column
                               range of up to chunks_per_block chunks is one region, or two 2-chunk
                               regions in turn) */
  int32_t table_chunks;     /* chunks whose tables a workgroup holds in LDS at once: chunks_per_block, or
                               fewer (several batch rows; two-region banked ranges), the tables then built
                               in groups of this many chunks in turn while the range's sign words stream */
  int32_t threads_per_block; /* threads of one workgroup: 64 per row tile of rows_per_block, or 128 / 256 where
                               two / four waves share each row tile, each over one part of the column range
                               (g = 4, one batch row, layers whose ranges would otherwise be 2 chunks long) */
} fluxbin_plan;

int32_t fluxbin_abi_version(void);
const char *fluxbin_status_string(fluxbin_status s);
/* Thread-local description of the last error returned on this thread. */
const char *fluxbin_last_error(void);

/* Words of the TILED layout for a rows x cols sign matrix (host-side arithmetic). */
int64_t fluxbin_tiled_words(int64_t rows, int64_t cols);

/* Pack int8 signs [rows][ld] (first `cols` of each row used) into sign words
 * in `layout`.  +1 sets a bit, -1 clears it.  Any other value is packed as a
 * cleared bit and, when `invalid_count` (device uint32, caller-zeroed) is not
 * NULL, adds 1 to it per such value.  `packed` must hold
 * rows*ceil(cols/32) words (ROWMAJOR) or fluxbin_tiled_words(rows, cols)
 * words (TILED); every word, padding included, is written.
 * Bit order and sign meaning: see fluxbin_layout (the ainews.surl.tw article
 * on FluxBin: weights streamed as compressed 32-bit words). */
fluxbin_status fluxbin_pack(const int8_t *signs, int64_t rows, int64_t cols, int64_t ld, int32_t layout,
                            uint32_t *packed, uint32_t *invalid_count, void *stream);

/* Convert sign words of a rows x cols matrix between layouts (ROWMAJOR <->
 * TILED, or a copy when they are equal).  src and dst must not overlap. */
fluxbin_status fluxbin_relayout(const uint32_t *src, int64_t rows, int64_t cols, int32_t src_layout,
                                int32_t dst_layout, uint32_t *dst, void *stream);

/* Elements of the TILED scale layout for a rows x groups fp16 matrix of
 * block-wise row scales, groups_per_chunk (1..128) groups to a 128-column
 * chunk (host-side arithmetic; 0 for invalid sizes). */
int64_t fluxbin_tiled_scale_elems(int64_t rows, int64_t groups, int64_t groups_per_chunk);

/* Convert block-wise row scales between the row-major [rows][groups] fp16
 * matrix (FLUXBIN_LAYOUT_ROWMAJOR) and the TILED scale layout, or copy.
 * TILED: rows padded to a multiple of 64, groups to a multiple of m =
 * groups_per_chunk; element (row r, group q) at
 *     ((floor(r/64) * NC + floor(q/m)) * 64 + (r mod 64)) * m + (q mod m),
 * NC = ceil(groups/m), padding 0.  The m scales one row needs for one
 * 128-column chunk are contiguous, and those of a 64-row tile form one
 * block, which fluxbin_gemv streams beside the tile's sign words.  Global
 * bases use m = 1, salient bases m = 128 / sal_group.  src and dst must not
 * overlap; every destination element, padding included, is written. */
fluxbin_status fluxbin_relayout_scales(const uint16_t *src, int64_t rows, int64_t groups, int64_t groups_per_chunk,
                                       int32_t src_layout, int32_t dst_layout, uint16_t *dst, void *stream);

/* Virtual Columnar Mapping gather (FluxBin summary, section 3 bullet "Virtual
 * Columnar Mapping"): dst column c = src column idx[c], for c < s, of a
 * [rows][cols] source.  DT_I8 / DT_F16: element matrices, dst [rows][s].
 * DT_BITS: canonical sign words, src [rows][ceil(cols/32)], dst
 * [rows][ceil(s/32)] with zero padding bits.  idx entries must lie in
 * [0, cols) (checked on the device: out-of-range entries gather 0 / -1).
 * Used offline to build the compact salient bases and scales; fluxbin_gemv
 * gathers x[S] itself. */
fluxbin_status fluxbin_vcm_gather(const int32_t *idx, int64_t s, const void *src, int64_t rows, int64_t cols,
                                  int32_t dtype, void *dst, void *stream);

/* Workspace bytes a layer needs (host-side arithmetic, no device access): the
 * split-reduction words, max_batch * ceil(n/64)*64 packed 64-bit words when the
 * plan cuts a row's columns into several ranges (fluxbin_plan.splits > 1,
 * zeroed by fluxbin_create and left zero by every completed call), then, when
 * desc.layout is ROWMAJOR, the TILED copies fluxbin_create makes of the sign
 * words (and of block-wise row scales), each region 256-B aligned. */
fluxbin_status fluxbin_workspace_size(const fluxbin_layer_desc *d, size_t *bytes);

/* Validate the description (copies sal_idx to the host to check it), convert
 * ROWMAJOR sign words and block-wise scales into the workspace, zero the
 * split-reduction words, and return a handle.  Synchronises the device; not
 * capturable.  The environment variable FLUXBIN_FAULT=launch,
 * read here, makes every launching call of this handle fail with
 * FLUXBIN_ERR_HIP before launching (error-path testing). */
fluxbin_status fluxbin_create(const fluxbin_layer_desc *d, fluxbin_handle *out);
fluxbin_status fluxbin_destroy(fluxbin_handle h);
fluxbin_status fluxbin_get_plan(fluxbin_handle h, fluxbin_plan *plan);

/* The plan fluxbin_create would choose for d (host-side arithmetic on the
 * shape fields, no device access; pointers are not examined), for capacity
 * planning and tests.  Fails like fluxbin_workspace_size on an invalid or
 * unsupported shape. */
fluxbin_status fluxbin_plan_of(const fluxbin_layer_desc *d, fluxbin_plan *plan);

/* Floats fluxbin_build_lut writes for `batch` rows:
 * batch * (kb*ceil(k/g) + ks*ceil(s/g)) * 2^(g-1). */
fluxbin_status fluxbin_lut_size(fluxbin_handle h, int64_t batch, size_t *floats);

/* Scale-fused half tables (FluxBin summary, section 3 bullet "LUT-Based GEMV
 * Kernel" and appendix C.1; halving by the symmetry LUT[~p] = -LUT[p] of the
 * LUT Tensor Core notes, section 3.1.2).  x: fp16 [batch][k].  lut: float
 * [batch][segment][ceil(L/g)][2^(g-1)] with segments in handle order and L
 * the segment's width (k or s).  Entry q of sub-vector j is the table value
 * for pattern q | 2^(g-1):  v_{g-1} + sum_{t<g-1} (2*bit_t(q) - 1) * v_t,
 * v_t = c[jg+t] * x[jg+t] (global) or c_s[jg+t] * x[S[jg+t]] (salient),
 * v_t = 0 past L.  fluxbin_gemv builds the same tables itself, in LDS; this
 * call exposes them. */
fluxbin_status fluxbin_build_lut(fluxbin_handle h, const uint16_t *x, int64_t batch, float *lut, void *stream);

/* y = the layer applied to x.  x: fp16 [batch][k], y: fp16 [batch][n]
 * (round to nearest even), 0 <= batch <= max_batch (0 launches nothing).
 * Tables and accumulation are fp32 (or fp16 tables, see table_precision).
 * Each workgroup sums one column range of one segment; a per-row scale
 * multiplies that range's accumulated sum, block-wise scales multiply the sum
 * of each global chunk (one group) and of each 8 salient columns (one group,
 * or half of one when sal_group = 16), before those sums are added.  When the
 * plan cuts the columns into several ranges (fluxbin_plan.splits > 1), the
 * partial sums of a row are combined exactly as fixed-point integers: each
 * partial is rounded to a multiple of 2^-29 (an error of at most 2^-30); a
 * partial of magnitude 2^17 or more (or a non-finite one) cannot be
 * represented, and its row is then written as NaN, never as a wrong finite
 * number.  Uses the handle's workspace: at most one call per handle may be in
 * flight at a time (use one handle per concurrent stream).  For a given
 * handle the result of row b does not depend on the other rows of the batch,
 * and repeated calls give bitwise identical y. */
fluxbin_status fluxbin_gemv(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream);

/* fluxbin_gemv for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation), and
 * for handles created without a workspace: the split-reduction words live in
 * a static device array of the library (8 MiB: 2^20 64-bit words, one copy per
 * GPU, held until the process ends) instead of the handle's workspace.  The
 * words this call uses (batch * ceil(n/64)*64 when the plan splits the
 * columns) are cleared by a fill kernel on `stream` first, then the GEMV runs
 * as in fluxbin_gemv, with the same arithmetic (bitwise the same y).  Errors:
 * FLUXBIN_ERR_UNSUPPORTED when those words exceed 2^20.  Allocates nothing
 * (no hipMalloc or allocating library call); the array's device address is
 * looked up once per device, on the first call there.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (concurrent streams,
 * threads) race and must be serialised by the caller. */
fluxbin_status fluxbin_gemv_static(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream);

/* fluxbin_gemv, and the device time of its kernels: start_event (a
 * hipEvent_t) is recorded when its first kernel starts and stop_event when
 * its last kernel ends (hipExtLaunchKernel), so hipEventElapsedTime gives the
 * kernels' own duration without the launch gaps around them.  For
 * measurement; not capturable in a HIP graph (events). */
fluxbin_status fluxbin_gemv_timed(fluxbin_handle h, const uint16_t *x, uint16_t *y, int64_t batch, void *stream,
                                  void *start_event, void *stop_event);

/* Zero the handle's split-reduction words (the workspace's first region,
 * max_batch * ceil(n/64)*64 64-bit words) with a fill kernel on `stream`.
 * Every completed fluxbin_gemv leaves them zero; a call that did not complete
 * (a device fault, an aborted stream) can leave them dirty, and this restores
 * them.  Nothing is launched when the plan has no split reduction.  Allocates
 * nothing and synchronises nothing (capturable); it must not overlap a
 * fluxbin_gemv on the same handle. */
fluxbin_status fluxbin_reset_workspace(fluxbin_handle h, void *stream);

/* Context kernel, not part of the method: dense fp16 y = W x with fp32
 * accumulation.  w: fp16 [n][k] row-major (16-B aligned, k a multiple of 8),
 * x: fp16 [batch][k], y: fp16 [batch][n], 1 <= batch <= 16. */
fluxbin_status fluxbin_dense_gemv_f16(const uint16_t *w, int64_t n, int64_t k, const uint16_t *x, uint16_t *y,
                                      int64_t batch, void *stream);

/* ------------------------------------------------------------------------
 * Measurement kernels, not part of the method: the device's own rooflines for
 * the GEMV's access and instruction patterns.  Each launches one kernel and
 * allocates nothing.
 * ------------------------------------------------------------------------ */

/* Read `bytes` (a multiple of 16, >= 1024) at `buf` (16-B aligned) with
 * non-temporal 16-byte loads: the buffer is cut into one contiguous span per
 * wave of `workgroups` x 4 waves, and each wave reads its span in 1 KiB
 * blocks (64 lanes x 16 bytes), `depth` (1, 2, 4, 8 or 16) loads in flight.
 * sink: uint32 [workgroups * 256], written only in the practically
 * impossible case that a lane's XOR of everything it read equals `never`. */
fluxbin_status fluxbin_probe_stream_read(const void *buf, int64_t bytes, int32_t depth, int64_t workgroups,
                                         uint32_t never, uint32_t *sink, void *stream);

/* An empty kernel of `workgroups` x `threads` (1..1024) threads: the cost of a
 * launch of that grid. */
fluxbin_status fluxbin_probe_empty(int64_t workgroups, int32_t threads, void *stream);

/* The GEMV's table lookups alone: every lane of `workgroups` x 256 threads
 * holds 16 bytes of pseudo-random sign words and looks them up `iters` times
 * in the tables of nb batch rows (g = 4: nb in 1, 2, 4, 8, 16; g = 8: 1, 2,
 * 4), with the same address, LDS-read and fp32-add instructions as
 * fluxbin_gemv; per call 64 * 4 * workgroups * iters * nb * 128 / g lookups.
 * sink: float [workgroups * 256], written only if a lane's sum equals
 * `never`. */
fluxbin_status fluxbin_probe_lds_lookup(int32_t g, int32_t nb, int64_t workgroups, int32_t iters, float never,
                                        float *sink, void *stream);

/* The same for the g = 8 bank-private tables of one batch row (the lookups of
 * the banked GEMV kernel: each lane's sub-vector order rotated by its row, one
 * v_perm_b32 per address, one fp32 add per lookup) over a region of `region`
 * (2 or 4) chunks: `workgroups` workgroups of 512 threads with region * 16 KiB
 * of LDS, each lane looking up region groups of 16 bytes `iters` times.
 * sink: float [workgroups * 512], written only if a lane's sum equals `never`.
 * FLUXBIN_ERR_UNSUPPORTED for another region. */
fluxbin_status fluxbin_probe_lds_lookup_banked(int32_t region, int64_t workgroups, int32_t iters, float never,
                                               float *sink, void *stream);

/* ------------------------------------------------------------------------
 * Offline decomposition W ~ sum_{b<kb} diag(r_b) B_b diag(c_b), the step that
 * produces the bases the GEMV streams (FluxBin summary, section 3 bullets
 * "Quantization" and "Parameter Optimization", appendices A.1 and A.2).
 *
 * Minimises E = sum_ij d_j (W_ij - W_hat_ij)^2 (weighted least squares with
 * per-column weights d, NULL = all 1) by alternating exact minimisations:
 *   row step (basis b):    r_b,i = sum_j d_j R_ij B_b,ij c_b,j / sum_j d_j c_b,j^2
 *   column step (basis b): c_b,j = sum_i R_ij B_b,ij r_b,i / sum_i r_b,i^2
 *     with R = W - sum_{l != b} diag(r_l) B_l diag(c_l); a zero denominator
 *     gives 0;
 *   sign step: every element takes the sign combination m in [0, 2^kb) (bit b
 *     of m set = +1 on basis b) minimising |W_ij - sum_b (+-) r_b,i c_b,j|,
 *     the sum taken in basis order in fp64 with each product rounded once;
 *     ties go to the smallest m (an exhaustive search, globally optimal for
 *     fixed scales).
 * fluxbin_decompose: initialise basis b = 0..kb-1 in order (signs of the
 * residual of the bases before it, R >= 0 -> +1; c_b = 1; one row step, one
 * column step), run `iters` iterations (row then column step of every basis,
 * then the sign step), round the scales to fp16 (nearest even), and end with
 * a sign step against the rounded scales.  The Hessian-guided parts of the
 * pages' pipeline (error compensation, saliency search) are not here.
 *
 * Layouts (all device memory): W fp16 [n][k] row-major; bits canonical sign
 * words [kb][n][ceil(k/32)] (FLUXBIN_LAYOUT_ROWMAJOR per basis); r fp64
 * [kb][n]; c fp64 [kb][k]; col_weight fp64 [k] or NULL.  1 <= kb <= 4,
 * 1 <= n <= 2^22, 1 <= k <= 2^30.  Working scales are fp64; sums over a row
 * or a column are split over lanes and workgroups in a fixed order (repeated
 * calls give identical results).  workspace: 256-B aligned,
 * fluxbin_decomp_workspace_size() bytes; one call at a time per workspace.
 * ------------------------------------------------------------------------ */
fluxbin_status fluxbin_decomp_workspace_size(int64_t n, int64_t k, int32_t kb, size_t *bytes);

/* The whole decomposition.  Outputs bits [kb][n][ceil(k/32)], r16 [kb][n],
 * c16 [kb][k] (fp16), r64/c64 (the fp64 scales before rounding), and, if
 * trace != NULL, 2 + iters * (2 kb + 1) fp64 errors E: after the
 * initialisation, after every row, column and sign step of every iteration,
 * and after the rounding and its sign step. */
fluxbin_status fluxbin_decompose(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t iters,
                                 const double *col_weight, uint32_t *bits, uint16_t *r16, uint16_t *c16, double *r64,
                                 double *c64, double *trace, void *workspace, size_t workspace_bytes, void *stream);

/* Single steps (the same kernels fluxbin_decompose runs).  The row step
 * writes r_out [n] for basis `basis` (it reads the other bases' row scales
 * only, so r_out may be r + basis * n); the column step writes c_out [k]
 * likewise; the sign step writes all kb bases of bits_out; the residual-sign
 * step writes basis_bits_out [n][ceil(k/32)] (+1 where W minus the other bases
 * is >= 0); the error step writes E to err_out[0]. */
fluxbin_status fluxbin_decomp_row_scales(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                         const uint32_t *bits, const double *r, const double *c,
                                         const double *col_weight, double *r_out, void *workspace,
                                         size_t workspace_bytes, void *stream);
fluxbin_status fluxbin_decomp_col_scales(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                         const uint32_t *bits, const double *r, const double *c, double *c_out,
                                         void *workspace, size_t workspace_bytes, void *stream);
fluxbin_status fluxbin_decomp_signs(const uint16_t *w, int64_t n, int64_t k, int32_t kb, const double *r,
                                    const double *c, uint32_t *bits_out, void *stream);
fluxbin_status fluxbin_decomp_residual_signs(const uint16_t *w, int64_t n, int64_t k, int32_t kb, int32_t basis,
                                             const uint32_t *bits, const double *r, const double *c,
                                             uint32_t *basis_bits_out, void *stream);
fluxbin_status fluxbin_decomp_error(const uint16_t *w, int64_t n, int64_t k, int32_t kb, const uint32_t *bits,
                                    const double *r, const double *c, const double *col_weight, double *err_out,
                                    void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUXBIN_H */
