/* A plain C11 consumer of include/fluxbin.h: compiled with gcc against
 * libfluxbin.so by tests/test_c_abi.py.  It calls only the entry points that
 * do host work (no device memory, no kernel), so it runs without a GPU: the
 * version, a plan and a workspace size for a known layer shape, and the error
 * path.  Prints one line per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "fluxbin.h"

static int fails = 0;

static void check(int ok, const char *what) {
  printf("%s %s\n", ok ? "ok" : "FAIL", what);
  if (!ok) ++fails;
}

int main(void) {
  check(fluxbin_abi_version() == FLUXBIN_ABI_VERSION, "abi version matches the header");

  /* a 8192 -> 57344 layer: two global bases and one salient basis on 256
     columns, g = 4, one batch row, tiled words, automatic plan */
  fluxbin_layer_desc d;
  memset(&d, 0, sizeof d);
  d.abi_version = FLUXBIN_ABI_VERSION;
  d.g = 4;
  d.kb = 2;
  d.ks = 1;
  d.n = 57344;
  d.k = 8192;
  d.s = 256;
  d.max_batch = 1;
  d.layout = FLUXBIN_LAYOUT_TILED;
  d.table_precision = FLUXBIN_TABLE_F32;

  fluxbin_plan p;
  fluxbin_status st = fluxbin_plan_of(&d, &p);
  check(st == FLUXBIN_OK, "plan_of accepts the layer");
  printf("plan: rows_per_block %d chunks_per_block %d row_blocks %d splits %d total_chunks %d grid %lld "
         "threads_per_block %d\n",
         p.rows_per_block, p.chunks_per_block, p.row_blocks, p.splits, p.total_chunks, (long long)p.grid,
         p.threads_per_block);
  check(p.total_chunks == 2 * 64 + 2, "chunks: 64 per global basis, 2 for the salient one");
  check(p.grid == (int64_t)p.row_blocks * p.splits, "grid = row blocks x splits");
  check(p.row_blocks * p.rows_per_block >= 57344, "the row blocks cover every row");

  size_t ws = 0;
  st = fluxbin_workspace_size(&d, &ws);
  check(st == FLUXBIN_OK, "workspace_size accepts the layer");
  printf("workspace bytes %zu\n", ws);
  check(p.splits == 1 ? ws == 0 : ws == (size_t)57344 * 8, "one 64-bit reduction word per row when split");

  check(fluxbin_tiled_words(64, 128) == 64 * 4, "tiled words of one 64-row, 128-column tile");

  d.g = 5;
  st = fluxbin_plan_of(&d, &p);
  check(st == FLUXBIN_ERR_UNSUPPORTED, "g = 5 is rejected as unsupported");
  check(strlen(fluxbin_last_error()) > 0, "the error carries a message");
  check(strlen(fluxbin_status_string(st)) > 0, "the status has a name");
  printf("last error: %s\n", fluxbin_last_error());

  return fails ? 1 : 0;
}
