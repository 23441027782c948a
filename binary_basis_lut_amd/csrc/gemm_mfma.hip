// gemm_mfma.hip -- instances of the matrix-core layer product, the choice of
// instance per call and the automatic range length.
#include "gemm_mfma.hpp"

namespace fluxbin {

namespace {

// Automatic range length: 8 chunks for handles of at most 64 batch rows, 16
// above, doubled while at least kMfmaPlentyBlocks 128-row blocks times
// ranges remain (very tall layers: fewer partial sums to store and add).
// Measured on MI355X on the 7B shapes (4, 8, 16, 32 chunks): q_proj 4096x4096
// at b = 32 / 64 / 128 best or level with 8 / 8 / 8-16 chunks (17.5 / 21.9 /
// 29.5 us), 4096 -> 11008 with 8 / 8 / 16 (21.4 / 30.5 / 51.8 us; 33.0 at
// b = 64 with 16), 11008 -> 4096 within 10 % of its best (23.2 / 31.8 / 50.9
// us with 16 / 16 / 32).
constexpr int64_t kMfmaPlentyBlocks = 2048;

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

}  // namespace

MfmaInstance mfma_instance(int64_t batch, int rs) {
  if (batch < 1 || batch > 32 * kMfmaMaxBlocks) return {nullptr, 0, 0, 0};
  // One instance for every batch: a wave multiplies 64 weight rows by 32 batch rows, a workgroup
  // 256 by 32, and wider batches run as more workgroups along the batch.  Instances that stage 64
  // or 128 batch rows per workgroup expand each weight bit for more batch rows but give fewer
  // workgroups and waves to hide the staging; measured on MI355X they were slower or level at
  // every batch of 32..128 rows (q_proj 4096x4096 at b = 96 / 128: 23.7 / 29.6 us against
  // 37.9 / 39.6 us; 11008 -> 4096 at b = 128: 51.9 against 58.4 us; block-wise s8 at b = 128:
  // q_proj 66.8 against 75.6 us, 11008 -> 4096 139 against 205 us).
  static_assert(kMfmaRowsPerBlock == kMfmaWaves * 32 * 2, "rows per workgroup of the instance");
  if (rs == 0) return {gemm_mfma_kernel<1, 1, 2, 0>, 1, 1, 2};
  return {gemm_mfma_kernel<1, 1, 2, 1>, 1, 1, 2};
}

int32_t mfma_auto_cpb(int32_t row_blocks, int32_t kb, int32_t nc_g, int32_t ks, int32_t nc_s, int64_t max_batch) {
  auto splits = [&](int32_t c) { return kb * ceil_div(nc_g, c) + ks * (nc_s ? ceil_div(nc_s, c) : 0); };
  int32_t cpb = max_batch > 64 ? 16 : 8;
  while (cpb < kMaxCpb && (int64_t)row_blocks * splits(cpb * 2) >= kMfmaPlentyBlocks) cpb *= 2;
  return cpb;
}

}  // namespace fluxbin
