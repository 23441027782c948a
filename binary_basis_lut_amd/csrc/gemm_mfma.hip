// gemm_mfma.hip -- instances of the matrix-core layer product, the choice of
// instance per call and the automatic range length.
#include "gemm_mfma.hpp"

namespace fluxbin {

namespace {

// Automatic range length: 8 chunks for handles of at most 32 batch rows, 16
// above, doubled while the grid keeps at least kMfmaPlentyBlocks workgroups of
// 128 rows (very tall layers: fewer partial sums to store and add).  Measured
// on MI355X on the 7B shapes: q_proj 4096x4096 17.5 / 39.6 us at b = 32 / 128
// with 8 / 16 chunks (20.2 / 58.3 with 4, 32.5 / 50.3 with 32); the MLP
// projections within 5 % of their best.
constexpr int64_t kMfmaPlentyBlocks = 2048;

int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

}  // namespace

MfmaInstance mfma_instance(int64_t batch, int rs) {
  if (batch < 1 || batch > 32 * kMfmaMaxBlocks) return {nullptr, 0, 0, 0};
  if (rs == 0) {
    if (batch <= 32) return {gemm_mfma_kernel<1, 1, 2, 0>, 1, 1, 2};
    // 32 weight rows per wave here: twice the workgroups of 64 (q_proj 4096x4096 at b = 64:
    // 23.5 against 28.2 us; the MLP projections within 3 %)
    if (batch <= 64) return {gemm_mfma_kernel<2, 1, 1, 0>, 2, 1, 1};
    return {gemm_mfma_kernel<2, 2, 2, 0>, 2, 2, 2};
  }
  // block-wise scales fold per group into a second accumulator set: one batch block per wave, so
  // that two waves per SIMD fit; wider batches take more waves along the batch
  if (batch <= 32) return {gemm_mfma_kernel<1, 1, 2, 1>, 1, 1, 2};
  if (batch <= 64) return {gemm_mfma_kernel<1, 2, 2, 1>, 1, 2, 2};
  return {gemm_mfma_kernel<1, 4, 2, 1>, 1, 4, 2};
}

int32_t mfma_auto_cpb(int32_t row_blocks, int32_t kb, int32_t nc_g, int32_t ks, int32_t nc_s, int64_t max_batch) {
  auto splits = [&](int32_t c) { return kb * ceil_div(nc_g, c) + ks * (nc_s ? ceil_div(nc_s, c) : 0); };
  int32_t cpb = max_batch > 32 ? 16 : 8;
  while (cpb < kMaxCpb && (int64_t)row_blocks * splits(cpb * 2) >= kMfmaPlentyBlocks) cpb *= 2;
  return cpb;
}

}  // namespace fluxbin
