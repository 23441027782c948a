// gemm_mfma.hip -- instances of the matrix-core layer product: NBT batch
// blocks of 32 rows per wave, WB waves along the batch, per-row or block-wise
// row scales.
#include "gemm_mfma.hpp"

namespace fluxbin {

mfma_fn mfma_pick(int nbt, int wb, int rs) {
  if (rs == 0) {
    if (nbt == 1 && wb == 1) return gemm_mfma_kernel<1, 1, 0>;
    if (nbt == 2 && wb == 1) return gemm_mfma_kernel<2, 1, 0>;
    if (nbt == 2 && wb == 2) return gemm_mfma_kernel<2, 2, 0>;
  } else if (rs == 1) {
    if (nbt == 1 && wb == 1) return gemm_mfma_kernel<1, 1, 1>;
    if (nbt == 2 && wb == 1) return gemm_mfma_kernel<2, 1, 1>;
    if (nbt == 2 && wb == 2) return gemm_mfma_kernel<2, 2, 1>;
  }
  return nullptr;
}

}  // namespace fluxbin
