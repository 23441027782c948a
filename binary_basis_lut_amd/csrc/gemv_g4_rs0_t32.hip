// gemv_g4_rs0_t32.hip -- LUT GEMV kernel instances for g = 4, per-row row scales,
// fp32 table entries.
#include "gemv_kernel.hpp"

namespace fluxbin {

gemv_fn gemv_pick_g4_rs0_t32(int nb, int waves, int pf) { return gemv_pick<4, 0, 0>(nb, waves, pf); }

gemv_fn gemv_pick_g4_ks(int ks, int waves, int pf) {
  if (waves != 8 || pf != 2) return nullptr;
  return ks == 2 ? lut_gemv_ks2_kernel<4, 8, 2, 0, 0> : ks == 4 ? lut_gemv_ks4_kernel<4, 8, 2, 0, 0> : nullptr;
}

}  // namespace fluxbin
