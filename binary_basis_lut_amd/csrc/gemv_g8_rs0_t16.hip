// gemv_g8_rs0_t16.hip -- LUT GEMV kernel instances for g = 8, per-row row scales,
// fp16 table entries.
#include "gemv_kernel.hpp"

namespace fluxbin {

gemv_fn gemv_pick_g8_rs0_t16(int nb, int waves, int pf) { return gemv_pick<8, 0, 1>(nb, waves, pf); }

}  // namespace fluxbin
