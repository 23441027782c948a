// gemv_g4_rs1_t16.hip -- LUT GEMV kernel instances for g = 4, block-wise row scales,
// fp16 table entries.
#include "gemv_kernel.hpp"

namespace fluxbin {

gemv_fn gemv_pick_g4_rs1_t16(int nb, int waves, int pf) { return gemv_pick<4, 1, 1>(nb, waves, pf); }

}  // namespace fluxbin
