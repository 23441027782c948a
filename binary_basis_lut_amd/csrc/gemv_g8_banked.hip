// gemv_g8_banked.hip -- instances of the g = 8 bank-private-table GEMV kernel.
#include "gemv_banked.hpp"

namespace fluxbin {

gemv_fn gemv_pick_g8_banked(int region, int regions, int waves) {
  if (regions == 2) return region == 2 ? gemv_pick_banked_waves<2, 2>(waves) : nullptr;
  if (regions != 1) return nullptr;
  return region == 4 ? gemv_pick_banked_waves<4, 1>(waves) : region == 2 ? gemv_pick_banked_waves<2, 1>(waves) : nullptr;
}

}  // namespace fluxbin
