// gemv_g8_banked.hip -- instances of the g = 8 bank-private-table GEMV kernel.
#include "gemv_banked.hpp"

namespace fluxbin {

gemv_fn gemv_pick_g8_banked(int region, int waves) {
  return region == 4 ? gemv_pick_banked_waves<4>(waves) : region == 2 ? gemv_pick_banked_waves<2>(waves) : nullptr;
}

}  // namespace fluxbin
