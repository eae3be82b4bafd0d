// q8_0 weights x fp32 activations, M = 3..8 (activation staged in LDS).
#include "gemv_instances.h"

namespace skg {
void register_gemv_q8_0_f32_m38(std::vector<GemvEntry>& out) {
  SKG_M3_8(SKG_Q8_0_F32, 4, 1, true, 2)
  SKG_I(SKG_Q8_0_F32, 4, 8, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 8, 8, 1, true, 4, SKG_EPI_NONE)
}
}  // namespace skg
