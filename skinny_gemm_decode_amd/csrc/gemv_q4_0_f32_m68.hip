// q4_0 weights x fp32 activations, M = 6..8 (activation staged in LDS).
#include "gemv_instances.h"

namespace skg {
void register_gemv_q4_0_f32_m68(std::vector<GemvEntry>& out) {
  SKG_M(SKG_Q4_0_F32, 6, 8, 1, true, 4)
  SKG_M(SKG_Q4_0_F32, 7, 8, 1, true, 4)
  SKG_M(SKG_Q4_0_F32, 8, 8, 1, true, 4)
  SKG_I(SKG_Q4_0_F32, 8, 4, 1, true, 4, SKG_EPI_NONE)
}
}  // namespace skg
