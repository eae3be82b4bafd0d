// q4_0 weights x fp32 activations, M = 3..5 (activation staged in LDS).
#include "gemv_instances.h"

namespace skg {
void register_gemv_q4_0_f32_m35(std::vector<GemvEntry>& out) {
  SKG_M(SKG_Q4_0_F32, 3, 8, 1, true, 4)
  SKG_M(SKG_Q4_0_F32, 4, 8, 1, true, 4)
  SKG_M(SKG_Q4_0_F32, 5, 8, 1, true, 4)
}
}  // namespace skg
