// q4_0 / q8_0 weights x Q8_1 activations (integer dot).
#include "gemv_instances.h"

namespace skg {
void register_gemv_q8_1(std::vector<GemvEntry>& out) {
  // The first instance of each (format, M, epilogue) is its default, chosen
  // by measurement on MI355X under cold-cache rotation (K = 4096 and 11008).
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 2, 1, 4, SKG_EPI_SWIGLU, 2)
  SKG_IK(SKG_Q8_0_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_M12(SKG_Q4_0_Q8_1, 8, 2, 8, 1, 4, 4)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 8, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 4)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 2, 1, 4, SKG_EPI_NONE, 4)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 2, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 1, 4, SKG_EPI_SWIGLU, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 2, 1, 4, SKG_EPI_SWIGLU, 4)
  SKG_M3_8(SKG_Q4_0_Q8_1, 4, 1, false, 2)
  SKG_M12(SKG_Q8_0_Q8_1, 4, 2, 4, 1, 2, 2)
  SKG_M3_8(SKG_Q8_0_Q8_1, 4, 1, false, 2)
  SKG_I(SKG_Q4_0_Q8_1, 1, 4, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 16, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 8, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 16, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 4, 6, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 8, 6, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 8, 2, false, 8, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 1, 2, 2, false, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_0_Q8_1, 1, 8, 2, false, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q8_0_Q8_1, 1, 8, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_Q8_1, 1, 2, 2, false, 4, SKG_EPI_NONE)
}
}  // namespace skg
