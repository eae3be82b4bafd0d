// q4_0 / q8_0 weights x fp32 activations quantised to Q8_1 inside the kernel
// (integer dot).  The instances mirror the Q8_1 ones variant for variant, so
// for every (M, epilogue) the default accumulates in the same order as the
// standalone quantiser followed by the Q8_1 GEMV, and the two agree bit for
// bit.
#include "gemv_instances.h"

namespace skg {
void register_gemv_q8_1f(std::vector<GemvEntry>& out) {
  SKG_IK(SKG_Q4_0_Q8_1F, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_Q8_1F, 1, 2, 1, 4, SKG_EPI_SWIGLU, 2)
  SKG_IK(SKG_Q8_0_Q8_1F, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_M12(SKG_Q4_0_Q8_1F, 8, 2, 8, 1, 4, 4)
  SKG_M3_8(SKG_Q4_0_Q8_1F, 4, 1, false, 2)
  SKG_M12(SKG_Q8_0_Q8_1F, 4, 2, 4, 1, 2, 2)
  SKG_M3_8(SKG_Q8_0_Q8_1F, 4, 1, false, 2)
}
}  // namespace skg
