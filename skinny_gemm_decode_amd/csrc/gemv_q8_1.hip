// q4_0 / q8_0 weights x Q8_1 activations (integer dot).
#include "gemv_instances.h"

// M = 2..8 with the Q8_1 SwiGLU epilogue: 8 row groups of 4 outputs (32 rows).
#define SKG_Q8_1_EPI_M2_8(F)                       \
  SKG_I(F, 2, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1) \
  SKG_I(F, 3, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1) \
  SKG_I(F, 4, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1) \
  SKG_I(F, 5, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1) \
  SKG_I(F, 6, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1) \
  SKG_I(F, 7, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1) \
  SKG_I(F, 8, 4, 1, false, 8, SKG_EPI_SWIGLU_Q8_1)

namespace skg {
void register_gemv_q8_1(std::vector<GemvEntry>& out) {
  // The first instance of each (format, M, epilogue) is its default, chosen
  // by measurement on MI355X under cold-cache rotation (K = 4096 and 11008).
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 2, 1, 4, SKG_EPI_SWIGLU, 2)
  SKG_IK(SKG_Q8_0_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_M12(SKG_Q4_0_Q8_1, 8, 2, 8, 1, 4, 4)
  // M = 3..8: activation staged in LDS, 8 rows per wave (M = 4: 10.5 us
  // against 11.2 us from registers; M = 8: 16.0 against 19.0 us)
  SKG_M3_8(SKG_Q4_0_Q8_1, 8, 1, true, 2)
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
  // SwiGLU with the Q8_1 form of h: whole 32-row blocks per workgroup
  // (default measured at gate/up 2 x 11008 x 4096: 12.0 us, against 14.9 us
  // for 16 waves in pairs and 10.4 us for the plain SwiGLU default)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 2, 1, 16, SKG_EPI_SWIGLU_Q8_1, 1)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 1, 8, SKG_EPI_SWIGLU_Q8_1, 1)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 4, 1, 16, SKG_EPI_SWIGLU_Q8_1, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 8, 1, 8, SKG_EPI_SWIGLU_Q8_1, 2)
  SKG_IK(SKG_Q4_0_Q8_1, 1, 8, 1, 4, SKG_EPI_SWIGLU_Q8_1, 1)
  SKG_IK(SKG_Q8_0_Q8_1, 1, 2, 1, 16, SKG_EPI_SWIGLU_Q8_1, 1)
  SKG_IK(SKG_Q8_0_Q8_1, 1, 4, 1, 16, SKG_EPI_SWIGLU_Q8_1, 2)
  SKG_Q8_1_EPI_M2_8(SKG_Q4_0_Q8_1)
  SKG_Q8_1_EPI_M2_8(SKG_Q8_0_Q8_1)
  // activation staged in LDS (one copy per workgroup instead of one per wave)
  SKG_I(SKG_Q4_0_Q8_1, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 2, 8, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 4, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 8, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 8, 4, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_Q8_1, 4, 4, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_Q8_1, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_Q8_1, 4, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_Q8_1, 8, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_Q8_1, 8, 8, 1, true, 4, SKG_EPI_NONE)
}
}  // namespace skg
