// q8_0 weights x fp32 activations, M = 1, 2 and measurement variants.
#include "gemv_instances.h"

namespace skg {
void register_gemv_q8_0_f32(std::vector<GemvEntry>& out) {
  // The first instance of each (format, M, epilogue) is its default, chosen
  // by measurement on MI355X under cold-cache rotation.
  // M = 1 at K = 4096, N = 14336: 11.8 us (4 rows per wave, 1 unit per lane)
  // against 12.6 us with 2 units per lane and 11.9-14.4 us for 1-8 rows per
  // wave and 2-16 waves
  SKG_I(SKG_Q8_0_F32, 1, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_M12(SKG_Q8_0_F32, 4, 2, 4, 1, 2, 2)
  SKG_IK(SKG_Q8_0_F32, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q8_0_F32, 1, 8, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q8_0_F32, 1, 2, 1, 4, SKG_EPI_NONE, 4)
  SKG_I(SKG_Q8_0_F32, 1, 2, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 8, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 4, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 8, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 8, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 4, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 2, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 1, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 1, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 4, 1, true, 2, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 2, 2, true, 2, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 2, 1, true, 2, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 8, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q8_0_F32, 1, 2, 2, true, 8, SKG_EPI_NONE)
  // activation in LDS with K split across the waves of a row group
  SKG_IKL(SKG_Q8_0_F32, 1, 4, 1, 8, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q8_0_F32, 1, 2, 1, 8, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q8_0_F32, 1, 2, 1, 16, SKG_EPI_NONE, 2)
}
}  // namespace skg
