// q4_0 weights x fp32 activations, M = 1, 2 and measurement variants.
#include "gemv_instances.h"

namespace skg {
void register_gemv_q4_0_f32(std::vector<GemvEntry>& out) {
  // The first instance of each (format, M, epilogue) is its default, chosen
  // by measurement on MI355X under cold-cache rotation.
  // M = 1 at K = 4096, N = 14336: 8.39 us (2 rows per wave, 8-row
  // workgroups, activation in LDS) against 8.61-8.90 us with 4 rows per wave
  // and 8.6-15.1 us for the other measured organisations
  SKG_I(SKG_Q4_0_F32, 1, 2, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 4, 2, true, 4, SKG_EPI_NONE)
  SKG_M12(SKG_Q4_0_F32, 8, 2, 8, 1, 4, 4)
  SKG_IK(SKG_Q4_0_F32, 1, 8, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_F32, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_0_F32, 1, 4, 1, 4, SKG_EPI_NONE, 4)
  SKG_I(SKG_Q4_0_F32, 1, 4, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 16, 2, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 8, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 16, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 16, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 2, 8, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 8, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 8, 2, true, 2, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 8, 2, true, 1, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 4, 2, true, 2, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 8, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 8, 2, true, 8, SKG_EPI_NONE)
  // activation in LDS with K split across the waves of a row group
  SKG_IKL(SKG_Q4_0_F32, 1, 4, 1, 8, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q4_0_F32, 1, 2, 1, 8, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q4_0_F32, 1, 8, 1, 8, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q4_0_F32, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q4_0_F32, 1, 2, 1, 16, SKG_EPI_NONE, 2)
  SKG_I(SKG_Q4_0_F32, 1, 2, 2, true, 8, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 1, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_0_F32, 1, 1, 2, true, 8, SKG_EPI_NONE)
  SKG_IKL(SKG_Q4_0_F32, 1, 2, 1, 4, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q4_0_F32, 1, 1, 1, 4, SKG_EPI_NONE, 2)
}
}  // namespace skg
