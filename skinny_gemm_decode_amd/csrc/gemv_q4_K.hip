// q4_K super-block weights x fp32 or Q8_1 activations, and measurement
// variants.  The first instance of each (format, M, epilogue) is its default,
// chosen by measurement on MI355X at K = 4096, N = 14336 under cold-cache
// rotation.
#include "gemv_instances.h"

namespace skg {
void register_gemv_q4_K(std::vector<GemvEntry>& out) {
  // q4_K x fp32, activation in LDS: 2 rows per wave at M = 1, 2, 4 (M = 1
  // 9.63 us against 9.83-10.31; M = 2 13.19 against 14.25; M = 4 20.72
  // against 21.85), 4 rows at M = 3, 5..8 (M = 8 34.13 against 39.2-39.4)
  SKG_I(SKG_Q4_K_F32, 1, 2, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 2, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 3, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 4, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 5, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 6, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 7, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 8, 4, 1, true, 4, SKG_EPI_NONE)
  // SwiGLU: M = 1, 2 from registers, M >= 3 in LDS, 4 output rows per wave
  SKG_I(SKG_Q4_K_F32, 1, 4, 2, false, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 2, 4, 1, false, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 3, 4, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 4, 4, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 5, 4, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 6, 4, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 7, 4, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q4_K_F32, 8, 4, 1, true, 4, SKG_EPI_SWIGLU)
  // measurement variants
  SKG_I(SKG_Q4_K_F32, 1, 4, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 1, 8, 2, false, 4, SKG_EPI_NONE)
  SKG_IKL(SKG_Q4_K_F32, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IKL(SKG_Q4_K_F32, 1, 2, 1, 4, SKG_EPI_NONE, 2)
  SKG_I(SKG_Q4_K_F32, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 2, 8, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 2, 4, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 3, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 4, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 5, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 6, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 7, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 8, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_N3_8(SKG_Q4_K_F32, 8, 1, true)
  // q4_K x Q8_1: M = 1 7.7 us; M = 2 9.2 us (4 rows per wave); M >= 3 8 rows
  // per wave, activation in LDS (M = 8: 17.8 us against 18.9-19.6 us)
  SKG_IK(SKG_Q4_K_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_Q4_K_Q8_1, 1, 2, 1, 4, SKG_EPI_SWIGLU, 2)
  SKG_I(SKG_Q4_K_Q8_1, 2, 4, 1, false, 4, SKG_EPI_NONE)
  SKG_M12(SKG_Q4_K_Q8_1, 8, 2, 8, 1, 4, 4)
  SKG_M3_8(SKG_Q4_K_Q8_1, 8, 1, true, 2)
  SKG_N3_8(SKG_Q4_K_Q8_1, 4, 1, true)
  SKG_N3_8(SKG_Q4_K_Q8_1, 4, 1, false)
}
}  // namespace skg
