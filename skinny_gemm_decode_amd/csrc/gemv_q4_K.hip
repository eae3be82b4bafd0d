// q4_K super-block weights x fp32 or Q8_1 activations, and measurement
// variants.  The first instance of each (format, M, epilogue) is its default,
// chosen by measurement on MI355X at K = 4096, N = 14336 under cold-cache
// rotation.
#include "gemv_instances.h"

namespace skg {
void register_gemv_q4_K(std::vector<GemvEntry>& out) {
  // q4_K x fp32: M = 1 10.0 us (4 rows per wave, activation in LDS); M >= 2
  // with 4 rows per wave and the activation in LDS (M = 2: 14.2 us against
  // 20.2-22.5 us from registers; M = 8: 41.4 us against 42.3 us with 8 rows)
  SKG_I(SKG_Q4_K_F32, 1, 4, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q4_K_F32, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_N3_8(SKG_Q4_K_F32, 4, 1, true)
  SKG_M12(SKG_Q4_K_F32, 8, 2, 8, 1, 4, 4)
  SKG_M3_8(SKG_Q4_K_F32, 8, 1, true, 4)
  SKG_IKL(SKG_Q4_K_F32, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_I(SKG_Q4_K_F32, 2, 4, 1, false, 4, SKG_EPI_NONE)
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
