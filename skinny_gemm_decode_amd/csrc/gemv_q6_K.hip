// q6_K super-block weights x fp32 or Q8_1 activations, and measurement
// variants.  The first instance of each (format, M, epilogue) is its default,
// chosen by measurement on MI355X at K = 4096, N = 14336 under cold-cache
// rotation.
#include "gemv_instances.h"

namespace skg {
void register_gemv_q6_K(std::vector<GemvEntry>& out) {
  // q6_K x fp32, activation in LDS: 4 rows per wave where the kernel keeps two
  // waves per SIMD (M = 1, 3, 5, 6: M = 6 28.6 us against 34.2 us), 2 rows
  // where 4 rows would leave one (M = 2, 4, 7, 8: M = 4 24.5 against 36.4 us)
  SKG_I(SKG_Q6_K_F32, 1, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 2, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 3, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 4, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 5, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 6, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 7, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 8, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_M12(SKG_Q6_K_F32, 4, 2, 4, 1, 2, 2)
  SKG_M3_8(SKG_Q6_K_F32, 4, 1, true, 2)
  SKG_IKL(SKG_Q6_K_F32, 1, 4, 1, 8, SKG_EPI_NONE, 2)
  SKG_I(SKG_Q6_K_F32, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_N3_8(SKG_Q6_K_F32, 2, 1, true)
  // q6_K x Q8_1: M = 1 9.4 us; M >= 3 8 rows per wave, activation in LDS
  // (M = 8: 21.4 us against 23.0-24.5 us)
  SKG_IK(SKG_Q6_K_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_N3_8(SKG_Q6_K_Q8_1, 8, 1, true)
  SKG_M12(SKG_Q6_K_Q8_1, 4, 2, 4, 1, 2, 2)
  SKG_M3_8(SKG_Q6_K_Q8_1, 4, 1, false, 2)
  SKG_N3_8(SKG_Q6_K_Q8_1, 4, 1, true)
}
}  // namespace skg
