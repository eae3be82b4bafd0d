// bf16 weights x bf16 activations.
#include "gemv_instances.h"

namespace skg {
void register_gemv_bf16(std::vector<GemvEntry>& out) {
  // The first instance of each (format, M, epilogue) is its default, chosen
  // by measurement on MI355X under cold-cache rotation.
  // M = 1, 2: K split across the waves of a workgroup.
  SKG_IK(SKG_BF16_BF16, 1, 2, 1, 8, SKG_EPI_NONE, 8)
  SKG_IK(SKG_BF16_BF16, 1, 1, 2, 4, SKG_EPI_NONE, 4)
  SKG_IK(SKG_BF16_BF16, 1, 1, 2, 4, SKG_EPI_SWIGLU, 4)
  SKG_IK(SKG_BF16_BF16, 2, 1, 2, 4, SKG_EPI_NONE, 4)
  SKG_IK(SKG_BF16_BF16, 2, 1, 2, 4, SKG_EPI_SWIGLU, 4)
  SKG_M12(SKG_BF16_BF16, 2, 8, 2, 4, 1, 1)
  SKG_IK(SKG_BF16_BF16, 1, 2, 2, 4, SKG_EPI_NONE, 4)
  SKG_IK(SKG_BF16_BF16, 1, 1, 4, 4, SKG_EPI_NONE, 2)
  SKG_IK(SKG_BF16_BF16, 1, 1, 2, 8, SKG_EPI_NONE, 4)
  SKG_IK(SKG_BF16_BF16, 1, 1, 1, 8, SKG_EPI_NONE, 8)
  SKG_M3_8(SKG_BF16_BF16, 2, 1, false, 1)
  // M=1 variants for measurement
  SKG_I(SKG_BF16_BF16, 1, 1, 8, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 4, 8, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 2, 4, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 4, 4, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 8, 4, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 2, 8, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 4, 8, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 2, 8, false, 8, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 2, 8, false, 2, SKG_EPI_NONE)
  SKG_I(SKG_BF16_BF16, 1, 1, 8, false, 2, SKG_EPI_NONE)
}
}  // namespace skg
