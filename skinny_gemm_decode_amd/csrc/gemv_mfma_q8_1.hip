// q4_0 / q8_0 weights x Q8_1 activations on the integer matrix cores, M = 2..8.
#include "gemv_instances.h"
#include "gemv_mfma.h"

// MF8(F, M, waves, blocks per wave, prefetch depth)
#define SKG_MF8(F, M, W, B, PD) out.push_back(skg::gemv_mfma_entry<F, M, W, B, 1, SKG_EPI_NONE, PD>());

namespace skg {
// Registered before the vector-ALU Q8_1 instances: the defaults where they
// measure faster on MI355X (K = 4096, N = 14336, cold-cache rotation): q4_0
// M = 7 / 8 14.1 / 13.8 us against 14.6 / 16.0 us on the vector ALU, q8_0
// 18.1 / 17.6 (weights through an LDS ring) against 19.1 / 19.7 us.  From M = 6 down the vector kernels win
// (M = 4: 10.6 against 13.4 us for q4_0).  Other K (not a multiple of 256, or
// above 4096) fall through to the vector kernels.
void register_gemv_mfma_q8_1(std::vector<GemvEntry>& out) {
  SKG_MF8(SKG_Q4_0_Q8_1, 7, 16, 8, 1)
  SKG_MF8(SKG_Q4_0_Q8_1, 8, 16, 8, 1)
  // q8_0 at M = 7, 8: the weights streamed into an LDS ring, 18.08 / 17.55 us
  // against 18.45 / 18.12 for the register-fed kernel (three A1 B1 B2 A2
  // cycles; K = 4096 only, other K take the register-fed kernel)
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 7, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 8, 1, 2, true>());
  SKG_MF8(SKG_Q8_0_Q8_1, 7, 16, 8, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 8, 16, 8, 1)
}

// Registered after them: measurement variants.
void register_gemv_mfma_q8_1_alt(std::vector<GemvEntry>& out) {
  SKG_MF8(SKG_Q4_0_Q8_1, 2, 16, 8, 1)
  SKG_MF8(SKG_Q4_0_Q8_1, 3, 16, 8, 1)
  SKG_MF8(SKG_Q4_0_Q8_1, 4, 16, 8, 1)
  SKG_MF8(SKG_Q4_0_Q8_1, 5, 16, 8, 1)
  SKG_MF8(SKG_Q4_0_Q8_1, 6, 16, 8, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 2, 16, 8, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 3, 16, 8, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 4, 16, 8, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 5, 16, 8, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 6, 16, 8, 1)
  // 8 waves of 16 blocks: 1.5-2 us slower at every M
  SKG_MF8(SKG_Q4_0_Q8_1, 4, 8, 16, 2)
  SKG_MF8(SKG_Q4_0_Q8_1, 8, 8, 16, 2)
  SKG_MF8(SKG_Q8_0_Q8_1, 4, 8, 16, 1)
  SKG_MF8(SKG_Q8_0_Q8_1, 8, 8, 16, 1)
  // weights streamed into an LDS ring (K = 4096 only): ties the vector
  // kernel for q8_0 at M = 6; slower for q8_0 at M = 4, 5 (15-16%) and for
  // q4_0 at M = 6..8 (5-9%), which are not compiled
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 6, 1, 2, true>());
}
}  // namespace skg
