// q4_0 / q8_0 weights x Q8_1 activations on the integer matrix cores, M = 2..8.
#include "gemv_instances.h"
#include "gemv_mfma.h"

// MF8(F, M, waves, blocks per wave, prefetch depth)
#define SKG_MF8(F, M, W, B, PD) out.push_back(skg::gemv_mfma_entry<F, M, W, B, 1, SKG_EPI_NONE, PD>());

namespace skg {
// Registered before the vector-ALU Q8_1 instances: the defaults where they
// measure faster on MI355X (K = 4096, N = 14336, cold-cache rotation).  The
// weights streamed into an LDS ring, two blocks per 64-deep integer MFMA:
// q4_0 M = 6 / 7 / 8 10.45 / 10.15 / 10.05 us, q8_0 14.21 / 14.04 / 13.80 us
// (one block per MFMA before: 12.79 / 12.92 / 12.71 and 16.93 / 17.07 /
// 16.72; the next best kernels, vector at M = 6 and register-fed integer
// MFMA at 7, 8, took 13.44 / 14.06 / 13.52 and 17.83 / 18.45 / 18.12).  The
// ring kernels take K = 4096 only; other K (not a multiple of 256, or above
// 4096) fall through to the register-fed or vector kernels.  At M = 4 / 5 the
// ring kernel is the default too: q4_0 10.28 / 10.84 us against 10.63 /
// 12.19 for the vector kernel, q8_0 14.43 / 14.65 against 14.73 / 15.89; at
// M = 2 / 3 the vector kernel stays ahead (q4_0 8.77 / 9.62 against 9.33 /
// 10.18, q8_0 12.18 / 13.49 against 13.38 / 13.98).
// q4_0 at M = 3..8 takes three ring slots with the staging in the last (two
// tiles requested at the start, the third once the activation is staged):
// M = 3 / 4 / 5 / 6 / 7 / 8 9.32-9.33 / 9.67-9.69 / 9.95-9.99 /
// 10.00-10.03 / 10.04 / 9.96-9.99 us against 9.41 / 9.90-9.91 / 10.02 /
// 10.14-10.16 / 10.18-10.19 / 10.11-10.13 with two slots (and 9.60-9.62
// for the vector kernel at M = 3); without the aliasing (two slots and an
// own staging area) 10.25 / 10.47 / 10.52 at M = 4 / 6 / 8.  q8_0's slots
// fit the LDS only twice.
void register_gemv_mfma_q8_1(std::vector<GemvEntry>& out) {
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 3, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 4, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 5, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 4, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 5, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 6, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 7, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 8, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 6, 1, 2, true>());
  SKG_MF8(SKG_Q4_0_Q8_1, 7, 16, 8, 1)
  SKG_MF8(SKG_Q4_0_Q8_1, 8, 16, 8, 1)
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
  // weights streamed into an LDS ring at M = 2 / 3: slower than the vector
  // kernels (figures above)
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 2, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_Q8_1, 3, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 2, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 3, 1, 2, true>());
  // q4_0 with four slots, every tile of a workgroup in flight from the
  // start: slower (M = 6 / 7 / 8: 14.90 / 14.75 / 14.87 us against 12.80 /
  // 12.92 / 12.73 for the two-slot defaults)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 6, 1, 4, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 7, 1, 4, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 8, 1, 4, true>());
  // q4_0 with two slots (the defaults before the three-slot ones)
  for (auto e : {gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 4, 1, 2, true>(), gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 5, 1, 2, true>(),
                 gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 6, 1, 2, true>(), gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 7, 1, 2, true>(),
                 gemv_mfma_dma_entry<SKG_Q4_0_Q8_1, 8, 1, 2, true>()})
    out.push_back(e);
}
}  // namespace skg
