// q8_0 weights x fp32 activations on the matrix cores, M = 1..8.
#include "gemv_instances.h"
#include "gemv_mfma.h"
#include "gemv_mfma_pw.h"

// MF(M, fp16 activation terms, prefetch depth)
#define SKG_MF(M, XT, PD) out.push_back(skg::gemv_mfma_entry<SKG_Q8_0_F32, M, 8, 16, XT, SKG_EPI_NONE, PD>());

namespace skg {
// Registered before the vector-ALU instances: the defaults for M = 2..8,
// measured on MI355X under cold-cache rotation (K = 4096, N = 14336).  With
// two planes per block the two-term activation does not fit the register
// file beyond M = 2, so these carry the activation as one fp16 term.
void register_gemv_mfma_q8_0(std::vector<GemvEntry>& out) {
  // M = 2..8: the LDS-ring kernel with grouped blocks (four per MFMA chain
  // for M <= 4, two for M = 5..8), two slots, the activation staged in the
  // second one, one fp16 term.  Alternating timings against the kernels
  // below, us (grouped / previous default, the ring with one block per
  // MFMA): M = 2 13.85 / 14.67, 3 14.19 / 15.00, 4 14.23 / 15.02, 5 15.15 /
  // 15.76, 6 14.97 / 15.58, 7 15.46 / 16.02, 8 15.10 / 15.65.
  for (auto e : {gemv_mfma_grp_entry<SKG_Q8_0_F32, 2, 2, true>(), gemv_mfma_grp_entry<SKG_Q8_0_F32, 3, 2, true>(),
                 gemv_mfma_grp_entry<SKG_Q8_0_F32, 4, 2, true>(), gemv_mfma_grp_entry<SKG_Q8_0_F32, 5, 2, true>(),
                 gemv_mfma_grp_entry<SKG_Q8_0_F32, 6, 2, true>(), gemv_mfma_grp_entry<SKG_Q8_0_F32, 7, 2, true>(),
                 gemv_mfma_grp_entry<SKG_Q8_0_F32, 8, 2, true>()})
    out.push_back(e);
  // Before them:
  // M = 2..8: the LDS-ring kernel (weights copied straight into LDS) with
  // one fp16 activation term (one rounding, 2^-11, inside the accuracy
  // bound) beats the ring with two terms, the register-fed and the vector
  // kernels; three A1 B1 B2 A2 cycles each, us (one term / two terms /
  // previous default): M = 2 15.46 / 15.70 / 15.98 vector, M = 3 15.73 /
  // 16.47 / 18.07 vector, M = 4 15.65 / 16.52, M = 5 16.10 / 16.79 / 17.66,
  // M = 6 16.36 / 17.03 / 17.85, M = 7 16.54 / 17.05 / 18.21, M = 8 17.06 /
  // 19.73 / 18.81 register-fed.  It is compiled for K = 4096 only; other K
  // fall through to the register-fed kernel (M >= 4) or the vector kernel.
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 2, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 3, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 4, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 5, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 6, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 7, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 8, 1, 2, true>());
  SKG_MF(4, 1, 1)
  SKG_MF(5, 1, 1)
  SKG_MF(6, 1, 1)
  SKG_MF(7, 1, 1)
  SKG_MF(8, 1, 1)
}
// Registered after the vector-ALU instances: measurement variants.
void register_gemv_mfma_q8_0_alt(std::vector<GemvEntry>& out) {
  // grouped blocks with the activation as two fp16 terms (two blocks per
  // MFMA chain; four hi and four lo rows per block for M <= 4, a second
  // chain of lo operands for M = 5..8)
  for (auto e : {gemv_mfma_grp_entry<SKG_Q8_0_F32, 2, 2, true, 2>(), gemv_mfma_grp_entry<SKG_Q8_0_F32, 3, 2, true, 2>(),
                 gemv_mfma_grp_entry<SKG_Q8_0_F32, 4, 2, true, 2>(), gemv_mfma_grp_entry<SKG_Q8_0_F32, 5, 2, true, 2>(),
                 gemv_mfma_grp_entry<SKG_Q8_0_F32, 6, 2, true, 2>(), gemv_mfma_grp_entry<SKG_Q8_0_F32, 7, 2, true, 2>(),
                 gemv_mfma_grp_entry<SKG_Q8_0_F32, 8, 2, true, 2>()})
    out.push_back(e);
  // per-wave weight rings (measurement variants)
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 2, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 2, 2, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 3, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 3, 2, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 4, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 4, 2, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 5, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 5, 2, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 6, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 6, 2, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 7, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 7, 2, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 8, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q8_0_F32, 8, 2, 2>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 1, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 5, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 6, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 7, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 8, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 2, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 3, 2, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q8_0_F32, 4, 2, 2, true>());
  SKG_MF(1, 2, 1)
  SKG_MF(2, 2, 1)
  SKG_MF(3, 2, 1)
  SKG_MF(4, 2, 1)
  SKG_MF(8, 2, 1)
  out.push_back(skg::gemv_mfma_entry<SKG_Q8_0_F32, 1, 16, 8, 2, SKG_EPI_NONE, 1>());
}
}  // namespace skg
