// q4_0 weights x fp32 activations on the matrix cores, M = 1..8.
#include "gemv_instances.h"
#include "gemv_mfma.h"
#include "gemv_mfma_pw.h"

// MF(M, fp16 activation terms, prefetch depth)
#define SKG_MF(M, XT, PD) out.push_back(skg::gemv_mfma_entry<SKG_Q4_0_F32, M, 8, 16, XT, SKG_EPI_NONE, PD>());

namespace skg {
// Registered before the vector-ALU instances: the defaults for M = 2..8,
// measured on MI355X under cold-cache rotation (K = 4096, N = 14336).
void register_gemv_mfma_q4_0(std::vector<GemvEntry>& out) {
  // M = 2..8: the LDS-ring kernel with grouped blocks (four per MFMA chain
  // for M <= 4, two for M = 5..8), the activation as one fp16 term (one
  // rounding, 2^-11, inside the accuracy bound).  Alternating timings against
  // the kernels below, us (grouped / previous default): M = 2 10.25 / 11.35
  // (ring, two terms), 3 10.64 / 11.57, 4 10.70 / 11.76, 5 11.12 / 12.44,
  // 6 11.16 / 12.40, 7 11.39 / 11.78, 8 11.39 / 11.78 (ring, one block per
  // MFMA).  M = 2..4 take three slots with the staging in the last (two
  // tiles requested at the start, the third once the activation is staged):
  // 9.98-10.08 / 10.39-10.41 / 10.36-10.44 us against 10.24-10.25 /
  // 10.62-10.63 / 10.69 with two slots and their own staging area; at
  // M = 5, 6, 8 they trail by 0.5-1% (11.16-11.22, 11.25-11.29, 11.47).
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_0_F32, 2, 3, true>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 3, 3, true>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 4, 3, true>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 5, 2, false>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 6, 2, false>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 7, 2, false>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 8, 2, false>()})
    out.push_back(e);
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_0_F32, 2, 2, false>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 3, 2, false>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 4, 2, false>()})
    out.push_back(e);
  // Before them: M = 2: the LDS-ring kernel with two fp16 activation terms, 11.35 us
  // against 11.82 (register-fed, two terms); M = 3 / 5: the ring with one
  // term, 11.61 / 12.41 us against 12.16 / 12.59 (register-fed, two terms)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 2, 2, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 3, 1, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 5, 1, 3, false>());
  SKG_MF(2, 2, 1)
  SKG_MF(3, 2, 1)
  // M = 4, 6: the LDS-ring kernel with one fp16 activation term, 12.00 /
  // 12.79 us against 12.58 / 12.94 (it loses at M = 2, 3, 5 by 1-2%)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 4, 1, 3, false>());
  SKG_MF(4, 2, 1)
  SKG_MF(5, 2, 1)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 6, 1, 3, false>());
  SKG_MF(6, 2, 1)
  // M = 7, 8: the LDS-ring kernel with one fp16 activation term (one
  // rounding, 2^-11, inside the accuracy bound), 12.24 / 12.82 us against
  // 12.99 (the ring with two terms) / 14.18 (register-fed, one term), three
  // A1 B1 B2 A2 cycles; K = 4096 only, other K take the register-fed kernels
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 7, 1, 2, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 8, 1, 2, false>());
  SKG_MF(7, 2, 1)
  SKG_MF(8, 1, 2)  // one fp16 term: within the accuracy bound, 8% faster at M = 8
}
// Registered after them: measurement variants (at M = 1 the vector kernel
// is faster; the LDS-ring kernel trails the register-fed one at every M).
void register_gemv_mfma_q4_0_alt(std::vector<GemvEntry>& out) {
  // grouped blocks with the activation as two fp16 terms (two blocks per
  // MFMA chain; four hi and four lo rows per block for M <= 4, a second
  // chain of lo operands for M = 5..8)
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_0_F32, 2, 2, false, 2>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 3, 2, false, 2>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 4, 2, false, 2>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 5, 2, false, 2>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 6, 2, false, 2>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 7, 2, false, 2>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 8, 2, false, 2>()})
    out.push_back(e);
  // grouped blocks with three ring slots and their own staging area (all
  // three tiles requested at the start): 0.6-0.8 us slower than two slots
  // (M = 2 / 3 / 4: 10.82 / 11.44 / 11.50 us; 8: 12.18-12.20).  At M = 2..4
  // the three-slot defaults (staging in the last slot) hold their keys.
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_0_F32, 5, 3, false>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 6, 3, false>(),
                 gemv_mfma_grp_entry<SKG_Q4_0_F32, 7, 3, false>(), gemv_mfma_grp_entry<SKG_Q4_0_F32, 8, 3, false>()})
    out.push_back(e);
  // per-wave weight rings (measurement variants)
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 2, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 2, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 3, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 3, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 4, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 4, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 5, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 5, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 6, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 6, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 7, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 7, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 8, 1, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 8, 2, 3>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 4, 1, 2>());
  out.push_back(gemv_mfma_pw_entry<SKG_Q4_0_F32, 8, 1, 2>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 1, 2, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 4, 2, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 7, 2, 2, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 8, 2, 2, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 8, 1, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 7, 1, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 3, 2, 3, false>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 5, 2, 3, false>());
  // four slots, every tile of a workgroup in flight from the start: slower
  // at every M (M = 4 / 6 / 7 / 8: 12.34 / 12.94 / 13.15 / 13.02 us against
  // 11.71 / 12.38 / 11.77 / 11.75 for the defaults)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 4, 1, 4, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 6, 1, 4, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 7, 1, 4, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_0_F32, 8, 1, 4, true>());
  SKG_MF(1, 2, 1)
  SKG_MF(1, 1, 2)
  SKG_MF(8, 2, 1)
  // 16 waves of 8 blocks: twice the waves per SIMD to hide latency
  out.push_back(skg::gemv_mfma_entry<SKG_Q4_0_F32, 1, 16, 8, 2, SKG_EPI_NONE, 1>());
  out.push_back(skg::gemv_mfma_entry<SKG_Q4_0_F32, 1, 16, 8, 1, SKG_EPI_NONE, 1>());
  out.push_back(skg::gemv_mfma_entry<SKG_Q4_0_F32, 2, 16, 8, 2, SKG_EPI_NONE, 1>());
}
}  // namespace skg
