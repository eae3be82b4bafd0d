// q4_K super-block weights x fp32 or Q8_1 activations, and measurement
// variants.  The first instance of each (format, M, epilogue) is its default,
// chosen by measurement on MI355X at K = 4096, N = 14336 under cold-cache
// rotation.
#include "gemv_instances.h"
#include "gemv_mfma.h"

// q4_K x fp32 on the matrix cores: MF(M, waves, blocks per wave, fp16
// activation terms, prefetch depth)
#define SKG_MFK(M, W, B, XT, PD) out.push_back(skg::gemv_mfma_entry<SKG_Q4_K_F32, M, W, B, XT, SKG_EPI_NONE, PD>());

namespace skg {
void register_gemv_q4_K(std::vector<GemvEntry>& out) {
  // q4_K x fp32 at M = 2..8: the LDS-ring kernel with grouped blocks (four
  // sub-blocks per MFMA chain for M <= 4, two for M = 5..8; codes as exact
  // fp16 subnormals, d sc_j per sub-block, the min term from block sums of
  // the staged activation), the activation as one fp16 term; K = 4096 only,
  // other K take the register-fed kernels below.  Alternating timings, us
  // (grouped / previous default, register-fed): M = 2 10.05 / 12.61 (two
  // terms), 3 10.51 / 13.92 (two terms), 4 10.69 / 13.04, 5 11.97 / 13.89,
  // 6 12.03 / 14.04, 7 12.46 / 14.42, 8 12.63 / 14.48; grouped with two
  // terms 10.73 / 11.69 / 12.40 / 13.53 / 13.68 / 14.37 / 14.44.  M = 2..4
  // take three slots with the staging in the last (two tiles requested at
  // the start, the third once the activation is staged): 9.73-9.81 /
  // 10.39-10.47 / 10.58-10.61 us against 10.10-10.11 / 10.54 / 10.69-10.72
  // with two slots and their own staging area; at M = 7 12.53 against 12.46.
  // M = 5, 6, 7 take two slots with the staging in the last (tile 1
  // requested once the activation is staged): 11.61-11.62 / 11.84-11.85 /
  // 12.22-12.24 us against 11.99-12.00 / 12.06-12.08 / 12.49 (at M = 8 the
  // staging and block sums outgrow a slot).
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_K_F32, 2, 3, true>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 3, 3, true>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 4, 3, true>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 5, 2, true>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 6, 2, true>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 7, 2, true>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 8, 2, false>()})
    out.push_back(e);
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_K_F32, 2, 2, false>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 3, 2, false>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 4, 2, false>()})
    out.push_back(e);
  // q4_K x Q8_1 at M = 3..8: the integer matrix cores with the weights
  // streamed into an LDS ring (two sub-blocks per 64-deep MFMA, the d sc_j
  // scaling and the dmin m_j s min term per sub-block on the vector ALU;
  // K = 4096 only, other K fall through to the vector kernels below).
  // Alternating timings, us (ring / vector default before): M = 3 10.10 /
  // 10.38, 4 10.49 / 11.67, 5 10.35 / 13.46, 6 10.54 / 15.05, 7 10.56 /
  // 16.51, 8 10.53 / 17.87.
  for (auto e : {gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 3, 1, 2, true>(), gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 4, 1, 2, true>(),
                 gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 5, 1, 2, true>(), gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 6, 1, 2, true>(),
                 gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 7, 1, 2, true>(), gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 8, 1, 2, true>()})
    out.push_back(e);
  // q4_K x fp32 at M = 2..8 on the matrix cores (K a multiple of 256 up to
  // 4096; others fall through to the vector kernels below): the activation
  // as two fp16 terms at M = 2, 3 (13.01 / 14.11 us against 13.28 / 17.62 for
  // the vector kernel) and as one term from M = 4, inside the accuracy bound
  // as for q4_0 (M = 4 / 5 / 6 / 7 / 8: 13.17 / 13.86 / 14.13 / 14.63 / 14.58
  // us against 21.07 / 24.82 / 27.69 / 30.67 / 34.21; two terms 15.30 /
  // 18.69 / 17.34 / 18.15 / 17.51)
  SKG_MFK(2, 16, 8, 2, 1)
  SKG_MFK(3, 8, 16, 2, 1)
  SKG_MFK(4, 16, 8, 1, 1)
  SKG_MFK(5, 16, 8, 1, 1)
  SKG_MFK(6, 16, 8, 1, 1)
  SKG_MFK(7, 16, 8, 1, 1)
  SKG_MFK(8, 16, 8, 1, 1)
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
  // q4_K x fp32 on the matrix cores: measurement variants (16 waves with two
  // terms spill at M = 3: 20.33 us)
  SKG_MFK(2, 8, 16, 1, 1)
  SKG_MFK(2, 8, 16, 2, 1)
  SKG_MFK(3, 8, 16, 1, 1)
  SKG_MFK(3, 16, 8, 2, 1)
  SKG_MFK(3, 16, 8, 1, 1)
  SKG_MFK(4, 8, 16, 1, 1)
  SKG_MFK(4, 8, 16, 2, 1)
  SKG_MFK(5, 8, 16, 1, 1)
  SKG_MFK(5, 8, 16, 2, 1)
  SKG_MFK(6, 8, 16, 1, 1)
  SKG_MFK(6, 8, 16, 2, 1)
  SKG_MFK(7, 8, 16, 1, 1)
  SKG_MFK(7, 8, 16, 2, 1)
  SKG_MFK(8, 8, 16, 1, 1)
  SKG_MFK(8, 8, 16, 1, 2)
  SKG_MFK(8, 8, 16, 2, 1)
  // q4_K x fp32 on the LDS-ring kernel with grouped blocks, two fp16
  // activation terms (measurement variants)
  for (auto e : {gemv_mfma_grp_entry<SKG_Q4_K_F32, 2, 2, false, 2>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 3, 2, false, 2>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 4, 2, false, 2>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 5, 2, false, 2>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 6, 2, false, 2>(),
                 gemv_mfma_grp_entry<SKG_Q4_K_F32, 7, 2, false, 2>(), gemv_mfma_grp_entry<SKG_Q4_K_F32, 8, 2, false, 2>()})
    out.push_back(e);
  // q4_K x Q8_1 on the integer matrix cores at M = 2: slower than the
  // vector kernel (9.50 against 9.30 us)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 2, 1, 2, true>());
  // q4_K x Q8_1 with three slots (staging in the last): slower than two at
  // M = 4 / 6 / 8 (10.53-10.54 / 10.90-10.91 / 11.04-11.05 against 10.42 /
  // 10.53-10.54 / 10.50-10.55 us)
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 4, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 6, 1, 3, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q4_K_Q8_1, 8, 1, 3, true>());
}
}  // namespace skg
