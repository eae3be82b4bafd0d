// q6_K super-block weights x fp32 or Q8_1 activations, and measurement
// variants.  The first instance of each (format, M, epilogue) is its default,
// chosen by measurement on MI355X at K = 4096, N = 14336 under cold-cache
// rotation.
#include "gemv_instances.h"
#include "gemv_mfma.h"

namespace skg {
void register_gemv_q6_K(std::vector<GemvEntry>& out) {
  // q6_K x fp32 at M = 3..8: the matrix cores with the weights streamed into
  // an LDS ring (block-halves per MFMA so each result row has one int8 scale,
  // codes as the exact fp16 q - 32, the activation as one fp16 term with a
  // power of two per row and wave; K = 4096 only, other K take the vector
  // kernels below).  Alternating timings, us (ring / vector default
  // before): M = 3 15.83 / 18.98, 4 15.92 / 20.68, 5 18.05 / 25.27,
  // 6 18.42 / 25.76, 7 18.67 / 33.53, 8 18.70 / 36.58.  The partial sums of
  // a workgroup's tiles meet once after its last tile (instead of after each
  // tile's barrier): M = 3 / 4 / 6 / 8 15.13-15.16 / 15.31-15.32 /
  // 17.35-17.37 / 17.85-17.91 us against 15.85-15.86 / 15.87-15.88 /
  // 18.41-18.42 / 18.70-18.72; with the activation staged in the second
  // slot too (its tile requested once the staging is read): M = 4 / 8
  // 14.77-14.79 / 17.13-17.16 against 15.28-15.30 / 17.88-17.91.
  // At M = 2 the same kernel (activation as one fp16 term) takes 13.92-13.94
  // us against 14.27-14.51 for the vector kernels (fp32 activation), and
  // 15.23-15.24 with its own staging area and a reduction per tile.
  for (auto e : {gemv_mfma_q6f_entry<2, 2, true, true>(), gemv_mfma_q6f_entry<3, 2, true, true>(),
                 gemv_mfma_q6f_entry<4, 2, true, true>(),
                 gemv_mfma_q6f_entry<5, 2, true, true>(), gemv_mfma_q6f_entry<6, 2, true, true>(),
                 gemv_mfma_q6f_entry<7, 2, true, true>(), gemv_mfma_q6f_entry<8, 2, true, true>()})
    out.push_back(e);
  // q6_K x Q8_1 at M = 4..8: the integer matrix cores with the weights
  // streamed into an LDS ring (low units, high units, int8 scale pairs and d
  // per row; block-halves per 64-deep MFMA, the -32 of the codes as a chained
  // MFMA against constant -32; K = 4096 only, other K fall through to the
  // vector kernels below).  Alternating timings, us (ring / vector default
  // before): M = 4 13.45 / 14.03, 5 15.89 / 16.58, 6 16.08 / 18.29,
  // 7 16.32 / 19.78, 8 15.88 / 21.39.  With the partial sums reduced once
  // after the last tile: M = 4 / 6 / 8 12.92 / 15.07 / 15.59-15.60 us
  // against 13.47-13.48 / 16.09-16.10 / 15.93.
  for (auto e : {gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 4, 1, 2, true, true>(),
                 gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 5, 1, 2, true, true>(),
                 gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 6, 1, 2, true, true>(),
                 gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 7, 1, 2, true, true>(),
                 gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 8, 1, 2, true, true>()})
    out.push_back(e);
  // q6_K x fp32, activation in LDS: 2 rows per wave (M = 1: 2 units per
  // lane, 11.09 us against 11.83-12.20; M = 6 27.29 against 40.19 with 4
  // rows), 4 rows at M = 3, 5 (M = 5 22.44 against 24.46)
  SKG_I(SKG_Q6_K_F32, 1, 2, 2, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 2, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 3, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 4, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 5, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 6, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 7, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 8, 2, 1, true, 4, SKG_EPI_NONE)
  // SwiGLU: M = 1, 2 from registers, M >= 3 in LDS, 2 output rows per wave
  SKG_I(SKG_Q6_K_F32, 1, 2, 2, false, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 2, 2, 1, false, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 3, 2, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 4, 2, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 5, 2, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 6, 2, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 7, 2, 1, true, 4, SKG_EPI_SWIGLU)
  SKG_I(SKG_Q6_K_F32, 8, 2, 1, true, 4, SKG_EPI_SWIGLU)
  // measurement variants
  SKG_I(SKG_Q6_K_F32, 1, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 1, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 1, 4, 2, false, 4, SKG_EPI_NONE)
  SKG_IKL(SKG_Q6_K_F32, 1, 4, 1, 8, SKG_EPI_NONE, 2)
  SKG_I(SKG_Q6_K_F32, 2, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 2, 4, 1, false, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 3, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 4, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 5, 2, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 6, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 7, 4, 1, true, 4, SKG_EPI_NONE)
  SKG_I(SKG_Q6_K_F32, 8, 4, 1, true, 4, SKG_EPI_NONE)
  // q6_K x Q8_1: M = 1 9.4 us; M >= 3 8 rows per wave, activation in LDS
  // (M = 8: 21.4 us against 23.0-24.5 us)
  SKG_IK(SKG_Q6_K_Q8_1, 1, 4, 1, 4, SKG_EPI_NONE, 2)
  SKG_N3_8(SKG_Q6_K_Q8_1, 8, 1, true)
  SKG_M12(SKG_Q6_K_Q8_1, 4, 2, 4, 1, 2, 2)
  SKG_M3_8(SKG_Q6_K_Q8_1, 4, 1, false, 2)
  SKG_N3_8(SKG_Q6_K_Q8_1, 4, 1, true)
  // q6_K x Q8_1 on the integer matrix cores at M = 2, 3: slower than the
  // vector kernels (12.67 / 13.51 against 11.40 / 12.63 us; 12.18 / 13.10
  // with the partial sums reduced after the last tile)
  out.push_back(gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 2, 1, 2, true>());
  out.push_back(gemv_mfma_dma_entry<SKG_Q6_K_Q8_1, 3, 1, 2, true>());

}
}  // namespace skg
