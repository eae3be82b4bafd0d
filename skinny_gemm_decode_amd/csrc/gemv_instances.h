// Compiled GEMV kernel instances.  Each format's translation unit expands the
// list for its formats; the host dispatch finds instances by
// (fmt, M, epilogue, rows per wave, units per lane, LDS staging, waves).
#pragma once

#include <vector>

#include "gemv_impl.h"

// I(FMT, M, RO, J, XLDS, WAVES, EPI): one row group per wave.
#define SKG_I(F, M, RO, J, X, W, E) out.push_back(skg::gemv_entry<F, M, RO, J, X, W, E, 1>());
// IK(..., KW): KW waves share each row group and split its K chunks.
#define SKG_IK(F, M, RO, J, W, E, KW) out.push_back(skg::gemv_entry<F, M, RO, J, false, W, E, KW>());
// IKL(..., KW): the same with the activation staged in LDS, one region per K class.
#define SKG_IKL(F, M, RO, J, W, E, KW) out.push_back(skg::gemv_entry<F, M, RO, J, true, W, E, KW>());

// Default instances, split by M so translation units compile in parallel.
// Arguments: format; rows per wave and units per lane for M = 1, for M = 2,
// for M >= 3; LDS staging for M >= 3; rows per wave of the SwiGLU variants.
#define SKG_M12(F, RO1, J1, RO2, J2, SRO1, SRO2)  \
  SKG_I(F, 1, RO1, J1, false, 4, SKG_EPI_NONE)    \
  SKG_I(F, 2, RO2, J2, false, 4, SKG_EPI_NONE)    \
  SKG_I(F, 1, SRO1, J1, false, 4, SKG_EPI_SWIGLU) \
  SKG_I(F, 2, SRO2, J2, false, 4, SKG_EPI_SWIGLU)

#define SKG_M(F, M, ROL, JL, XL, SROL)          \
  SKG_I(F, M, ROL, JL, XL, 4, SKG_EPI_NONE)     \
  SKG_I(F, M, SROL, JL, XL, 4, SKG_EPI_SWIGLU)

#define SKG_M3_8(F, ROL, JL, XL, SROL) \
  SKG_M(F, 3, ROL, JL, XL, SROL)       \
  SKG_M(F, 4, ROL, JL, XL, SROL)       \
  SKG_M(F, 5, ROL, JL, XL, SROL)       \
  SKG_M(F, 6, ROL, JL, XL, SROL)       \
  SKG_M(F, 7, ROL, JL, XL, SROL)       \
  SKG_M(F, 8, ROL, JL, XL, SROL)

// plain GEMV only, M = 3..8
#define SKG_N3_8(F, RO, J, X)           \
  SKG_I(F, 3, RO, J, X, 4, SKG_EPI_NONE) \
  SKG_I(F, 4, RO, J, X, 4, SKG_EPI_NONE) \
  SKG_I(F, 5, RO, J, X, 4, SKG_EPI_NONE) \
  SKG_I(F, 6, RO, J, X, 4, SKG_EPI_NONE) \
  SKG_I(F, 7, RO, J, X, 4, SKG_EPI_NONE) \
  SKG_I(F, 8, RO, J, X, 4, SKG_EPI_NONE)
