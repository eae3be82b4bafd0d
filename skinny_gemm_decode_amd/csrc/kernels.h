// Host-side launchers of the library's kernels (internal).
#pragma once

#include <atomic>
#include <vector>

#include "common.h"

namespace skg {

hipError_t launch_pack(int wk, int64_t N, int64_t K, const void* src, void* dst, hipStream_t stream);
hipError_t launch_quantize_q8_1(int64_t M, int64_t K, const float* x, void* xq, hipStream_t stream);
// RMSNorm (+ Q8_1 of its output): K <= kNormMaxK, K % 32 == 0, M <= kNormMaxM.
constexpr int64_t kNormMaxK = 16384;
constexpr int64_t kNormMaxM = int64_t(1) << 24;
hipError_t launch_rmsnorm_q8_1(int64_t M, int64_t K, const float* x, const float* g, float eps, float* xn,
                               void* xq, hipStream_t stream);
hipError_t launch_block_dots(int fmt, const void* W, const Layout& L, int64_t n0, int64_t nr, const void* xq,
                             int32_t* out, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, hipStream_t stream);
hipError_t launch_empty(int64_t grid, int block, hipStream_t stream);
// Prefill kernel in use: 0 = one role per wave, 1 = producer/consumer waves.
extern std::atomic<int> g_gemm_variant;
extern const int kGemmDefaultVariant;

hipError_t launch_gemm_i8(int64_t M, int64_t K, int64_t N, const void* W, const Layout& L, const void* xq, float* y,
                          hipStream_t stream);
hipError_t launch_gemm_tiled(int64_t M, int64_t K, int64_t N, const void* W, const Layout& L, const void* x,
                             float* y, hipStream_t stream);

}  // namespace skg
