// Activation quantisation to Q8_1 blocks {fp16 d, fp16 s, int8 q[32]}: the
// standalone dispatch that feeds the Q8_1 integer-dot GEMVs (the per-block
// steps are quantize_block_q8_1).
#include "common.h"
#include "kernels.h"

namespace skg {

// One thread per block: 8 16-byte loads of x, one 36-byte store.
__global__ void quantize_q8_1_kernel(const float* __restrict__ x, uint8_t* __restrict__ xq, int64_t nblocks) {
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(x + b * QK);
  float v[QK];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const f32x4 t = src[p];
    v[4 * p + 0] = t.x;
    v[4 * p + 1] = t.y;
    v[4 * p + 2] = t.z;
    v[4 * p + 3] = t.w;
  }
  const Q8_1Block q = quantize_block_q8_1(v);
  uint32_t* dst = reinterpret_cast<uint32_t*>(xq + b * 36);
  dst[0] = q.d16 | (q.s16 << 16);
#pragma unroll
  for (int k = 0; k < 8; ++k) dst[1 + k] = q.q[k];
}

hipError_t launch_quantize_q8_1(int64_t M, int64_t K, const float* x, void* xq, hipStream_t stream) {
  const int64_t nblocks = M * (K / QK);
  const int threads = 64;
  const int64_t grid = (nblocks + threads - 1) / threads;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3(unsigned(grid)), dim3(threads), 0, stream, x,
                     static_cast<uint8_t*>(xq), nblocks);
  return hipGetLastError();
}

}  // namespace skg
