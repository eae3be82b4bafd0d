// Activation quantisation to Q8_1 blocks {fp16 d, fp16 s, int8 q[32]}.
//
// The RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach &
// Methodology) feeds Q8_1 activations to the Q4_0 integer-dot matvec, written
// either by a standalone quantisation dispatch (this kernel) or by the fused
// RMSNorm.  Per 32-element block, all in IEEE binary32 (the library is built
// without fast-math, so '/' is correctly rounded):
//   amax = max|x_i|, d = amax / 127, id = d != 0 ? 1 / d : 0,
//   q_i = round-half-away(x_i * id), stored d = fp16_rne(d),
//   stored s = fp16_rne(d * (float)sum_i q_i).
#include "common.h"
#include "kernels.h"

namespace skg {

// One thread per block: 8 16-byte loads of x, one 36-byte store.
__global__ void quantize_q8_1_kernel(const float* __restrict__ x, uint8_t* __restrict__ xq, int64_t nblocks) {
  // Every step below is one IEEE binary32 operation: no contraction, so that
  // fp16(d * sum) rounds the binary32 product, never the exact one (a fused
  // multiply-convert rounds once and differs on rare double-rounding ties).
#pragma clang fp contract(off)
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
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QK; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  int sum = 0;
  uint32_t packed[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = int(roundf(v[4 * k + i] * id));
      q = q > 127 ? 127 : (q < -127 ? -127 : q);
      sum += q;
      word |= (uint32_t(q) & 0xFFu) << (8 * i);
    }
    packed[k] = word;
  }
  const uint32_t dbits = __half_as_ushort(__float2half_rn(d));
  // The empty asm pins the binary32 product in a register: without it the
  // backend folds multiply and conversion into one v_fma_mix (one rounding).
  float sp = d * float(sum);
  asm volatile("" : "+v"(sp));
  const uint32_t sbits = __half_as_ushort(__float2half_rn(sp));
  uint32_t* dst = reinterpret_cast<uint32_t*>(xq + b * 36);
  dst[0] = dbits | (sbits << 16);
#pragma unroll
  for (int k = 0; k < 8; ++k) dst[1 + k] = packed[k];
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
