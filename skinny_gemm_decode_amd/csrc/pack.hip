// Load-time weight repacking: canonical blocks -> 16-byte-aligned payload
// units plus a separate fp16 scale stream.
//
// "The Shape That Actually Matters" (Round 1, Round 2) re-lays the weights out
// once at load time so the decode GEMV's loads coalesce; "Six hypotheses,
// four refutations" (What the failure left behind) has every lane stream whole
// q4_0 blocks through wide loads.  An 18-byte (q4_0) or 34-byte (q8_0) block
// cannot be read with aligned 16-byte loads, so the codes and the scales are
// split apart; the payload keeps K order inside each row.  This is a pure
// byte permutation: the packed buffer holds exactly the canonical bits.
#include "common.h"
#include "kernels.h"

namespace skg {

// One thread per q4_0 block: 18 bytes at a 2-byte-aligned address in, one
// 16-byte payload unit and one fp16 scale out.
__global__ void pack_q4_0_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ payload,
                                 uint16_t* __restrict__ scales, int64_t nblocks) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const uint16_t* b = src + i * 9;
  uint32_t h[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) h[k] = b[k];
  scales[i] = uint16_t(h[0]);
  u32x4 p;
  p.x = h[1] | (h[2] << 16);
  p.y = h[3] | (h[4] << 16);
  p.z = h[5] | (h[6] << 16);
  p.w = h[7] | (h[8] << 16);
  *reinterpret_cast<u32x4*>(payload + i * 16) = p;
}

// One thread per q8_0 block: codes 0..15 go to plane 0 of the row, codes
// 16..31 to plane 1 (row = i / nb, block = i % nb).
__global__ void pack_q8_0_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ payload,
                                 uint16_t* __restrict__ scales, int64_t nblocks, int64_t nb) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const uint16_t* b = src + i * 17;
  uint32_t h[17];
#pragma unroll
  for (int k = 0; k < 17; ++k) h[k] = b[k];
  scales[i] = uint16_t(h[0]);
  const int64_t row = i / nb, blk = i % nb;
  uint8_t* rp = payload + row * nb * 32;
  u32x4 p0, p1;
  p0.x = h[1] | (h[2] << 16);
  p0.y = h[3] | (h[4] << 16);
  p0.z = h[5] | (h[6] << 16);
  p0.w = h[7] | (h[8] << 16);
  p1.x = h[9] | (h[10] << 16);
  p1.y = h[11] | (h[12] << 16);
  p1.z = h[13] | (h[14] << 16);
  p1.w = h[15] | (h[16] << 16);
  *reinterpret_cast<u32x4*>(rp + blk * 16) = p0;
  *reinterpret_cast<u32x4*>(rp + (nb + blk) * 16) = p1;
}

hipError_t launch_pack(int wk, int64_t N, int64_t K, const void* src, void* dst, hipStream_t stream) {
  const Layout L = layout_of(wk, N, K);
  if (wk == WK_BF16) {
    // The canonical bf16 row is already the packed row.
    return hipMemcpyAsync(dst, src, L.payload_bytes, hipMemcpyDeviceToDevice, stream);
  }
  const int64_t nblocks = N * L.nb;
  uint8_t* payload = static_cast<uint8_t*>(dst);
  uint16_t* scales = reinterpret_cast<uint16_t*>(payload + L.scale_off);
  const int threads = 256;
  const int64_t grid = (nblocks + threads - 1) / threads;
  if (wk == WK_Q4_0) {
    hipLaunchKernelGGL(pack_q4_0_kernel, dim3(unsigned(grid)), dim3(threads), 0, stream,
                       static_cast<const uint16_t*>(src), payload, scales, nblocks);
  } else {
    hipLaunchKernelGGL(pack_q8_0_kernel, dim3(unsigned(grid)), dim3(threads), 0, stream,
                       static_cast<const uint16_t*>(src), payload, scales, nblocks, L.nb);
  }
  return hipGetLastError();
}

}  // namespace skg
