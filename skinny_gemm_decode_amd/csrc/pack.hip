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

// One thread per q4_K super-block (144 bytes, 2-byte aligned): the 16-byte
// header {d, dmin, scale bytes} goes to the header stream unchanged; each
// 32-element sub-block j (codes: the low nibbles of code bytes 32 (j / 2) ..
// +31 for even j, their high nibbles for odd j) becomes one 16-byte unit with
// element i in the low nibble of byte i and element 16 + i in its high nibble.
__global__ void pack_q4_K_kernel(const uint16_t* __restrict__ src, uint8_t* __restrict__ payload,
                                 uint16_t* __restrict__ heads, int64_t nsuper) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nsuper) return;
  const uint16_t* b = src + i * 72;
  uint32_t h[72];
#pragma unroll
  for (int k = 0; k < 72; ++k) h[k] = b[k];
  uint32_t* hd = reinterpret_cast<uint32_t*>(heads + i * 8);
#pragma unroll
  for (int k = 0; k < 4; ++k) hd[k] = h[2 * k] | (h[2 * k + 1] << 16);
  // code dwords: qs[4t .. 4t+3] = q[t], t = 0..31
  uint32_t q[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) q[t] = h[8 + 2 * t] | (h[8 + 2 * t + 1] << 16);
  uint8_t* out = payload + i * 8 * 16;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 lo, hi;
    uint32_t l[4], u[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t A = q[8 * c + t], B = q[8 * c + 4 + t];  // bytes 32c + 4t.., 32c + 16 + 4t..
      l[t] = (A & 0x0F0F0F0Fu) | ((B & 0x0F0F0F0Fu) << 4);
      u[t] = ((A >> 4) & 0x0F0F0F0Fu) | (B & 0xF0F0F0F0u);
    }
    lo = u32x4{l[0], l[1], l[2], l[3]};
    hi = u32x4{u[0], u[1], u[2], u[3]};
    *reinterpret_cast<u32x4*>(out + (2 * c) * 16) = lo;
    *reinterpret_cast<u32x4*>(out + (2 * c + 1) * 16) = hi;
  }
}

// One thread per q6_K super-block (210 bytes): each 32-element sub-block j
// is written as a 16-byte low unit (the low four bits of its codes, in the
// q4_0 order) and an 8-byte high unit (their top two bits, see Layout); the 16
// int8 scales and d go to their streams unchanged.  Element 32 j + t takes
// its low bits from nibble (j >> 1) & 1 of ql[64 (j >> 2) + 32 (j & 1) + t]
// and its high bits from bits 2 (j & 3) .. +1 of qh[32 (j >> 2) + t].
__global__ void pack_q6_K_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ payload,
                                 uint8_t* __restrict__ scales, uint16_t* __restrict__ dsup, int64_t nsuper,
                                 int64_t nb) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nsuper) return;
  const uint8_t* b = src + i * 210;
  const int64_t nsb = nb / 8;
  const int64_t row = i / nsb, sb = i % nsb;
  uint8_t* rp = payload + size_t(row) * size_t(nb) * 24;
#pragma unroll 1
  for (int j = 0; j < 8; ++j) {
    const uint8_t* lp = b + 64 * (j >> 2) + 32 * (j & 1);
    const int lsh = 4 * ((j >> 1) & 1);
    const uint8_t* hp = b + 128 + 32 * (j >> 2);
    const int hsh = 2 * (j & 3);
    uint32_t lo[4], hw[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t v = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int t0 = 4 * k + bb, t1 = 16 + 4 * k + bb;
        const uint32_t l0 = (uint32_t(lp[t0]) >> lsh) & 15u, l1 = (uint32_t(lp[t1]) >> lsh) & 15u;
        const uint32_t h0 = (uint32_t(hp[t0]) >> hsh) & 3u, h1 = (uint32_t(hp[t1]) >> hsh) & 3u;
        v |= (l0 | (l1 << 4)) << (8 * bb);
        hw[k >> 1] |= h0 << (8 * bb + 4 - 4 * (k & 1));
        hw[k >> 1] |= h1 << (8 * bb + 6 - 4 * (k & 1));
      }
      lo[k] = v;
    }
    const int64_t unit = sb * 8 + j;
    *reinterpret_cast<u32x4*>(rp + unit * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    uint32_t* hq = reinterpret_cast<uint32_t*>(rp + nb * 16 + unit * 8);
    hq[0] = hw[0];
    hq[1] = hw[1];
  }
  uint8_t* sp = scales + size_t(row) * size_t(nb) * 2 + sb * 16;
#pragma unroll
  for (int k = 0; k < 16; ++k) sp[k] = b[192 + k];
  dsup[i] = uint16_t(b[208] | (uint32_t(b[209]) << 8));
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
  if (wk == WK_Q4_K || wk == WK_Q6_K) {
    const int64_t nsuper = N * (K / QK_K);
    const int64_t sgrid = (nsuper + threads - 1) / threads;
    if (wk == WK_Q4_K)
      hipLaunchKernelGGL(pack_q4_K_kernel, dim3(unsigned(sgrid)), dim3(threads), 0, stream,
                         static_cast<const uint16_t*>(src), payload, scales, nsuper);
    else
      hipLaunchKernelGGL(pack_q6_K_kernel, dim3(unsigned(sgrid)), dim3(threads), 0, stream,
                         static_cast<const uint8_t*>(src), payload, reinterpret_cast<uint8_t*>(scales),
                         reinterpret_cast<uint16_t*>(payload + L.d_off), nsuper, L.nb);
    return hipGetLastError();
  }
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
