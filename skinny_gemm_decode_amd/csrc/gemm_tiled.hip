// Tiled prefill GEMM on MFMA: y[m][n] = sum_k W[n][k] x[m][k], q4_0 weights,
// bf16 activations, fp32 output.
//
// "Chapter 2.2 - speed - 64-lane Metal" (the tile) stops re-reading and
// re-unpacking the weights for every activation row: a workgroup decodes a
// weight tile once into on-chip memory and serves every row of its output
// tile from it; (the +1) pads each on-chip row so rows stop landing on the
// same bank.  On gfx950 the tile is:
//
// * block tile BM = 256 rows of x by BN = 16*NB16 weight rows, K in steps of
//   BK = 64 (two q4_0 blocks); 4 waves, wave w owns x rows [64w, 64w + 64).
// * each step, 2*BN threads decode one q4_0 block each to bf16
//   (w = bf16_rne(d * (c - 8))) into an LDS tile whose rows are padded by 16
//   bytes (row stride 144 bytes), double-buffered so one barrier per step
//   suffices and the decode of step s+1 overlaps the MFMAs of step s.
// * v_mfma_f32_16x16x32_bf16: A fragments (x) come straight from global
//   memory / L2 into registers one step ahead, B fragments (decoded weights)
//   from LDS; fp32 accumulators, 4 x NB16 16x16 tiles per wave.
//
// MFMA 16x16x32 operand layout (lane l, 0..63): A supplies row l%16, k
// 8*(l/16)..+7; B supplies column l%16, the same k; the 16x16 result gives
// lane l rows 4*(l/16)..+3 of column l%16.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace skg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int GT_BM = 256;
constexpr int GT_BK = 64;
constexpr int GT_LDS_ROW = GT_BK + 8;  // bf16 per LDS row: 128 data bytes + 16 pad bytes

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <int NB16>
__global__ __launch_bounds__(256) void gemm_q4_0_bf16_kernel(PackedW P, const uint16_t* __restrict__ A,
                                                             float* __restrict__ y, int M, int N, int K) {
  constexpr int BN = 16 * NB16;
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * GT_LDS_ROW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int mtiles = (M + GT_BM - 1) / GT_BM;
  const int m0 = (blockIdx.x % mtiles) * GT_BM;
  const int n0 = (blockIdx.x / mtiles) * BN;
  const int nbk = int(P.nb);  // q4_0 blocks per row
  const int steps = (K + GT_BK - 1) / GT_BK;

  // ---- weight decode: thread t < 2*BN owns (tile row t/2, block t%2) ----
  const bool dec = tid < 2 * BN;
  const int drow = tid >> 1;
  const int dblk = tid & 1;
  const int dn = min(n0 + drow, N - 1);
  const uint8_t* dpay = P.payload + size_t(dn) * P.row_bytes;
  const uint16_t* dsc = P.scales + size_t(dn) * P.nb;

  u32x4 wraw = {0u, 0u, 0u, 0u};
  uint32_t wsc = 0;
  auto load_w = [&](int s) {
    const int kb = s * 2 + dblk;
    if (dec && kb < nbk) {
      wraw = ld_u32x4(dpay + size_t(kb) * 16);
      wsc = dsc[kb];
    } else {
      wraw = u32x4{0u, 0u, 0u, 0u};
      wsc = 0;  // d = 0: the block decodes to zeros
    }
  };
  auto store_w = [&](int buf) {
    if (!dec) return;
    const float d = h2f(wsc);
    const float nd8 = -8.0f * d;
    const uint32_t pw[4] = {wraw.x, wraw.y, wraw.z, wraw.w};
    uint32_t o[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = pw[k] & 0x0F0F0F0Fu;
      const uint32_t hi = (pw[k] >> 4) & 0x0F0F0F0Fu;
      // (c - 8) * d is exact in fp32 (at most 15 significant bits); fma
      // forms it with a single rounding, then one RNE rounding to bf16.
      o[2 * k + 0] = pack_bf16x2(fmaf(float(lo & 0xFF), d, nd8), fmaf(float((lo >> 8) & 0xFF), d, nd8));
      o[2 * k + 1] = pack_bf16x2(fmaf(float((lo >> 16) & 0xFF), d, nd8), fmaf(float(lo >> 24), d, nd8));
      o[8 + 2 * k + 0] = pack_bf16x2(fmaf(float(hi & 0xFF), d, nd8), fmaf(float((hi >> 8) & 0xFF), d, nd8));
      o[8 + 2 * k + 1] = pack_bf16x2(fmaf(float((hi >> 16) & 0xFF), d, nd8), fmaf(float(hi >> 24), d, nd8));
    }
    u32x4* dst = reinterpret_cast<u32x4*>(&Bs[buf][drow * GT_LDS_ROW + dblk * 32]);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
  };

  // ---- activation fragments: lane supplies row l%16, k 8*(l/16)..+7 ----
  const int arow_base = m0 + wave * 64 + (lane & 15);
  const int akoff = (lane >> 4) * 8;
  u32x4 afr[2][4][2];  // [buffer][mi][kk]
  auto load_a = [&](int buf, int s) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int m = min(arow_base + mi * 16, M - 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = s * GT_BK + kk * 32 + akoff;
        if (k < K)
          afr[buf][mi][kk] = ld_u32x4(A + size_t(m) * size_t(K) + size_t(k));
        else
          afr[buf][mi][kk] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x4 acc[4][NB16];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_w(0);
  load_a(0, 0);
  store_w(0);
  __syncthreads();

  // One step: prefetch step s+1 (weights raw, activation fragments), run the
  // MFMAs of step s from LDS buffer CUR, decode step s+1 into the other
  // buffer, barrier.  CUR is a compile-time constant so the fragment double
  // buffer stays in registers.
  auto step = [&](auto cur_c, int s) {
    constexpr int CUR = decltype(cur_c)::value;
    const bool more = s + 1 < steps;
    if (more) {
      load_w(s + 1);
      load_a(CUR ^ 1, s + 1);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int nj = 0; nj < NB16; ++nj) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(
            &Bs[CUR][(nj * 16 + (lane & 15)) * GT_LDS_ROW + kk * 32 + akoff]);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, afr[CUR][mi][kk]);
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[mi][nj], 0, 0, 0);
        }
      }
    }
    if (more) store_w(CUR ^ 1);
    __syncthreads();
  };
  for (int s = 0; s < steps; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < steps) step(std::integral_constant<int, 1>{}, s + 1);
  }

  // ---- store: lane holds rows 4*(l/16)..+3 of column l%16 of each tile ----
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) {
      const int n = n0 + nj * 16 + (lane & 15);
      const float v[4] = {acc[mi][nj].x, acc[mi][nj].y, acc[mi][nj].z, acc[mi][nj].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wave * 64 + mi * 16 + (lane >> 4) * 4 + r;
        if (m < M && n < N) y[size_t(m) * size_t(N) + size_t(n)] = v[r];
      }
    }
  }
}

hipError_t launch_gemm_tiled(int64_t M, int64_t K, int64_t N, const void* W, const Layout& L, const void* x,
                             float* y, hipStream_t stream) {
  const PackedW P = packed_view(W, L);
  const int64_t mtiles = (M + GT_BM - 1) / GT_BM;
  // Tile width: 7 or 8 16-column groups, whichever leaves the fewest idle
  // compute units in the last wave of tiles (N = 14336, M = 512 -> 7: 256 tiles).
  const int64_t t7 = mtiles * ((N + 111) / 112), t8 = mtiles * ((N + 127) / 128);
  const int cus = 256;
  const double e7 = double(t7) / double(((t7 + cus - 1) / cus) * cus);
  const double e8 = double(t8) / double(((t8 + cus - 1) / cus) * cus);
  if (e7 > e8) {
    hipLaunchKernelGGL(gemm_q4_0_bf16_kernel<7>, dim3(unsigned(t7)), dim3(256), 0, stream, P,
                       static_cast<const uint16_t*>(x), y, int(M), int(N), int(K));
  } else {
    hipLaunchKernelGGL(gemm_q4_0_bf16_kernel<8>, dim3(unsigned(t8)), dim3(256), 0, stream, P,
                       static_cast<const uint16_t*>(x), y, int(M), int(N), int(K));
  }
  return hipGetLastError();
}

}  // namespace skg
