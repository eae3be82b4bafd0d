// Tiled prefill GEMM on the integer matrix cores: y[m][n] = sum_k W[n][k] a[m][k]
// with q4_0 or q8_0 weights and Q8_1 activations (the int8 arm of the
// dequantise-to-bf16/int8 prefill; "Chapter 2.2 - speed - 64-lane Metal", the
// tile, with the q4_0 x Q8_1 integer dot of the RX 6700 XT write-up, Approach &
// Methodology).
//
// Both operands carry one scale per 32-element block, so the product of a
// block is exact only as an integer: every v_mfma_i32_16x16x32_i8 covers
// exactly one block (K = 32) of a 16 x 16 output tile, and its int32 result is
// converted and scaled by dA[m] * dW[n] into the fp32 accumulator on the
// vector ALU (three operations per output per block).  That scaling is the
// cost this organisation adds over the bf16 tile, which folds the weight scale
// into its bf16 operand once per weight element.
//
// * block tile 256 rows of a by 16 * NB16 weight rows, K in steps of 64 (two
//   blocks); 4 waves, wave w owns rows [64 w, 64 w + 64) of the tile.
// * weights: 2 * BN threads each take one block per step from a PW-deep ring
//   of raw loads, write its 32 codes as int8 (q4_0: 16 (c - 8), its scale
//   divided by 16; q8_0: the codes) and the scale as binary32 into a
//   double-buffered LDS tile; one barrier per step.
// * activation: each wave copies its 64 rows x two Q8_1 blocks per step into
//   a wave-private LDS slice (codes at a 72-byte row stride, d as binary32),
//   one step ahead, and reads the MFMA A fragments and the d of its output
//   rows from there.
//
// MFMA 16x16x32 i8 operand layout (lane l): A supplies row l % 16, k
// 8 (l / 16) .. + 7; B supplies column l % 16, the same k; the result gives
// lane l rows 4 (l / 16) .. + 3 of column l % 16.
#include <utility>

#include "common.h"
#include "kernels.h"

namespace skg {

typedef int i32x4 __attribute__((ext_vector_type(4)));

static constexpr int GI_BM = 256;
static constexpr int GI_BROW = 80;  // LDS bytes per weight row: 2 x 32 codes + 16 pad
static constexpr int GI_AROW = 18;  // LDS dwords per activation row: 2 x 8 code dwords + 2 pad
static constexpr int GI_PW = 4;     // weight prefetch distance in K steps

static __device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int WK, int NB16, int PW>
__global__ __launch_bounds__(256) void gemm_q8_1_i8_kernel(PackedW P, const uint8_t* __restrict__ xq,
                                                           float* __restrict__ y, int M, int N, int K) {
  constexpr int BN = 16 * NB16;
  constexpr int NP = (WK == WK_Q8_0) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * GI_BROW];
  __shared__ float Ds[2][2][BN];
  __shared__ __attribute__((aligned(16))) uint32_t As[4][2][64 * GI_AROW];
  __shared__ __attribute__((aligned(16))) float DAs[4][2][2][64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int mtiles = (M + GI_BM - 1) / GI_BM;
  const int m0 = (blockIdx.x % mtiles) * GI_BM;
  const int n0 = (blockIdx.x / mtiles) * BN;
  const int nbk = int(P.nb);
  const int steps = K / 64;

  // ---- weights: thread t < 2 BN owns (tile row t / 2, block t % 2 of the step) ----
  const bool wthr = tid < 2 * BN;
  const int drow = wthr ? (tid >> 1) : 0;
  const int dblk = tid & 1;
  const int dn = min(n0 + drow, N - 1);
  const uint8_t* dpay = P.payload + size_t(dn) * P.row_bytes;
  const uint16_t* dsc = P.scales + size_t(dn) * P.nb;
  u32x4 wraw[PW][NP];
  uint32_t wsc[PW];
  bool wok[PW];
  auto load_w = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    const int kb = s * 2 + dblk;
    const int kc = min(kb, nbk - 1);
    wok[SL] = kb < nbk;
    if (!wthr) return;  // waves 2 and 3 when the tile has 64 rows: no weight block
#pragma unroll
    for (int p = 0; p < NP; ++p) wraw[SL][p] = ld_u32x4(dpay + (size_t(p) * size_t(nbk) + size_t(kc)) * 16);
    wsc[SL] = dsc[kc];
  };
  auto store_w = [&](auto slot_c, int buf) {
    constexpr int SL = decltype(slot_c)::value;
    u32x4 lo, hi;
    float d;
    if constexpr (WK == WK_Q4_0) {
      // 16 (c - 8) as int8: the nibble moved to the high half, its sign bit flipped
      const uint32_t w[4] = {wraw[SL][0].x, wraw[SL][0].y, wraw[SL][0].z, wraw[SL][0].w};
      uint32_t l[4], h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        l[k] = ((w[k] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;  // elements 4k .. 4k + 3
        h[k] = (w[k] & 0xF0F0F0F0u) ^ 0x80808080u;         // elements 16 + 4k ..
      }
      lo = u32x4{l[0], l[1], l[2], l[3]};
      hi = u32x4{h[0], h[1], h[2], h[3]};
      d = wok[SL] ? h2f(wsc[SL]) * 0.0625f : 0.0f;
    } else {
      lo = wraw[SL][0];
      hi = wraw[SL][1];
      d = wok[SL] ? h2f(wsc[SL]) : 0.0f;
    }
    if (wthr) {
      u32x4* dst = reinterpret_cast<u32x4*>(&Bs[buf][drow * GI_BROW + dblk * 32]);
      dst[0] = lo;
      dst[1] = hi;
      Ds[buf][dblk][drow] = d;
    }
  };

  // ---- activation slice: 64 rows x 2 blocks of this wave, one step ahead ----
  // load t of lane l takes dword j = i % 8 of the codes of block (i / 8) % 2
  // of row i / 16 (i = 64 t + l): 32 contiguous bytes per 8 lanes; the two
  // block headers of row r come from loads 16 and 17 (i = 64 (t - 16) + l:
  // row i / 2, block i % 2).
  const int mw = m0 + wave * 64;
  uint32_t araw[18];
  auto load_a = [&](int s) {
    const int ss = min(s, steps - 1);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = 64 * t + lane;
      const int r = i >> 4, blk = (i >> 3) & 1, j = i & 7;
      const int m = min(mw + r, M - 1);
      araw[t] = *reinterpret_cast<const uint32_t*>(xq + (size_t(m) * size_t(nbk) + size_t(2 * ss + blk)) * 36 + 4 +
                                                   size_t(j) * 4);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = 64 * t + lane;
      const int r = i >> 1, blk = i & 1;
      const int m = min(mw + r, M - 1);
      araw[16 + t] = *reinterpret_cast<const uint32_t*>(xq + (size_t(m) * size_t(nbk) + size_t(2 * ss + blk)) * 36);
    }
  };
  auto park_a = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = 64 * t + lane;
      const int r = i >> 4, blk = (i >> 3) & 1, j = i & 7;
      As[wave][buf][r * GI_AROW + blk * 8 + j] = araw[t];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = 64 * t + lane;
      DAs[wave][buf][i & 1][i >> 1] = h2f(araw[16 + t] & 0xFFFFu);
    }
  };

  float acc[4][NB16][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mi][nj][r] = 0.f;

  // prologue: ring filled, step 0 decoded and parked, step 1's slice requested
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (load_w(std::integral_constant<int, I>{}, I), ...);
  }(std::make_integer_sequence<int, PW>{});
  load_a(0);
  park_a(0);
  load_a(1);
  store_w(std::integral_constant<int, 0>{}, 0);
  load_w(std::integral_constant<int, 0>{}, PW);
  lds_sync();

  auto step = [&](auto cur_c, auto slot_c, int s) {
    constexpr int CUR = decltype(cur_c)::value;
    // fragments of step s
    uint64_t af[4][2], bf[NB16][2];
    f32x4 da[4][2];
    float dw[NB16][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        af[mi][blk] = *reinterpret_cast<const uint64_t*>(&As[wave][CUR][(mi * 16 + c) * GI_AROW + blk * 8 + 2 * g]);
        da[mi][blk] = *reinterpret_cast<const f32x4*>(&DAs[wave][CUR][blk][mi * 16 + 4 * g]);
      }
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        bf[nj][blk] = *reinterpret_cast<const uint64_t*>(&Bs[CUR][(nj * 16 + c) * GI_BROW + blk * 32 + 8 * g]);
        dw[nj][blk] = Ds[CUR][blk][nj * 16 + c];
      }
    // the slice of step s + 1 (requested one step ago) into the other buffer,
    // and the request of step s + 2
    park_a(CUR ^ 1);
    load_a(s + 2);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int nj = 0; nj < NB16; ++nj)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const i32x4 v = __builtin_amdgcn_mfma_i32_16x16x32_i8(long(af[mi][blk]), long(bf[nj][blk]),
                                                                i32x4{0, 0, 0, 0}, 0, 0, 0);
          const f32x4 sc = da[mi][blk] * dw[nj][blk];
          acc[mi][nj][0] = fmaf(float(v.x), sc.x, acc[mi][nj][0]);
          acc[mi][nj][1] = fmaf(float(v.y), sc.y, acc[mi][nj][1]);
          acc[mi][nj][2] = fmaf(float(v.z), sc.z, acc[mi][nj][2]);
          acc[mi][nj][3] = fmaf(float(v.w), sc.w, acc[mi][nj][3]);
        }
    store_w(slot_c, CUR ^ 1);
    load_w(slot_c, s + 1 + PW);
    lds_sync();
  };
  constexpr int U = (PW % 2 == 0) ? PW : 2 * PW;
  for (int s0 = 0; s0 < steps; s0 += U) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((s0 + I < steps ? step(std::integral_constant<int, I % 2>{}, std::integral_constant<int, (I + 1) % PW>{},
                              s0 + I)
                       : void()),
       ...);
    }(std::make_integer_sequence<int, U>{});
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) {
      const int n = n0 + nj * 16 + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mw + mi * 16 + 4 * g + r;
        if (m < M && n < N) y[size_t(m) * size_t(N) + size_t(n)] = acc[mi][nj][r];
      }
    }
}

hipError_t launch_gemm_i8(int64_t M, int64_t K, int64_t N, const void* W, const Layout& L, const void* xq, float* y,
                          hipStream_t stream) {
  const PackedW P = packed_view(W, L);
  constexpr int NB16 = 4;  // 64 weight rows per tile
  const int64_t mtiles = (M + GI_BM - 1) / GI_BM;
  const unsigned grid = unsigned(mtiles * ((N + 16 * NB16 - 1) / (16 * NB16)));
  const uint8_t* x = static_cast<const uint8_t*>(xq);
  if (L.wk == WK_Q8_0)
    hipLaunchKernelGGL((gemm_q8_1_i8_kernel<WK_Q8_0, NB16, GI_PW>), dim3(grid), dim3(256), 0, stream, P, x, y, int(M),
                       int(N), int(K));
  else
    hipLaunchKernelGGL((gemm_q8_1_i8_kernel<WK_Q4_0, NB16, GI_PW>), dim3(grid), dim3(256), 0, stream, P, x, y, int(M),
                       int(N), int(K));
  return hipGetLastError();
}

}  // namespace skg
