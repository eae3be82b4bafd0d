// Tiled prefill GEMM on MFMA: y[m][n] = sum_k W[n][k] x[m][k], q4_0 weights
// (q8_0, q4_K and q6_K on the pipelined organisation), bf16 activations, fp32
// output.
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
#include <utility>

#include "common.h"
#include "kernels.h"

namespace skg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

constexpr int GT_BM = 256;
constexpr int GT_BK = 64;
constexpr int GT_LDS_ROW = GT_BK + 8;  // bf16 per LDS row: 128 data bytes + 16 pad bytes
constexpr int GT_PW = 4;              // weight prefetch distance in K steps

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Workgroup barrier for the LDS tile only: waits for this wave's LDS
// accesses, not for its outstanding global loads (the weight prefetch ring
// must stay in flight across the barrier).
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NB16, int PW>
__global__ __launch_bounds__(256) void gemm_q4_0_bf16_kernel(PackedW P, const uint16_t* __restrict__ A,
                                                             float* __restrict__ y, int M, int N, int K) {
  constexpr int BN = 16 * NB16;
  // 128 LDS rows whatever BN: threads past the tile's 2*BN blocks decode a
  // clamped duplicate into rows that are never read, so no thread branches.
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * GT_LDS_ROW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int mtiles = (M + GT_BM - 1) / GT_BM;
  const int m0 = (blockIdx.x % mtiles) * GT_BM;
  const int n0 = (blockIdx.x / mtiles) * BN;
  const int nbk = int(P.nb);  // q4_0 blocks per row
  const int steps = (K + GT_BK - 1) / GT_BK;

  // ---- weight decode: thread t owns (tile row t/2, block t%2 of the step) ----
  const int drow = tid >> 1;
  const int dblk = tid & 1;
  const int dn = min(n0 + drow, N - 1);
  const uint8_t* dpay = P.payload + size_t(dn) * P.row_bytes;
  const uint16_t* dsc = P.scales + size_t(dn) * P.nb;

  // Ring of PW raw blocks: the block of step s is requested PW steps before
  // it is decoded, which covers HBM latency with one wave per SIMD.  A block
  // past the end of K reads the last block and decodes with scale 0.  The
  // loads are ordinary (cached) loads: a step takes 32 bytes of each row, so
  // one 128-byte line serves four consecutive steps, and a streaming hint
  // lets it be evicted in between (measured on MI355X at M=512, K=4096,
  // N=14336: 84 -> 72 us).
  u32x4 wraw[PW];
  uint32_t wsc[PW];
  bool wok[PW];
  auto load_w = [&](auto slot_c, int s) {
    constexpr int SL = decltype(slot_c)::value;
    const int kb = s * 2 + dblk;
    const int kc = min(kb, nbk - 1);
    wraw[SL] = ld_u32x4(dpay + size_t(kc) * 16);
    wsc[SL] = dsc[kc];
    wok[SL] = kb < nbk;
  };
  auto store_w = [&](auto slot_c, int buf) {
    constexpr int SL = decltype(slot_c)::value;
    const float d = wok[SL] ? h2f(wsc[SL]) : 0.0f;
    const float nd8 = -8.0f * d;
    const uint32_t pw[4] = {wraw[SL].x, wraw[SL].y, wraw[SL].z, wraw[SL].w};
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
  // Past the end of K the fragment reads the last 8 columns; the weights
  // there decode to zero, so it contributes exactly 0.
  const int arow_base = m0 + wave * 64 + (lane & 15);
  const int akoff = (lane >> 4) * 8;
  u32x4 afr[2][4][2];  // [buffer][mi][kk]
  auto load_a = [&](auto buf_c, int s) {
    constexpr int BUF = decltype(buf_c)::value;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int m = min(arow_base + mi * 16, M - 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = min(s * GT_BK + kk * 32 + akoff, K - 8);
        afr[BUF][mi][kk] = ld_u32x4(A + size_t(m) * size_t(K) + size_t(k));
      }
    }
  };

  f32x4 acc[4][NB16];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: fill the ring, decode step 0, refill its slot
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (load_w(std::integral_constant<int, I>{}, I), ...);
  }(std::make_integer_sequence<int, PW>{});
  load_a(std::integral_constant<int, 0>{}, 0);
  store_w(std::integral_constant<int, 0>{}, 0);
  load_w(std::integral_constant<int, 0>{}, PW);
  lds_barrier();

  // Step s: activation fragments of s+1 requested; the B fragments of s read
  // from LDS; the MFMAs of s; the raw block of s+1 (requested PW steps ago)
  // decoded into the other LDS buffer and its ring slot refilled with s+1+PW;
  // one barrier.  CUR and SLOT are compile-time constants.
  auto step = [&](auto cur_c, auto slot_c, int s) {
    constexpr int CUR = decltype(cur_c)::value;
    constexpr int SLOT = decltype(slot_c)::value;  // ring slot of step s+1
    load_a(std::integral_constant<int, CUR ^ 1>{}, s + 1);
    u32x4 bfr[2][NB16];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nj = 0; nj < NB16; ++nj)
        bfr[kk][nj] = *reinterpret_cast<const u32x4*>(&Bs[CUR][(nj * 16 + (lane & 15)) * GT_LDS_ROW + kk * 32 + akoff]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nj = 0; nj < NB16; ++nj) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, bfr[kk][nj]);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, afr[CUR][mi][kk]);
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[mi][nj], 0, 0, 0);
        }
      }
    store_w(slot_c, CUR ^ 1);
    load_w(slot_c, s + 1 + PW);
    lds_barrier();
  };
  constexpr int U = (PW % 2 == 0) ? PW : 2 * PW;  // steps per unrolled iteration
  for (int s0 = 0; s0 < steps; s0 += U) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((s0 + I < steps ? step(std::integral_constant<int, I % 2>{}, std::integral_constant<int, (I + 1) % PW>{},
                              s0 + I)
                       : void()),
       ...);
    }(std::make_integer_sequence<int, U>{});
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

// Producer/consumer variant: CW consumer waves and 4 producer waves per
// workgroup.  The consumer waves own the output rows (BM / CW each: activation
// slices staged through LDS, B fragments from LDS, MFMAs); the producer waves
// own the weight stream (the PW-deep ring of raw blocks and the decode into
// LDS).  With CW = 4 each SIMD runs one wave of each kind, so decode VALU work
// and MFMAs overlap; with CW = 8 each SIMD also has two MFMA waves, so one
// wave's LDS and barrier waits are covered by the other's MFMAs (at the cost
// of reading each B fragment twice as often).
template <int NB16, int PW, int CW>
__global__ __launch_bounds__((CW + 4) * 64) void gemm_q4_0_bf16_pc_kernel(PackedW P, const uint16_t* __restrict__ A,
                                                                          float* __restrict__ y, int M, int N, int K) {
  constexpr int BN = 16 * NB16;
  constexpr int MI = 16 / CW;        // 16-row groups per consumer wave (4 or 2)
  constexpr int WR = 16 * MI;        // rows per consumer wave
  constexpr int AL = WR / 8;         // 16-byte activation loads per lane per step
  static_assert(CW == 4 || CW == 8, "4 or 8 consumer waves");
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * GT_LDS_ROW];
  // CW waves x 2 steps x WR rows x 128 B of activation slices
  __shared__ __attribute__((aligned(16))) uint8_t As_raw[CW * 2 * WR * 8 * 16];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int mtiles = (M + GT_BM - 1) / GT_BM;
  const int m0 = (blockIdx.x % mtiles) * GT_BM;
  const int n0 = (blockIdx.x / mtiles) * BN;
  const int nbk = int(P.nb);
  const int steps = (K + GT_BK - 1) / GT_BK;
  constexpr int U = (PW % 2 == 0) ? PW : 2 * PW;

  if (wave >= CW) {
    // ---------------- producer: weight ring + decode ----------------
    const int ptid = tid - CW * 64;
    const int drow = ptid >> 1;
    const int dblk = ptid & 1;
    const int dn = min(n0 + drow, N - 1);
    const uint8_t* dpay = P.payload + size_t(dn) * P.row_bytes;
    const uint16_t* dsc = P.scales + size_t(dn) * P.nb;
    u32x4 wraw[PW];
    uint32_t wsc[PW];
    bool wok[PW];
    auto load_w = [&](auto slot_c, int s) {
      constexpr int SL = decltype(slot_c)::value;
      const int kb = s * 2 + dblk;
      const int kc = min(kb, nbk - 1);
      wraw[SL] = ld_u32x4(dpay + size_t(kc) * 16);
      wsc[SL] = dsc[kc];
      wok[SL] = kb < nbk;
    };
    auto store_w = [&](auto slot_c, int buf) {
      constexpr int SL = decltype(slot_c)::value;
      const float d = wok[SL] ? h2f(wsc[SL]) : 0.0f;
      const float nd8 = -8.0f * d;
      const uint32_t pw[4] = {wraw[SL].x, wraw[SL].y, wraw[SL].z, wraw[SL].w};
      uint32_t o[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo = pw[k] & 0x0F0F0F0Fu;
        const uint32_t hi = (pw[k] >> 4) & 0x0F0F0F0Fu;
        o[2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(lo), d, nd8), fmaf(cvt_ubyte<1>(lo), d, nd8));
        o[2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(lo), d, nd8), fmaf(cvt_ubyte<3>(lo), d, nd8));
        o[8 + 2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(hi), d, nd8), fmaf(cvt_ubyte<1>(hi), d, nd8));
        o[8 + 2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(hi), d, nd8), fmaf(cvt_ubyte<3>(hi), d, nd8));
      }
      u32x4* dst = reinterpret_cast<u32x4*>(&Bs[buf][drow * GT_LDS_ROW + dblk * 32]);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    };
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (load_w(std::integral_constant<int, I>{}, I), ...);
    }(std::make_integer_sequence<int, PW>{});
    store_w(std::integral_constant<int, 0>{}, 0);
    load_w(std::integral_constant<int, 0>{}, PW);
    lds_barrier();
    auto pstep = [&](auto cur_c, auto slot_c, int s) {
      constexpr int CUR = decltype(cur_c)::value;
      store_w(slot_c, CUR ^ 1);
      load_w(slot_c, s + 1 + PW);
      lds_barrier();
    };
    for (int s0 = 0; s0 < steps; s0 += U) {
      [&]<int... I>(std::integer_sequence<int, I...>) {
        ((s0 + I < steps ? pstep(std::integral_constant<int, I % 2>{}, std::integral_constant<int, (I + 1) % PW>{},
                                 s0 + I)
                         : void()),
         ...);
      }(std::make_integer_sequence<int, U>{});
    }
    return;
  }

  // ---------------- consumer: activation slice + MFMA ----------------
  // Each consumer wave loads its own WR rows x 64 columns of x per step with
  // full-cache-line loads (instruction i: rows 8i..8i+7, 128 contiguous bytes
  // each), parks them in a wave-private LDS slice, and reads the MFMA
  // fragments from there.  Slot of (row r, 16-byte chunk c) =
  // 8r + (c ^ ((r >> 1) & 7)): a fragment read takes one chunk of 16
  // consecutive rows; rows of equal parity share a half of the 64 banks (a
  // row is 128 bytes), and within each parity the 8 rows' chunks land on 8
  // different 4-bank groups, so the 16 reads cover all 64 banks once.  Only the owning
  // wave touches its slice, and a wave's LDS operations complete in order, so
  // the slice needs no barrier.  Rows past M read row M-1; columns past K read
  // the last 8 (their weights decode to zero).
  constexpr int SLICE = WR * 8;  // 16-byte slots per step
  u32x4* As = reinterpret_cast<u32x4*>(As_raw) + wave * (2 * SLICE);
  const int mw = m0 + wave * WR;
  u32x4 araw[AL];
  auto load_a = [&](int s) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int m = min(mw + r, M - 1);
      const int k = min(s * GT_BK + (lane & 7) * 8, K - 8);
      araw[i] = ld_u32x4(A + size_t(m) * size_t(K) + size_t(k));
    }
  };
  auto park_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int c = lane & 7;
      As[buf * SLICE + r * 8 + (c ^ ((r >> 1) & 7))] = araw[i];
    }
  };
  f32x4 acc[MI][NB16];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};
  load_a(0);
  park_a(0);
  load_a(1);
  lds_barrier();
  auto cstep = [&](auto cur_c, int s) {
    constexpr int CUR = decltype(cur_c)::value;
    park_a(CUR ^ 1);  // slice of step s+1 (loaded one step ago)
    load_a(s + 2);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 afr[MI], bfr[NB16];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = mi * 16 + (lane & 15);
        const int c = kk * 4 + (lane >> 4);
        afr[mi] = As[CUR * SLICE + r * 8 + (c ^ ((r >> 1) & 7))];
      }
#pragma unroll
      for (int nj = 0; nj < NB16; ++nj)
        bfr[nj] = *reinterpret_cast<const u32x4*>(&Bs[CUR][(nj * 16 + (lane & 15)) * GT_LDS_ROW + kk * 32 + (lane >> 4) * 8]);
#pragma unroll
      for (int nj = 0; nj < NB16; ++nj) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, bfr[nj]);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, afr[mi]);
          acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[mi][nj], 0, 0, 0);
        }
      }
    }
    lds_barrier();
  };
  for (int s0 = 0; s0 < steps; s0 += U) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((s0 + I < steps ? cstep(std::integral_constant<int, I % 2>{}, s0 + I) : void()), ...);
    }(std::make_integer_sequence<int, U>{});
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) {
      const int n = n0 + nj * 16 + (lane & 15);
      const float v[4] = {acc[mi][nj].x, acc[mi][nj].y, acc[mi][nj].z, acc[mi][nj].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mw + mi * 16 + (lane >> 4) * 4 + r;
        if (m < M && n < N) y[size_t(m) * size_t(N) + size_t(n)] = v[r];
      }
    }
  }
}

// Pipelined producer/consumer variant: 4 consumer waves of 64 rows and 4
// producer waves, with the decoded weight tile triple-buffered so a consumer
// reads the MFMA fragments of the next half-step while the MFMAs of the
// current one run (in the one-barrier-per-step kernel above, every consumer
// reads its fragments right after the barrier and then multiplies, so LDS
// reads and MFMAs alternate instead of overlapping).  Step s: the producers
// decode step s+2 into buffer (s+2) % 3; the consumers park the activation
// slice of step s+1, request that of step s+2, and run
//   read (s, second half) | MFMA (s, first half) | read (s+1, first half) |
//   MFMA (s, second half) | barrier.
//
// With ADMA the activation slices are copied straight from global memory into
// LDS (global_load_lds_dwordx4: no registers, no LDS store instructions) into a
// ring of three slots per consumer wave; the copy of step s+2 is issued at the
// start of step s and waited for (vector-memory counter, in order) just before
// the fragments of step s+1 are read.  Each lane fetches the chunk whose
// swizzled slot is its own destination, so the slots keep the swizzled
// layout the fragment reads expect.
// WK selects the weight format: q4_0 (one 16-byte unit per block), q8_0
// (two planes of 16 bytes per block: codes 0-15 and 16-31), q4_K (the 16-byte
// unit of a 32-element sub-block and its super-block header) or q6_K (the
// low unit, the 8-byte high unit, the int8 scale pair and d).
template <int NB16, int PW, bool ADMA, int WK = WK_Q4_0>
__global__ __launch_bounds__(512) void gemm_q4_0_bf16_pipe_kernel(PackedW P, const uint16_t* __restrict__ A,
                                                                  float* __restrict__ y, int M, int N, int K) {
  static_assert(WK == WK_Q4_0 || WK == WK_Q8_0 || WK == WK_Q4_K || WK == WK_Q6_K, "weight format");
  constexpr int NPL = (WK == WK_Q4_0) ? 1 : 2;  // 16-byte words held per block
  constexpr int BN = 16 * NB16;
  constexpr int ASLOTS = ADMA ? 3 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t Bs[3][128 * GT_LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t As_raw[4 * ASLOTS * 64 * 8 * 16];

  const int tid = threadIdx.x;
  // wave-uniform (scalar registers): the copy bases below derive from it
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int mtiles = (M + GT_BM - 1) / GT_BM;
  const int m0 = (blockIdx.x % mtiles) * GT_BM;
  const int n0 = (blockIdx.x / mtiles) * BN;
  const int nbk = int(P.nb);
  const int steps = (K + GT_BK - 1) / GT_BK;
  // steps per unrolled iteration: ring slot (mod PW), weight buffer (mod 3)
  // and activation slot / fragment set (mod 2) all compile-time
  constexpr int U = (PW % 3 == 0 ? PW : 3 * PW) * (PW % 2 == 0 ? 1 : 2);

  if (wave >= 4) {
    // ---------------- producer: weight ring + decode, two steps ahead ----------------
    // Thread (row, block): each 16-lane group writes one block of 16
    // consecutive tile rows, whose 144-byte rows start on 16 different 4-bank
    // groups, so every 16-byte store instruction covers the 64 banks once.
    const int ptid = tid - 256;
    const int drow = (ptid & 15) + 16 * (ptid >> 5);
    const int dblk = (ptid >> 4) & 1;
    const int dn = min(n0 + drow, N - 1);
    const uint8_t* dpay = P.payload + size_t(dn) * P.row_bytes;
    const uint16_t* dsc = P.scales + size_t(dn) * P.nb;
    const uint16_t* dsup = (WK == WK_Q6_K) ? P.dsup + size_t(dn) * (P.nb / 8) : nullptr;
    u32x4 wraw[PW][NPL];
    uint32_t wsc[PW];
    bool wok[PW];
    auto load_w = [&](auto slot_c, int s) SKG_INL {
      constexpr int SL = decltype(slot_c)::value;
      const int kb = s * 2 + dblk;
      const int kc = min(kb, nbk - 1);
      if constexpr (WK == WK_Q4_K) {
        wraw[SL][0] = ld_u32x4(dpay + size_t(kc) * 16);
        wraw[SL][1] = ld_u32x4(dsc + size_t(kc >> 3) * 8);  // super-block header
        wsc[SL] = uint32_t(kc) & 7u;                          // sub-block index
      } else if constexpr (WK == WK_Q6_K) {
        wraw[SL][0] = ld_u32x4(dpay + size_t(kc) * 16);
        const uint32_t* hp = reinterpret_cast<const uint32_t*>(dpay + size_t(nbk) * 16 + size_t(kc) * 8);
        wraw[SL][1] = u32x4{hp[0], hp[1], dsc[kc], dsup[kc >> 3]};
      } else {
#pragma unroll
        for (int p = 0; p < NPL; ++p) wraw[SL][p] = ld_u32x4(dpay + (size_t(p) * size_t(nbk) + size_t(kc)) * 16);
        wsc[SL] = dsc[kc];
      }
      wok[SL] = kb < nbk;
    };
    // o[j] = bf16 pair (element 2j, element 2j+1) of the block, each
    // bf16_rne(d * code) with the product exact in fp32 (fma: one rounding).
    auto store_w = [&](auto slot_c, auto buf_c) SKG_INL {
      constexpr int SL = decltype(slot_c)::value;
      constexpr int BUF = decltype(buf_c)::value;
      uint32_t o[16];
      if constexpr (WK == WK_Q4_K) {
        // w = fp32_rn(a q - b), a = d sc_j, b = dmin m_j (both exact), q in
        // the q4_0 unit order
        uint32_t sc, m;
        q4_K_sc_m(wraw[SL][1].y, wraw[SL][1].z, wraw[SL][1].w, wsc[SL], sc, m);
        const float a = wok[SL] ? h2f(wraw[SL][1].x & 0xFFFFu) * float(sc) : 0.0f;
        const float nb = wok[SL] ? -(h2f(wraw[SL][1].x >> 16) * float(m)) : 0.0f;
        const uint32_t pw[4] = {wraw[SL][0].x, wraw[SL][0].y, wraw[SL][0].z, wraw[SL][0].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo = pw[k] & 0x0F0F0F0Fu;
          const uint32_t hi = (pw[k] >> 4) & 0x0F0F0F0Fu;
          o[2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(lo), a, nb), fmaf(cvt_ubyte<1>(lo), a, nb));
          o[2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(lo), a, nb), fmaf(cvt_ubyte<3>(lo), a, nb));
          o[8 + 2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(hi), a, nb), fmaf(cvt_ubyte<1>(hi), a, nb));
          o[8 + 2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(hi), a, nb), fmaf(cvt_ubyte<3>(hi), a, nb));
        }
      } else if constexpr (WK == WK_Q6_K) {
        // w = fp32_rn(a (q - 32)), a = d * scale of the half (exact)
        const float d = h2f(wraw[SL][1].w);
        const uint32_t sc = wraw[SL][1].z;
        const float alo = wok[SL] ? d * float(int8_t(sc & 0xFFu)) : 0.0f;
        const float ahi = wok[SL] ? d * float(int8_t(sc >> 8)) : 0.0f;
        const float nlo = -32.0f * alo, nhi = -32.0f * ahi;
        const uint32_t lw[4] = {wraw[SL][0].x, wraw[SL][0].y, wraw[SL][0].z, wraw[SL][0].w};
        const uint32_t hw[2] = {wraw[SL][1].x, wraw[SL][1].y};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t ca, cb;
          q6_K_codes(lw, hw, k, ca, cb);
          o[2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(ca), alo, nlo), fmaf(cvt_ubyte<1>(ca), alo, nlo));
          o[2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(ca), alo, nlo), fmaf(cvt_ubyte<3>(ca), alo, nlo));
          o[8 + 2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(cb), ahi, nhi), fmaf(cvt_ubyte<1>(cb), ahi, nhi));
          o[8 + 2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(cb), ahi, nhi), fmaf(cvt_ubyte<3>(cb), ahi, nhi));
        }
      } else if constexpr (WK == WK_Q4_0) {
        // w = d (c - 8); element i < 16 is the low nibble of byte i, i + 16
        // its high nibble.  Each nibble pair becomes two exact fp16 values by
        // one mask-and-or: 1024 + c (low nibbles) or 1024 + 16 c (high
        // nibbles, still in place), and one mixed-precision fma per element
        // gives the exact fp32 product: (1024 + c) d - 1032 d and
        // (1024 + 16 c) (d / 16) - 72 d, where 1032 d, 72 d and d / 16 are
        // exact in fp32 (d has 11 significant bits).
        const float d = wok[SL] ? h2f(wsc[SL]) : 0.0f;
        const float d16 = d * 0.0625f;
        const float blo = -1032.0f * d, bhi = -72.0f * d;
        const uint32_t pw[4] = {wraw[SL][0].x, wraw[SL][0].y, wraw[SL][0].z, wraw[SL][0].w};
        // masks and the exponent pattern as register operands, so each
        // mask-and-or is one v_and_or_b32 (it takes no two literals)
        uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
        asm volatile("" : "+s"(mlo));
        asm volatile("" : "+s"(mhi));
        asm volatile("" : "+v"(magic));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t v = pw[k], v8 = pw[k] >> 8;
          // elements 4k, 4k+2 | 4k+1, 4k+3 | 16+4k, 16+4k+2 | 16+4k+1, 16+4k+3
          const h16x2 l02 = __builtin_bit_cast(h16x2, (v & mlo) | magic);
          const h16x2 l13 = __builtin_bit_cast(h16x2, (v8 & mlo) | magic);
          const h16x2 h02 = __builtin_bit_cast(h16x2, (v & mhi) | magic);
          const h16x2 h13 = __builtin_bit_cast(h16x2, (v8 & mhi) | magic);
          o[2 * k + 0] = pack_bf16x2(fmaf(float(l02[0]), d, blo), fmaf(float(l13[0]), d, blo));
          o[2 * k + 1] = pack_bf16x2(fmaf(float(l02[1]), d, blo), fmaf(float(l13[1]), d, blo));
          o[8 + 2 * k + 0] = pack_bf16x2(fmaf(float(h02[0]), d16, bhi), fmaf(float(h13[0]), d16, bhi));
          o[8 + 2 * k + 1] = pack_bf16x2(fmaf(float(h02[1]), d16, bhi), fmaf(float(h13[1]), d16, bhi));
        }
      } else {
        // w = d q; q + 128 is the unsigned byte of q ^ 0x80, so w = d (u - 128)
        const float d = wok[SL] ? h2f(wsc[SL]) : 0.0f;
        const float nd128 = -128.0f * d;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t pw[4] = {wraw[SL][p].x ^ 0x80808080u, wraw[SL][p].y ^ 0x80808080u,
                                  wraw[SL][p].z ^ 0x80808080u, wraw[SL][p].w ^ 0x80808080u};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            o[8 * p + 2 * k + 0] = pack_bf16x2(fmaf(cvt_ubyte<0>(pw[k]), d, nd128), fmaf(cvt_ubyte<1>(pw[k]), d, nd128));
            o[8 * p + 2 * k + 1] = pack_bf16x2(fmaf(cvt_ubyte<2>(pw[k]), d, nd128), fmaf(cvt_ubyte<3>(pw[k]), d, nd128));
          }
        }
      }
      u32x4* dst = reinterpret_cast<u32x4*>(&Bs[BUF][drow * GT_LDS_ROW + dblk * 32]);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    };
    using std::integral_constant;
    [&]<int... I>(std::integer_sequence<int, I...>) SKG_INL {
      (load_w(integral_constant<int, I>{}, I), ...);
    }(std::make_integer_sequence<int, PW>{});
    store_w(integral_constant<int, 0>{}, integral_constant<int, 0>{});
    load_w(integral_constant<int, 0>{}, PW);
    store_w(integral_constant<int, 1 % PW>{}, integral_constant<int, 1>{});
    load_w(integral_constant<int, 1 % PW>{}, PW + 1);
    lds_barrier();
    auto pstep = [&](auto slot_c, auto buf_c, int s) SKG_INL {
      store_w(slot_c, buf_c);
      load_w(slot_c, s + 2 + PW);
      lds_barrier();
    };
    for (int s0 = 0; s0 < steps; s0 += U) {
      [&]<int... I>(std::integer_sequence<int, I...>) SKG_INL {
        ((s0 + I < steps ? pstep(integral_constant<int, (I + 2) % PW>{}, integral_constant<int, (I + 2) % 3>{},
                                 s0 + I)
                         : void()),
         ...);
      }(std::make_integer_sequence<int, U>{});
    }
    return;
  }

  // ---------------- consumer: activation slice + fragments + MFMA ----------------
  // Activation slices as in the kernel above (wave-private, swizzled).
  u32x4* As = reinterpret_cast<u32x4*>(As_raw) + wave * (ASLOTS * 64 * 8);
  // wave-uniform (the copy destination is a scalar register)
  const uint32_t as_lds =
      __builtin_amdgcn_readfirstlane(lds_addr(As_raw) + uint32_t(wave) * (ASLOTS * 64 * 8 * 16));
  const int mw = m0 + wave * 64;
  u32x4 araw[8];
  auto load_a = [&](int s) SKG_INL {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int m = min(mw + r, M - 1);
      const int k = min(s * GT_BK + (lane & 7) * 8, K - 8);
      araw[i] = ld_u32x4(A + size_t(m) * size_t(K) + size_t(k));
    }
  };
  auto park_a = [&](int slot) SKG_INL {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int c = lane & 7;
      As[slot * 512 + r * 8 + (c ^ ((r >> 1) & 7))] = araw[i];
    }
  };
  // fragment sets: [set][mi] activation, [set][nj] weights
  u32x4 af[2][4], bf[2][NB16];
  auto read_frags = [&](auto set_c, int aslot, int bbuf, int kk) SKG_INL {
    constexpr int SET = decltype(set_c)::value;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = mi * 16 + (lane & 15);
      const int c = kk * 4 + (lane >> 4);
      af[SET][mi] = As[aslot * 512 + r * 8 + (c ^ ((r >> 1) & 7))];
    }
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj)
      bf[SET][nj] = *reinterpret_cast<const u32x4*>(&Bs[bbuf][(nj * 16 + (lane & 15)) * GT_LDS_ROW + kk * 32 + (lane >> 4) * 8]);
  };
  f32x4 acc[4][NB16];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mfmas = [&](auto set_c) SKG_INL {
    constexpr int SET = decltype(set_c)::value;
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, bf[SET][nj]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[SET][mi]), bv,
                                                              acc[mi][nj], 0, 0, 0);
    }
  };
  // slice of step s into slot `slot` by direct copies: instruction i fills
  // slots 64 i .. 64 i + 63 (row 8 i + l / 8, physical chunk l % 8 for lane l),
  // so lane l fetches logical chunk (l % 8) ^ ((row >> 1) & 7) of its row
  auto dma_a = [&](int slot, int s) SKG_INL {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 8 + (lane >> 3);
      const int cl = (lane & 7) ^ ((r >> 1) & 7);
      const int m = min(mw + r, M - 1);
      const int k = min(s * GT_BK + cl * 8, K - 8);
      dma16(A + size_t(m) * size_t(K) + size_t(k), as_lds + uint32_t(slot) * 8192u + uint32_t(i) * 1024u);
    }
  };
  // The same copies where no row or column is clamped (the wave's 64 rows
  // lie below M and step s ends inside K): one wave-uniform base per copy
  // and two per-lane offsets (copy i takes the even or odd one: the chunk
  // swizzle of row 8 i + l / 8 depends on i only through i % 2), so the copy
  // addresses cost scalar additions only.
  const bool rows_in = mw + 64 <= M;
  const uint32_t off_even = uint32_t(lane >> 3) * uint32_t(K) * 2u + uint32_t((lane & 7) ^ (lane >> 4)) * 16u;
  const uint32_t off_odd = uint32_t(lane >> 3) * uint32_t(K) * 2u + uint32_t((lane & 7) ^ (4 + (lane >> 4))) * 16u;
  const uint16_t* const a_wave = A + size_t(mw) * size_t(K);
  auto dma_a_fast = [&](int slot, int s) SKG_INL {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16_sv(a_wave + size_t(i) * 8u * size_t(K) + size_t(s) * GT_BK, (i & 1) ? off_odd : off_even,
               as_lds + uint32_t(slot) * 8192u + uint32_t(i) * 1024u);
  };
  auto dma_step = [&](int slot, int s) SKG_INL {
    if (rows_in && (s + 1) * GT_BK <= K)
      dma_a_fast(slot, s);
    else
      dma_a(slot, s);
  };
  using std::integral_constant;
  if constexpr (ADMA) {
    dma_a(0, 0);
    dma_a(1, 1);
    wait_vmcnt<8>();  // slice 0 has landed; slice 1 may be in flight
    asm volatile("" ::: "memory");
  } else {
    load_a(0);
    park_a(0);
    load_a(1);
  }
  lds_barrier();  // weight buffers 0 and 1 decoded
  read_frags(integral_constant<int, 0>{}, 0, 0, 0);
  // One fragment read of set SET, in the order the next half-step's MFMAs
  // consume them: r = 0 -> weights nj 0, r = 1..4 -> activation mi 0..3,
  // r >= 5 -> weights nj r-4.
  auto read1 = [&](auto set_c, auto r_c, int aslot, int bbuf, int kk) SKG_INL {
    constexpr int SET = decltype(set_c)::value;
    constexpr int R = decltype(r_c)::value;
    if constexpr (R >= 1 && R <= 4) {
      const int r = (R - 1) * 16 + (lane & 15);
      const int c = kk * 4 + (lane >> 4);
      af[SET][R - 1] = As[aslot * 512 + r * 8 + (c ^ ((r >> 1) & 7))];
    } else {
      constexpr int NJ = R == 0 ? 0 : R - 4;
      bf[SET][NJ] = *reinterpret_cast<const u32x4*>(&Bs[bbuf][(NJ * 16 + (lane & 15)) * GT_LDS_ROW + kk * 32 + (lane >> 4) * 8]);
    }
  };
  // The MFMAs of set USE (nj-major) with the 4 + NB16 fragment reads of the
  // other set spread one per two MFMAs, pinned in that order (the scheduler
  // otherwise gathers the reads next to their uses and the LDS latency shows
  // between MFMA groups).
  auto half = [&](auto use_c, int aslot, int bbuf, int kk) SKG_INL {
    constexpr int USE = decltype(use_c)::value;
    constexpr int NR = 4 + NB16;
    [&]<int... J>(std::integer_sequence<int, J...>) SKG_INL {
      (([&]() SKG_INL {
         constexpr int nj = J / 4, mi = J % 4;
         acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[USE][mi]),
                                                               __builtin_bit_cast(bf16x8, bf[USE][nj]), acc[mi][nj], 0,
                                                               0, 0);
         if constexpr (J % 2 == 1 && J / 2 < NR)
           read1(integral_constant<int, 1 - USE>{}, integral_constant<int, J / 2>{}, aslot, bbuf, kk);
         __builtin_amdgcn_sched_barrier(0);
       }()),
       ...);
    }(std::make_integer_sequence<int, 4 * NB16>{});
  };
  auto dstep = [&](auto ca_c, auto cb_c, int s) SKG_INL {
    constexpr int CA = decltype(ca_c)::value;  // activation slot of step s (mod 3)
    constexpr int CB = decltype(cb_c)::value;  // weight buffer of step s
    dma_step((CA + 2) % 3, s + 2);  // that slot was last read during step s-1
    __builtin_amdgcn_sched_barrier(0);
    half(integral_constant<int, 0>{}, CA, CB, 1);
    wait_vmcnt<8>();  // slice s+1 (requested one step ago) has landed
    asm volatile("" ::: "memory");
    half(integral_constant<int, 1>{}, (CA + 1) % 3, (CB + 1) % 3, 0);
    // No LDS wait here: the reads still in flight are those of step s+1
    // (weight buffer (s+1) % 3, written before the previous barrier; slot
    // (CA+1) % 3), which nothing overwrites before the next barrier; every read
    // of buffer s % 3 fed an MFMA of this step, so has completed before the
    // producers overwrite it in step s+1.
    asm volatile("s_barrier" ::: "memory");
  };
  auto cstep = [&](auto ca_c, auto cb_c, int s) SKG_INL {
    constexpr int CA = decltype(ca_c)::value;  // activation slot of step s
    constexpr int CB = decltype(cb_c)::value;  // weight buffer of step s
    park_a(CA ^ 1);  // slice of step s+1 (loaded one step ago)
    load_a(s + 2);
    read_frags(integral_constant<int, 1>{}, CA, CB, 1);
    mfmas(integral_constant<int, 0>{});
    read_frags(integral_constant<int, 0>{}, CA ^ 1, (CB + 1) % 3, 0);
    mfmas(integral_constant<int, 1>{});
    lds_barrier();
  };
  for (int s0 = 0; s0 < steps; s0 += U) {
    if constexpr (ADMA) {
      [&]<int... I>(std::integer_sequence<int, I...>) SKG_INL {
        ((s0 + I < steps ? dstep(integral_constant<int, I % 3>{}, integral_constant<int, I % 3>{}, s0 + I) : void()),
         ...);
      }(std::make_integer_sequence<int, U>{});
    } else {
      [&]<int... I>(std::integer_sequence<int, I...>) SKG_INL {
        ((s0 + I < steps ? cstep(integral_constant<int, I % 2>{}, integral_constant<int, I % 3>{}, s0 + I) : void()),
         ...);
      }(std::make_integer_sequence<int, U>{});
    }
  }
  if constexpr (ADMA) wait_vmcnt<0>();  // no copy into LDS outlives the workgroup
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int nj = 0; nj < NB16; ++nj) {
      const int n = n0 + nj * 16 + (lane & 15);
      const float v[4] = {acc[mi][nj].x, acc[mi][nj].y, acc[mi][nj].z, acc[mi][nj].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mw + mi * 16 + (lane >> 4) * 4 + r;
        if (m < M && n < N) y[size_t(m) * size_t(N) + size_t(n)] = v[r];
      }
    }
  }
}

// 0: one role per wave; 1: producer/consumer waves, 4 consumer waves of 64
// rows; 2: producer/consumer waves, 8 consumer waves of 32 rows; 3: pipelined
// producer/consumer waves (triple-buffered weight tile); 4: as 3 with the
// activation slices copied straight into LDS
// measured on MI355X at M=512, K=4096, N=14336: 80.8 / 71.3 / 71.4 / 67.6 / 64.2-64.8 us
extern const int kGemmDefaultVariant = 4;
std::atomic<int> g_gemm_variant{kGemmDefaultVariant};

// The pipelined organisations (3: activation through registers, 4: copied
// straight into LDS) for weight format WK.
template <int WK>
void launch_pipe(int variant, bool seven, unsigned grid, const PackedW& P, const uint16_t* xa, float* y, int64_t M,
                 int64_t N, int64_t K, hipStream_t stream) {
  if (variant == 3) {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<7, GT_PW, false, WK>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<8, GT_PW, false, WK>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
  } else {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<7, GT_PW, true, WK>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<8, GT_PW, true, WK>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
  }
}

hipError_t launch_gemm_tiled(int64_t M, int64_t K, int64_t N, const void* W, const Layout& L, const void* x,
                             float* y, hipStream_t stream) {
  const int variant = g_gemm_variant.load(std::memory_order_relaxed);
  if (L.wk != WK_Q4_0) {
    // q8_0, q4_K and q6_K weights: the pipelined organisations only
    const PackedW P = packed_view(W, L);
    const int64_t mtiles = (M + GT_BM - 1) / GT_BM;
    const int64_t t7 = mtiles * ((N + 111) / 112), t8 = mtiles * ((N + 127) / 128);
    const int cus = 256;
    const double e7 = double(t7) / double(((t7 + cus - 1) / cus) * cus);
    const double e8 = double(t8) / double(((t8 + cus - 1) / cus) * cus);
    const bool seven = e7 > e8;
    const unsigned grid = unsigned(seven ? t7 : t8);
    const uint16_t* xa = static_cast<const uint16_t*>(x);
    if (L.wk == WK_Q8_0)
      launch_pipe<WK_Q8_0>(variant, seven, grid, P, xa, y, M, N, K, stream);
    else if (L.wk == WK_Q4_K)
      launch_pipe<WK_Q4_K>(variant, seven, grid, P, xa, y, M, N, K, stream);
    else
      launch_pipe<WK_Q6_K>(variant, seven, grid, P, xa, y, M, N, K, stream);
    return hipGetLastError();
  }
  const PackedW P = packed_view(W, L);
  const int64_t mtiles = (M + GT_BM - 1) / GT_BM;
  // Tile width: 7 or 8 16-column groups, whichever leaves the fewest idle
  // compute units in the last wave of tiles (N = 14336, M = 512 -> 7: 256 tiles).
  const int64_t t7 = mtiles * ((N + 111) / 112), t8 = mtiles * ((N + 127) / 128);
  const int cus = 256;
  const double e7 = double(t7) / double(((t7 + cus - 1) / cus) * cus);
  const double e8 = double(t8) / double(((t8 + cus - 1) / cus) * cus);
  const bool seven = e7 > e8;
  const unsigned grid = unsigned(seven ? t7 : t8);
  const uint16_t* xa = static_cast<const uint16_t*>(x);
  if (variant == 0) {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_kernel<7, GT_PW>), dim3(grid), dim3(256), 0, stream, P, xa, y, int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_kernel<8, GT_PW>), dim3(grid), dim3(256), 0, stream, P, xa, y, int(M), int(N), int(K));
  } else if (variant == 1) {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_pc_kernel<7, GT_PW, 4>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_pc_kernel<8, GT_PW, 4>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
  } else if (variant == 2) {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_pc_kernel<7, GT_PW, 8>), dim3(grid), dim3(768), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_pc_kernel<8, GT_PW, 8>), dim3(grid), dim3(768), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
  } else if (variant == 3) {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<7, GT_PW, false>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<8, GT_PW, false>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
  } else {
    if (seven)
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<7, GT_PW, true>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
    else
      hipLaunchKernelGGL((gemm_q4_0_bf16_pipe_kernel<8, GT_PW, true>), dim3(grid), dim3(512), 0, stream, P, xa, y,
                         int(M), int(N), int(K));
  }
  return hipGetLastError();
}

}  // namespace skg
