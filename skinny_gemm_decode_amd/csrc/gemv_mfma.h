// Small-batch GEMV on the matrix cores: y[m][n] = sum_k W[n][k] x[m][k] for
// q4_0 / q8_0 / q4_K / q6_K weights against fp32 activations (fp16 MFMAs) or
// Q8_1 activations (int8 MFMAs), 1 <= M <= 8.  The register-fed kernel below
// is described first; the weight-ring kernel (gemv_mfma_dma_kernel, the
// defaults at K = 4096) and its operand layouts (block pairs, grouped blocks,
// q6_K block-halves) follow further down.
//
// With fp32 activations every weight element costs M fused multiply-adds on
// the vector ALU, so the vector kernel stops being bound by HBM as soon as
// M > 1 ("The Shape That Actually Matters": the 8-row kernel that keeps 64
// accumulators per thread loses to the one-row kernel at M = 1).  Here the
// products run on v_mfma_f32_16x16x32_f16 instead, and the vector ALU only
// decodes weights:
//
// * One MFMA takes one 32-element quantisation block of 16 weight rows (the
//   B operand, one column per row) against the same 32 activation elements of
//   up to 16 activation rows (the A operand; rows m >= M are don't-care, their
//   outputs are never read).  Its fp32 result is scaled by the block's fp16
//   scale and accumulated; so no two blocks share an MFMA accumulator.
// * Weights decode exactly to fp16: a q4_0 nibble n becomes 1024 + n (or
//   1024 + 16 n for a high nibble) by OR-ing it into the mantissa of 1024.0
//   (one v_and_or_b32 per two elements), and one packed fp16 add (or fma by
//   1/16) makes that n - 8; a q8_0 code q becomes 1024 + (q + 128) by a byte
//   permute with 0x64, then q.  Every weight value is a small integer, exact
//   in fp16, and a zero weight contributes exactly zero.
// * The activation is split into two fp16 terms, hi = fp16(x s) and
//   lo = fp16(x s - hi), where s is a power of two chosen per activation row
//   and per wave so that the largest |x| of the row in the wave's span of K
//   maps into [2^14, 2^15).  The pair carries ~22 significant bits for every
//   element within 2^-28 of that largest magnitude; smaller elements keep an
//   absolute error below 2^-39 of it.  Every product is exact in fp32.  With
//   M <= 8 the two terms share one MFMA: A rows 0..7 hold the hi parts of the
//   activation rows, rows 8..15 the lo parts, and the two halves of each
//   output row's sum (lane groups 0, 1 and 2, 3) are added once per tile.
// * Loads keep the row-major packed layout of the vector kernels: lane
//   (g, c) of a wave (g = lane / 16, c = lane % 16) reads the 16-byte unit of
//   block 4 q + g of row c, i.e. four consecutive blocks per row per load.
//   A 4 x 4 transpose across the four 16-lane rows (two v_permlane32_swap and
//   two v_permlane16_swap per four dwords) then leaves dword g of every block
//   in lane (g, c): exactly the B operand layout, where lane (g, c) holds
//   k = 8 g .. 8 g + 7 of column c.
// * Waves split K: wave w owns blocks BPW w .. BPW w + BPW - 1 and keeps their A
//   operands in registers for the whole launch.  Workgroups are persistent:
//   each stages the activation once (through wave-private LDS, in the A
//   operand order) and then walks tiles of 16 output rows, loading tile t + 1
//   before decoding tile t.  Partial sums of the waves meet in LDS.
#pragma once

#include "common.h"
#include "gemv_impl.h"

#include <type_traits>

namespace skg {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int MF_ROWS = 16;  // output rows per tile (MFMA N dimension)

struct MfSeg {
  PackedW w0, w1;
  float* y;
  int64_t N;
  int tile_begin;
};

struct MfArgs {
  MfSeg seg[MAX_SEGS];
  int nseg;
  int ntiles;
  int64_t K;
  uint32_t nb;
  const float* x;
};

__device__ inline uint32_t bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 half2_of(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<SKG_DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_ROW_MIRROR>(v));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// In-register 4 x 4 transpose across the four 16-lane rows of a wave: on
// entry v[q] in row r holds element (r, q); on exit v[q] in row r holds
// element (q, r).
__device__ inline void transpose_rows4(uint32_t (&v)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// No inline asm in this kernel: the compiler inserts the wait states an
// in-flight MFMA needs before another instruction writes or reads its
// registers only for instructions it can see.
// B operand of one block from dword g of its q4_0 unit (bytes 4g..4g+3: low
// nibbles are elements 4g..4g+3, high nibbles 16+4g..16+4g+3) as n - 8.
// Slot order: elements 4g, 4g+2, 4g+1, 4g+3, then the same plus 16.
__device__ inline f16x8 decode_q4_0(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t magic) {
  const uint32_t w8 = w >> 8;
  const f16x2 e0 = half2_of((w & mlo) | magic);   // 1024 + n
  const f16x2 e1 = half2_of((w8 & mlo) | magic);
  const f16x2 e2 = half2_of((w & mhi) | magic);   // 1024 + 16 n
  const f16x2 e3 = half2_of((w8 & mhi) | magic);
  const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const f16x2 r0 = e0 + off, r1 = e1 + off;
  const f16x2 r2 = __builtin_elementwise_fma(e2, sixteenth, off16);
  const f16x2 r3 = __builtin_elementwise_fma(e3, sixteenth, off16);
  return f16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// B operand of one block from dword g of each q8_0 plane (codes 4g..4g+3 and
// 16+4g..16+4g+3) as q, same slot order as decode_q4_0.
__device__ inline f16x8 decode_q8_0(uint32_t p0, uint32_t p1) {
  const uint32_t u0 = p0 ^ 0x80808080u, u1 = p1 ^ 0x80808080u;  // q + 128 as unsigned bytes
  const uint32_t hi = 0x64646464u;
  // bytes {u.b0, 0x64, u.b2, 0x64} and {u.b1, 0x64, u.b3, 0x64}: 1024 + q + 128
  const f16x2 e0 = half2_of(__builtin_amdgcn_perm(hi, u0, 0x04020400u));
  const f16x2 e1 = half2_of(__builtin_amdgcn_perm(hi, u0, 0x04030401u));
  const f16x2 e2 = half2_of(__builtin_amdgcn_perm(hi, u1, 0x04020400u));
  const f16x2 e3 = half2_of(__builtin_amdgcn_perm(hi, u1, 0x04030401u));
  const f16x2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2 r0 = e0 + off, r1 = e1 + off, r2 = e2 + off, r3 = e3 + off;
  return f16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// B operand of one q4_K sub-block from dword g of its unit (the q4_0 nibble
// order): each code c as the exact fp16 subnormal c 2^-24, one shift-free AND
// or a shift and an AND per pair (the matrix cores take fp16 subnormals
// exactly, checked on MI355X; the products stay exact in fp32).  q4_K has no
// code offset (w = d sc c - dmin m), so nothing cancels.
__device__ inline f16x8 decode_q4_K_sub(uint32_t w, uint32_t mlo) {
  return __builtin_bit_cast(f16x8, u32x4{w & mlo, (w >> 8) & mlo, (w >> 4) & mlo, (w >> 12) & mlo});
}

// Weight registers of one tile for one matrix: NP planes x BPW/4 quads of 16
// bytes and the fp16 scales of the wave's BPW blocks (aligned 16-byte loads:
// the kernel requires nb % BPW == 0).
template <int NP, int BPW>
struct MfW {
  u32x4 u[BPW / 4][NP];
  u32x4 sc[BPW / 8];
};

template <int NP, int BPW>
__device__ inline void mf_load_quad(MfW<NP, BPW>& r, int q, const uint8_t* rowp, uint32_t nb, uint32_t blk0,
                                    int g) {
#pragma unroll
  for (int p = 0; p < NP; ++p)
    r.u[q][p] = ld_u32x4_stream(rowp + (size_t(p) * nb + blk0 + uint32_t(4 * q + g)) * 16);
}

template <int NP, int BPW>
__device__ inline void mf_load_scales(MfW<NP, BPW>& r, const uint16_t* srow, uint32_t blk0) {
  const u32x4* sp = reinterpret_cast<const u32x4*>(srow + blk0);
#pragma unroll
  for (int i = 0; i < BPW / 8; ++i) r.sc[i] = __builtin_nontemporal_load(sp + i);
}

// Where the next tile of one matrix lives, for the rolling prefetch.
struct MfNext {
  const uint8_t* rowp;
  const uint16_t* srow;
  uint32_t nb;
};

// One tile of one matrix.  With RELOAD, each quad's registers are refilled
// with the same quad of the next tile as soon as they have been transposed,
// and the scales after their last use, so about one tile of loads stays in
// flight with a single register set.
//
// KQ (q4_K): the scale words are the 16-byte super-block headers {d, dmin,
// 12 scale bytes} of the wave's BPW / 8 super-blocks; block j's product is
// scaled by d sc_j, and the min term - sum_j dmin m_j S_j (S_j: the block's
// activation sum) is one MFMA per super-block over ksum, the block sums'
// operand from mf_stage: A slot 8g + i holds the high (g even) or low (g odd)
// fp16 part of 2^-6 S of block 8 (g / 2) + i, B the codes m_j as subnormals
// in the slots of that super-block.
template <int NP, int BPW, int RR, int XT, bool RELOAD, bool KQ = false>
__device__ inline void mf_tile(MfW<NP, BPW>& r, const f16x8 (&ah)[BPW], const f16x8 (&al)[BPW], float (&acc)[4],
                               uint32_t mlo, uint32_t mhi, uint32_t magic, const MfNext& nx, uint32_t blk0, int g,
                               const f16x8& ksum = f16x8{}) {
  uint32_t scw[BPW / 2];
#pragma unroll
  for (int i = 0; i < BPW / 8; ++i) {
    scw[4 * i + 0] = r.sc[i].x;
    scw[4 * i + 1] = r.sc[i].y;
    scw[4 * i + 2] = r.sc[i].z;
    scw[4 * i + 3] = r.sc[i].w;
  }
  if constexpr (RELOAD) {
    mf_load_scales<NP, BPW>(r, nx.srow, blk0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < BPW / 4; ++q) {
    uint32_t t[NP][4];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      t[p][0] = r.u[q][p].x;
      t[p][1] = r.u[q][p].y;
      t[p][2] = r.u[q][p].z;
      t[p][3] = r.u[q][p].w;
      transpose_rows4(t[p]);
    }
    if constexpr (RELOAD) {
      mf_load_quad<NP, BPW>(r, q, nx.rowp, nx.nb, blk0, g);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * q + jj;
      f16x8 bw;
      if constexpr (KQ)
        bw = decode_q4_K_sub(t[0][jj], mlo);
      else if constexpr (NP == 1)
        bw = decode_q4_0(t[0][jj], mlo, mhi, magic);
      else
        bw = decode_q8_0(t[0][jj], t[1][jj]);
      const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[j], bw, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      float s;
      if constexpr (KQ) {
        // d sc_j (exact in fp32: 11 x 6 bits)
        const int hb = 4 * (j >> 3);
        uint32_t sc, mn;
        q4_K_sc_m(scw[hb + 1], scw[hb + 2], scw[hb + 3], uint32_t(j & 7), sc, mn);
        s = h2f(scw[hb] & 0xFFFFu) * float(sc);
      } else {
        const uint32_t sw = scw[j >> 1];
        s = h2f((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
      }
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i] = fmaf(s, d[i], acc[i]);
    }
  }
  if constexpr (KQ) {
    // acc holds 2^-24 sum_j d sc_j sum_k c_k x_k; the min term's MFMA gives
    // 2^-30 sum_j m_j S_j per super-block
    float mt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < BPW / 8; ++sb) {
      uint32_t mp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t sc0, m0, sc1, m1;
        q4_K_sc_m(scw[4 * sb + 1], scw[4 * sb + 2], scw[4 * sb + 3], uint32_t(2 * i), sc0, m0);
        q4_K_sc_m(scw[4 * sb + 1], scw[4 * sb + 2], scw[4 * sb + 3], uint32_t(2 * i + 1), sc1, m1);
        mp[i] = m0 | (m1 << 16);
      }
      const bool mine = (g >> 1) == sb;
      const u32x4 bm = mine ? u32x4{mp[0], mp[1], mp[2], mp[3]} : u32x4{0u, 0u, 0u, 0u};
      const f32x4 cr = __builtin_amdgcn_mfma_f32_16x16x32_f16(ksum, __builtin_bit_cast(f16x8, bm),
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float dmin = h2f(scw[4 * sb] >> 16);
#pragma unroll
      for (int i = 0; i < RR; ++i) mt[i] = fmaf(dmin, cr[i], mt[i]);
    }
#pragma unroll
    for (int i = 0; i < RR; ++i) acc[i] = fmaf(acc[i], 16777216.0f, -1073741824.0f * mt[i]);
  }
  if constexpr (XT == 2) {
    // high-part rows (lane groups 0, 1) plus low-part rows (2, 3)
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      const uint32_t v = __float_as_uint(acc[i]);
      const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      acc[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
  }
}

// ---------------------------------------------------------------------------
// Q8_1 activations on the integer matrix cores (v_mfma_i32_16x16x32_i8).  The
// activation is already int8 with one scale per block, so the A operand of a
// block is read straight from its 36-byte Q8_1 block: lane (g, c) takes the
// codes of elements 4g..4g+3 and 16+4g..16+4g+3 of activation row c (dwords
// 1 + g and 5 + g; rows c >= M repeat row c % M and their outputs are never
// stored).  The B operand holds the same elements of weight row c as int8:
// 16 (code - 8) for q4_0 (a nibble shifted into the high half of a byte, sign
// bit flipped), the codes themselves for q8_0.  The block's int32 result is
// exact, and is scaled in fp32 by the weight scale (over 16 for q4_0) and the
// activation scale of each output row: y += dW dA S.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// A operands of the wave's BPW blocks and the activation scales of the four
// output rows 4g..4g+3 this lane accumulates (zero for rows >= M).  The wave's
// LDS row stride (dwords) of the Q8_1 staging: RW = 9 BPW, plus one where
// rows 4 apart would start on the same bank (RW = 144: 4 x 144 = 9 x 64), so
// the scales a lane gathers from rows 4 g .. 4 g + 3 and the 16 rows of a
// fragment read start on different banks.
template <int BPW>
constexpr int q8_stage_row() {
  return (4 * 9 * BPW) % 64 == 0 ? 9 * BPW + 1 : 9 * BPW;
}

// M x BPW blocks (BPW * 36 contiguous bytes per activation row) are copied
// with coalesced dword loads into the wave-private LDS area and picked apart
// there; between() runs once those loads are issued (the first tiles' weight
// loads go there), after_x() once they have been written to LDS (direct
// global-to-LDS weight transfers go there: the compiler would drain them
// before any later use of a register load).
template <int M, int BPW, int RWP, class Between>
__device__ inline void mf_copy_q8(const MfArgs& a, uint32_t* area, uint32_t blk0, int lane, Between between) {
  constexpr int RW = BPW * 9;                 // dwords per activation row of the wave's span
  constexpr int NL = (M * RW + 63) / 64;      // dword loads per lane
  static_assert(RWP >= RW, "row stride");
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(a.x);
  uint32_t v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = i * 64 + lane;              // flat dword of [m][RW]
    const int m = f / RW, o = f % RW;
    v[i] = (f < M * RW) ? xw[(size_t(m) * a.nb + blk0) * 9 + size_t(o)] : 0u;
  }
  __builtin_amdgcn_sched_barrier(0);
  between();
  __builtin_amdgcn_sched_barrier(0);
  // A wave's LDS accesses complete in order: its own writes are visible to
  // its later reads without a barrier.
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = i * 64 + lane;
    if (f < M * RW) area[(f / RW) * RWP + f % RW] = v[i];
  }
}

template <int M, int BPW, int RWP = q8_stage_row<BPW>(), class Between, class AfterX>
__device__ inline void mf_stage_q8(const MfArgs& a, uint32_t* area, uint32_t blk0, int lane, uint64_t (&aq)[BPW],
                                   f32x4 (&da)[BPW], Between between, AfterX after_x) {
  mf_copy_q8<M, BPW, RWP>(a, area, blk0, lane, between);
  after_x();
  const int g = lane >> 4, c = lane & 15;
  const int mr = (c < M) ? c : c % M;
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const uint32_t* blk = area + mr * RWP + j * 9;
    aq[j] = uint64_t(blk[1 + g]) | (uint64_t(blk[5 + g]) << 32);
    float d4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      d4[i] = (m < M) ? h2f(area[(m < M ? m : 0) * RWP + j * 9] & 0xFFFFu) : 0.f;
    }
    da[j] = f32x4{d4[0], d4[1], d4[2], d4[3]};
  }
}

// One tile of one matrix against Q8_1 activations; loads and reloads as in
// mf_tile.
template <int NP, int BPW, int RR, bool RELOAD>
__device__ inline void mf_tile_q8(MfW<NP, BPW>& r, const uint64_t (&aq)[BPW], const f32x4 (&da)[BPW],
                                  float (&acc)[4], const MfNext& nx, uint32_t blk0, int g) {
  uint32_t scw[BPW / 2];
#pragma unroll
  for (int i = 0; i < BPW / 8; ++i) {
    scw[4 * i + 0] = r.sc[i].x;
    scw[4 * i + 1] = r.sc[i].y;
    scw[4 * i + 2] = r.sc[i].z;
    scw[4 * i + 3] = r.sc[i].w;
  }
  if constexpr (RELOAD) {
    mf_load_scales<NP, BPW>(r, nx.srow, blk0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // q4_0 codes enter the product as 16 (c - 8)
  constexpr float WSCALE = (NP == 1) ? 0.0625f : 1.0f;
#pragma unroll
  for (int q = 0; q < BPW / 4; ++q) {
    uint32_t t[NP][4];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      t[p][0] = r.u[q][p].x;
      t[p][1] = r.u[q][p].y;
      t[p][2] = r.u[q][p].z;
      t[p][3] = r.u[q][p].w;
      transpose_rows4(t[p]);
    }
    if constexpr (RELOAD) {
      mf_load_quad<NP, BPW>(r, q, nx.rowp, nx.nb, blk0, g);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * q + jj;
      uint64_t bv;
      if constexpr (NP == 1) {
        const uint32_t w = t[0][jj];
        const uint32_t wl = ((w << 4) & 0xF0F0F0F0u) ^ 0x80808080u;  // elements 4g..4g+3
        const uint32_t wh = (w & 0xF0F0F0F0u) ^ 0x80808080u;         // elements 16+4g..16+4g+3
        bv = uint64_t(wl) | (uint64_t(wh) << 32);
      } else {
        bv = uint64_t(t[0][jj]) | (uint64_t(t[1][jj]) << 32);
      }
      const i32x4 sdot = __builtin_amdgcn_mfma_i32_16x16x32_i8(long(aq[j]), long(bv), i32x4{0, 0, 0, 0}, 0, 0, 0);
      const uint32_t sw = scw[j >> 1];
      const float s = h2f((j & 1) ? (sw >> 16) : (sw & 0xFFFFu)) * WSCALE;
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i] = fmaf(s, da[j][i] * float(sdot[i]), acc[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Two Q8_1 blocks per v_mfma_i32_16x16x64_i8 (weight-ring kernel, M <= 8).
// One block per 16 x 16 integer MFMA leaves result rows M..15 unused, and
// every lane scales four results of which at most two rows of four carry
// output.  The 64-deep instruction takes blocks b and b + 1 at once as a
// block-diagonal product: the B operand holds block b in lane groups g = 0, 1
// and block b + 1 in g = 2, 3; A rows 0..7 hold the activation rows of block
// b in groups 0, 1 and zeros in 2, 3, rows 8..15 those of block b + 1 in
// groups 2, 3 and zeros in 0, 1.  Result row r is then block b + r / 8's dot
// of activation row r % 8, exact in int32: an element of A lane (g, i) only
// ever meets the element in the same position of B lane (g, j), so which k
// the hardware gives each position does not matter.  Every lane's four
// results are output rows (for M > 4), half the scaling per block, and the B
// operand comes straight from the LDS slot with no transpose: lane (g, c)
// takes half g % 2 of block b + g / 2 of row c (8 bytes of nibbles, or one
// 16-byte q8_0 plane unit).  The two halves of an output row's sum (lane
// groups g and g + 2) are added once per tile.

// LDS position of chunk j of row r in a weight-ring slot (16-byte chunks,
// permuted within each aligned group of 16; see the ring kernel below).
__device__ inline int mf_swz(int j, int r) { return j ^ (r & 15); }

// A operands of the wave's BPW / 2 block pairs in that layout, and the
// activation scales of the four result rows of each lane (zero for rows >=
// M; over 16 for q4_0, whose B codes are 16 (code - 8)) and, for q4_K, the
// activation block sums s = dA sum(q) of those rows (the min term).
// WK: the weight kind (WK_Q4_0, WK_Q8_0 or WK_Q4_K; q4_K codes are q4_0's
// nibbles without the offset).
template <int M, int BPW, int WK, int RWP = q8_stage_row<BPW>(), class Between, class AfterX>
__device__ inline void mf_stage_q8p(const MfArgs& a, uint32_t* area, uint32_t blk0, int lane, i32x4 (&aq)[BPW / 2],
                                    f32x4 (&da)[BPW / 2], f32x4 (&sa)[BPW / 2], Between between, AfterX after_x) {
  constexpr bool Q4 = WK == WK_Q4_0 || WK == WK_Q4_K;
  static_assert(M <= 8 && BPW % 2 == 0, "two blocks of eight rows");
  mf_copy_q8<M, BPW, RWP>(a, area, blk0, lane, between);
  after_x();
  const int g = lane >> 4, c = lane & 15;
  const int h = g & 1, e = g >> 1;  // half of the block, block of the pair
  const int m = c & 7;
  const bool on = (c >> 3) == e && m < M;
  const uint32_t* row = area + (m < M ? m : 0) * RWP;
  constexpr float WS = WK == WK_Q4_0 ? 0.0625f : 1.0f;
#pragma unroll
  for (int p = 0; p < BPW / 2; ++p) {
    const uint32_t* blk = row + (2 * p + e) * 9;
    // q4_0: nibble bytes 8h..8h+7 hold elements 8h..8h+7 (low) and
    // 16+8h..16+8h+7 (high), decoded dword by dword as low, high; q8_0: plane
    // h holds elements 16h..16h+15 in order.  Element i sits in dword 1 + i/4.
    uint32_t v[4];
    if constexpr (Q4) {
      v[0] = blk[1 + 2 * h];
      v[1] = blk[5 + 2 * h];
      v[2] = blk[2 + 2 * h];
      v[3] = blk[6 + 2 * h];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = blk[1 + 4 * h + i];
    }
    aq[p] = on ? i32x4{int(v[0]), int(v[1]), int(v[2]), int(v[3])} : i32x4{0, 0, 0, 0};
    float d4[4], s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mo = 4 * h + i;
      const uint32_t ds = area[(mo < M ? mo : 0) * RWP + (2 * p + e) * 9];
      d4[i] = (mo < M) ? h2f(ds & 0xFFFFu) * WS : 0.f;
      s4[i] = (mo < M) ? h2f(ds >> 16) : 0.f;
    }
    da[p] = f32x4{d4[0], d4[1], d4[2], d4[3]};
    sa[p] = f32x4{s4[0], s4[1], s4[2], s4[3]};
  }
}

// One tile of the weight-ring kernel against Q8_1 activations in block pairs.
// slot: the tile's LDS slot (rows of RB payload bytes, mf_swz chunk order,
// then 16 rows of SRS scale bytes); RR: result rows per lane that can be
// output rows.  On return every lane holds the full sums of rows 4 (g % 2) ..
// 4 (g % 2) + 3 of column c.  KQ (q4_K): the scale bytes of a row are its 16
// super-block headers {d, dmin, 12 scale bytes}, the codes enter as 0..15,
// and block j of a super-block adds d sc_j dA S - dmin m_j s.
template <class G, int BPW, int RR, bool KQ = false>
__device__ inline void mf_tile_q8p(const uint8_t* slot, uint32_t blk0, int g, int c, const i32x4 (&aq)[BPW / 2],
                                   const f32x4 (&da)[BPW / 2], const f32x4 (&sa)[BPW / 2], float (&acc)[4]) {
  uint32_t scw[BPW / 2];
#pragma unroll
  for (int k = 0; k < BPW / 8; ++k) {
    const u32x4 s4 = *reinterpret_cast<const u32x4*>(slot + 16 * G::RB + c * G::SRS + mf_swz(int(blk0) / 8 + k, c) * 16);
    scw[4 * k + 0] = s4.x;
    scw[4 * k + 1] = s4.y;
    scw[4 * k + 2] = s4.z;
    scw[4 * k + 3] = s4.w;
  }
  const int h = g & 1, e = g >> 1;
  const uint32_t sh = uint32_t(e) * 16u;  // block b + 1's scale is the high half
  const uint8_t* row = slot + c * G::RB;
#pragma unroll
  for (int p = 0; p < BPW / 2; ++p) {
    const int b = int(blk0) + 2 * p + e;
    i32x4 bv;
    if constexpr (KQ) {
      // codes 0..15 as int8
      const uint2 u = *reinterpret_cast<const uint2*>(row + mf_swz(b, c) * 16 + 8 * h);
      bv = i32x4{int(u.x & 0x0F0F0F0Fu), int((u.x >> 4) & 0x0F0F0F0Fu), int(u.y & 0x0F0F0F0Fu),
                 int((u.y >> 4) & 0x0F0F0F0Fu)};
    } else if constexpr (G::NP == 1) {
      // 16 (code - 8) as int8: the nibble moved to the high half of its
      // byte, sign bit flipped
      const uint2 u = *reinterpret_cast<const uint2*>(row + mf_swz(b, c) * 16 + 8 * h);
      bv = i32x4{int(((u.x << 4) & 0xF0F0F0F0u) ^ 0x80808080u), int((u.x & 0xF0F0F0F0u) ^ 0x80808080u),
                 int(((u.y << 4) & 0xF0F0F0F0u) ^ 0x80808080u), int((u.y & 0xF0F0F0F0u) ^ 0x80808080u)};
    } else {
      bv = *reinterpret_cast<const i32x4*>(row + mf_swz(h * G::NB + b, c) * 16);
    }
    const i32x4 sdot = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[p], bv, i32x4{0, 0, 0, 0}, 0, 0, 0);
    if constexpr (KQ) {
      // header of super-block (2 p + e) / 8 of the wave's span (= p / 4),
      // sub-block (2 p + e) % 8; both products exact in fp32
      const int hb = 4 * (p >> 2);
      uint32_t sc, mn;
      q4_K_sc_m(scw[hb + 1], scw[hb + 2], scw[hb + 3], uint32_t((2 * p + e) & 7), sc, mn);
      const float aw = h2f(scw[hb] & 0xFFFFu) * float(sc);
      const float bw = h2f(scw[hb] >> 16) * float(mn);
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i] = fmaf(aw, da[p][i] * float(sdot[i]), fmaf(-bw, sa[p][i], acc[i]));
    } else {
      const float s = h2f(scw[p] >> sh);
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i] = fmaf(s, da[p][i] * float(sdot[i]), acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    const uint32_t v = __float_as_uint(acc[i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    acc[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
}

// ---------------------------------------------------------------------------
// q6_K weights against Q8_1 activations (weight-ring kernel).  A q6_K block
// scales each 16-element half by its own int8 scale, so a block's two halves
// must not meet in one result row: the 64-deep integer MFMA takes two blocks
// as four block-halves, lane group g holding half g % 2 of block b + g / 2
// (16 codes), and A rows 4 g .. 4 g + 3 carry activation rows 0..3 (a second
// chain: rows 4..7) of that block-half in group g only.  Result row r is then
// block-half r / 4's dot with activation row r % 4, and each lane's four
// results share one weight scale d sc.  The codes enter as 0..63; the -32 of
// the format is a chained MFMA against a constant B of int8 -32, so
// sum (q - 32) qa is exact in int32 with no vector-ALU work.  The four lane
// groups hold parts of the same sums, added once per tile.

// A operands (two chains for M > 4) and the activation scales of each lane's
// four result rows (zero for rows >= M) of the wave's BPW / 2 block pairs.
template <int M, int BPW, int RWP = q8_stage_row<BPW>(), class Between, class AfterX>
__device__ inline void mf_stage_q6q8(const MfArgs& a, uint32_t* area, uint32_t blk0, int lane,
                                     i32x4 (&aq)[2][BPW / 2], f32x4 (&da)[2][BPW / 2], Between between,
                                     AfterX after_x) {
  static_assert(M <= 8 && BPW % 2 == 0, "two chains of four rows");
  mf_copy_q8<M, BPW, RWP>(a, area, blk0, lane, between);
  after_x();
  const int g = lane >> 4, c = lane & 15;
  const int h = g & 1, e = g >> 1;
#pragma unroll
  for (int ch = 0; ch < (M > 4 ? 2 : 1); ++ch) {
    const int m = (c & 3) + 4 * ch;
    const bool on = (c >> 2) == g && m < M;
    const uint32_t* row = area + (on ? m : 0) * RWP;
#pragma unroll
    for (int p = 0; p < BPW / 2; ++p) {
      // elements 16 h .. 16 h + 15 of the block: dwords 1 + 4 h .. 4 + 4 h
      const uint32_t* blk = row + (2 * p + e) * 9 + 1 + 4 * h;
      aq[ch][p] = on ? i32x4{int(blk[0]), int(blk[1]), int(blk[2]), int(blk[3])} : i32x4{0, 0, 0, 0};
      float d4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mo = 4 * ch + i;
        d4[i] = (mo < M) ? h2f(area[(mo < M ? mo : 0) * RWP + (2 * p + e) * 9] & 0xFFFFu) : 0.f;
      }
      da[ch][p] = f32x4{d4[0], d4[1], d4[2], d4[3]};
    }
  }
}

// One tile against Q8_1 activations in that layout.  The slot holds per row
// the low units (16 bytes per block, q4_0 nibble order) then the high units
// (8 bytes per block), in mf_swz chunk order; then 16 rows of int8 scale
// pairs; then the rows' fp16 super-block d (G::DOFF, 32 bytes per row).  On
// return every lane holds the full sums of activation rows 0..3 (acc[0]) and
// 4..7 (acc[1]) of column c.
template <class G, int BPW, int M>
__device__ inline void mf_tile_q6q8(const uint8_t* slot, uint32_t blk0, int g, int c, const i32x4 (&aq)[2][BPW / 2],
                                    const f32x4 (&da)[2][BPW / 2], float (&acc)[2][4]) {
  constexpr int NCH = M > 4 ? 2 : 1;
  constexpr int RR0 = M < 4 ? M : 4;
  uint32_t scw[BPW / 2];
#pragma unroll
  for (int k = 0; k < BPW / 8; ++k) {
    const u32x4 s4 = *reinterpret_cast<const u32x4*>(slot + 16 * G::RB + c * G::SRS + mf_swz(int(blk0) / 8 + k, c) * 16);
    scw[4 * k + 0] = s4.x;
    scw[4 * k + 1] = s4.y;
    scw[4 * k + 2] = s4.z;
    scw[4 * k + 3] = s4.w;
  }
  static_assert(BPW == 16, "two super-blocks per wave span");
  // d of the span's two super-blocks (row c)
  const uint32_t dw = *reinterpret_cast<const uint32_t*>(slot + G::DOFF + c * 32 + (int(blk0) / 8) * 2);
  const float dsb[2] = {h2f(dw & 0xFFFFu), h2f(dw >> 16)};
  const uint8_t* row = slot + c * G::RB;
  const int h = g & 1, e = g >> 1;
  // per-lane shifts: the half's nibbles, and where its top two bits sit in
  // the high unit's dword (even k: bits 4h..; odd k: shifted up)
  const uint32_t sl = 4u * uint32_t(h), sre = 2u * uint32_t(h), slo = 4u - 2u * uint32_t(h);
  const i32x4 m32 = {int(0xE0E0E0E0u), int(0xE0E0E0E0u), int(0xE0E0E0E0u), int(0xE0E0E0E0u)};  // int8 -32
#pragma unroll
  for (int p = 0; p < BPW / 2; ++p) {
    const int b = int(blk0) + 2 * p + e;
    const u32x4 lw = *reinterpret_cast<const u32x4*>(row + mf_swz(b, c) * 16);
    const uint2 hw = *reinterpret_cast<const uint2*>(row + mf_swz(G::NB + (b >> 1), c) * 16 + 8 * (b & 1));
    const uint32_t w[4] = {lw.x, lw.y, lw.z, lw.w};
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t H = (k >> 1) ? hw.y : hw.x;
      const uint32_t hx = (k & 1) ? (H << slo) : (H >> sre);
      q[k] = ((w[k] >> sl) & 0x0F0F0F0Fu) | (hx & 0x30303030u);
    }
    const i32x4 bv = {int(q[0]), int(q[1]), int(q[2]), int(q[3])};
    // d sc of the lane's block-half (int8 scale: byte g of word p).  A plain
    // int8_t cast: the sign-extending bit-field builtin followed by the
    // conversion compiled to an unsigned int -> float conversion (every
    // negative scale became ~4.3e9).
    const float ds = dsb[p >> 2] * float(int(int8_t(uint8_t(scw[p] >> (8u * uint32_t(g))))));
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      i32x4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[ch][p], m32, i32x4{0, 0, 0, 0}, 0, 0, 0);
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[ch][p], bv, d, 0, 0, 0);
      const int rr = ch == 0 ? RR0 : M - 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < rr) acc[ch][i] = fmaf(ds, da[ch][p][i] * float(d[i]), acc[ch][i]);
    }
  }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = __float_as_uint(acc[ch][i]);
      const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      acc[ch][i] = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
      v = __float_as_uint(acc[ch][i]);
      const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      acc[ch][i] = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    }
}

// Bytes of one activation row in a staging pass (8 blocks of fp16, plus 16 so
// that the rows a fragment read takes start 4 banks apart).
constexpr int GRP_ROW = 8 * 32 * 2 + 16;

// ---------------------------------------------------------------------------
// q6_K weights against fp32 activations (weight-ring kernel, the activation
// as one fp16 term with a power of two per row and wave, as mf_stage_grp).
// The block-half layout of the integer kernel above on
// v_mfma_f32_16x16x32_f16: lane group g holds eight elements of half g % 2 of
// block b + g / 2 per MFMA (two MFMAs per pair of blocks and chain), A rows
// 4 g .. 4 g + 3 carry activation rows 0..3 (second chain: 4..7) in group g
// only, and the codes enter as the exact fp16 values q - 32 (a byte under the
// exponent of 1024 by one mask-and-or, one packed subtraction of 1056), so a
// zero weight contributes exactly zero.  ap[ch][2 p + j]: chain ch, pair p,
// elements 16 h + 8 j .. + 7 in the decode's slot order.
template <int M, int BPW, class Between, class AfterX>
__device__ inline void mf_stage_q6f(const MfArgs& a, uint8_t* area, uint32_t blk0, int lane, f16x8 (&ap)[2][BPW],
                                    float (&unscale)[4], Between between, AfterX after_x) {
  static_assert(M <= 8 && BPW % 8 == 0, "two chains of four rows, whole staging passes");
  const int g = lane >> 4, c = lane & 15;
  const int h = g & 1, e = g >> 1;
  f32x4 xv[M][BPW / 8];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int ee = 0; ee < BPW / 8; ++ee)
      xv[m][ee] = *reinterpret_cast<const f32x4*>(a.x + size_t(m) * size_t(a.K) + size_t(blk0) * 32 + 256 * ee + 4 * lane);
  __builtin_amdgcn_sched_barrier(0);
  between();
  __builtin_amdgcn_sched_barrier(0);
  float sc[M], us[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float mx = 0.f;
#pragma unroll
    for (int ee = 0; ee < BPW / 8; ++ee)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[m][ee].x), fabsf(xv[m][ee].y)), fmaxf(fabsf(xv[m][ee].z), fabsf(xv[m][ee].w))));
    mx = wave_max(mx);
    int se = 15 - __builtin_amdgcn_frexp_expf(mx);
    se = se > 126 ? 126 : (se < -126 ? -126 : se);
    sc[m] = __builtin_ldexpf(1.0f, se);
    us[m] = __builtin_ldexpf(1.0f, -se);
  }
  // the lane's written rows (below): group 1 rows 4..7, else rows 0..3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u0 = (i < M) ? us[i < M ? i : 0] : 1.f;
    const float u1 = (4 + i < M) ? us[4 + i < M ? 4 + i : 0] : 1.f;
    unscale[i] = (g == 1) ? u1 : u0;
  }
  after_x();
#pragma unroll
  for (int ee = 0; ee < BPW / 8; ++ee) {
    // a wave's LDS accesses complete in order: this pass's writes are seen by
    // its reads, and its reads finish before the next pass writes
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const f32x4 v = xv[m][ee] * sc[m];
      const f16x2 p01 = __builtin_convertvector((f32x2{v.x, v.y}), f16x2);
      const f16x2 p23 = __builtin_convertvector((f32x2{v.z, v.w}), f16x2);
      *reinterpret_cast<u32x2*>(area + m * GRP_ROW + 8 * lane) = u32x2{bits(p01), bits(p23)};
    }
#pragma unroll
    for (int ch = 0; ch < (M > 4 ? 2 : 1); ++ch) {
      const int m = (c & 3) + 4 * ch;
      const bool on = (c >> 2) == g && m < M;
      const uint8_t* rd = area + (on ? m : 0) * GRP_ROW;
#pragma unroll
      for (int gl = 0; gl < 4; ++gl)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 r = *reinterpret_cast<const u32x4*>(rd + 2 * (32 * (2 * gl + e) + 16 * h + 8 * j));
          const u32x4 sl = {__builtin_amdgcn_perm(r.y, r.x, 0x05040100u), __builtin_amdgcn_perm(r.y, r.x, 0x07060302u),
                            __builtin_amdgcn_perm(r.w, r.z, 0x05040100u), __builtin_amdgcn_perm(r.w, r.z, 0x07060302u)};
          ap[ch][2 * (4 * ee + gl) + j] = __builtin_bit_cast(f16x8, on ? sl : u32x4{0u, 0u, 0u, 0u});
        }
    }
  }
}

// One tile of q6_K against the fp16 operands above; slot as mf_tile_q6q8.  On
// return every lane holds the full (still scaled) sums of activation rows
// 0..3 (acc[0]) and 4..7 (acc[1]) of column c.
template <class G, int BPW, int M>
__device__ inline void mf_tile_q6f(const uint8_t* slot, uint32_t blk0, int g, int c, const f16x8 (&ap)[2][BPW],
                                   float (&acc)[2][4], uint32_t magic, uint32_t mbyte) {
  constexpr int NCH = M > 4 ? 2 : 1;
  constexpr int RR0 = M < 4 ? M : 4;
  uint32_t scw[BPW / 2];
#pragma unroll
  for (int k = 0; k < BPW / 8; ++k) {
    const u32x4 s4 = *reinterpret_cast<const u32x4*>(slot + 16 * G::RB + c * G::SRS + mf_swz(int(blk0) / 8 + k, c) * 16);
    scw[4 * k + 0] = s4.x;
    scw[4 * k + 1] = s4.y;
    scw[4 * k + 2] = s4.z;
    scw[4 * k + 3] = s4.w;
  }
  static_assert(BPW == 16, "two super-blocks per wave span");
  const uint32_t dw = *reinterpret_cast<const uint32_t*>(slot + G::DOFF + c * 32 + (int(blk0) / 8) * 2);
  const float dsb[2] = {h2f(dw & 0xFFFFu), h2f(dw >> 16)};
  const uint8_t* row = slot + c * G::RB;
  const int h = g & 1, e = g >> 1;
  const uint32_t sl = 4u * uint32_t(h), sre = 2u * uint32_t(h), slo = 4u - 2u * uint32_t(h);
  const f16x2 off = {(_Float16)-1056.0f, (_Float16)-1056.0f};
  // codes of one dword (bytes 0..3) as fp16 q - 32 in slot order 0, 2, 1, 3
  auto dec = [&](uint32_t q, f16x2& r02, f16x2& r13) {
    r02 = half2_of((q & mbyte) | magic) + off;
    r13 = half2_of(((q >> 8) & mbyte) | magic) + off;
  };
#pragma unroll
  for (int p = 0; p < BPW / 2; ++p) {
    const int b = int(blk0) + 2 * p + e;
    const u32x4 lw = *reinterpret_cast<const u32x4*>(row + mf_swz(b, c) * 16);
    const uint2 hw = *reinterpret_cast<const uint2*>(row + mf_swz(G::NB + (b >> 1), c) * 16 + 8 * (b & 1));
    const uint32_t w[4] = {lw.x, lw.y, lw.z, lw.w};
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t H = (k >> 1) ? hw.y : hw.x;
      const uint32_t hx = (k & 1) ? (H << slo) : (H >> sre);
      q[k] = ((w[k] >> sl) & 0x0F0F0F0Fu) | (hx & 0x30303030u);
    }
    f16x8 bw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f16x2 a02, a13, b02, b13;
      dec(q[2 * j], a02, a13);
      dec(q[2 * j + 1], b02, b13);
      bw[j] = f16x8{a02[0], a02[1], a13[0], a13[1], b02[0], b02[1], b13[0], b13[1]};
    }
    // d sc of the lane's block-half: a plain int8_t cast (see mf_tile_q6q8)
    const float ds = dsb[p >> 2] * float(int(int8_t(uint8_t(scw[p] >> (8u * uint32_t(g))))));
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[ch][2 * p], bw[0], d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[ch][2 * p + 1], bw[1], d, 0, 0, 0);
      const int rr = ch == 0 ? RR0 : M - 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < rr) acc[ch][i] = fmaf(ds, d[i], acc[ch][i]);
    }
  }
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = __float_as_uint(acc[ch][i]);
      const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      acc[ch][i] = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
      v = __float_as_uint(acc[ch][i]);
      const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      acc[ch][i] = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    }
}

// ---------------------------------------------------------------------------
// Grouped blocks for fp16 activations (weight-ring kernel, one fp16 term).
// With one term, A rows M..15 of the one-block-per-MFMA layout are padding.
// Here E = 16 / RB blocks share a chain of E v_mfma_f32_16x16x32_f16, RB = 8
// result rows per block for M <= 8 (E = 2) or RB = 4 for M <= 4 (E = 4):
// A rows RB e .. RB e + RB - 1 carry the activation rows of block b + e in lane
// group(s) of that block and zeros elsewhere, and the B operand of lane (g, c)
// holds only block b + g / (4 / E) of weight row c.  Each MFMA of the chain
// takes 32 / E elements of every block of the group, so after the chain
// result row r is block b + r / RB's full dot with activation row r % RB, and
// every lane's four results belong to one block: one scale per lane and
// group.  As in the integer version, only the pairing of positions matters:
// position i of A lane (g, r) meets position i of B lane (g, c).
//
// B operand of lane (g, c), chain step j, from the weight unit of its block
// (q4_0: byte i holds element i in the low and i + 16 in the high nibble;
// q8_0: plane p holds elements 16 p .. 16 p + 15):
//   E = 2, h = g % 2: elements 16 j + 8 h + (0..7) (q4_0: bytes 8h..8h+7,
//     low nibbles for j = 0, high for j = 1; q8_0: plane j, bytes 8h..8h+7);
//   E = 4: elements 8 j + (0..7) (q4_0: bytes 8 (j % 2) .. +7, low nibbles for
//     j < 2, high for j >= 2; q8_0: plane j / 2, bytes 8 (j % 2) .. +7).
// Within the eight, decode_q4_0 / decode_q8_0 leave the slot order
// 0, 2, 1, 3, 4, 6, 5, 7, and the A operand takes the same order.

// Element offset (in the wave's span of 8 blocks of one staging pass) of
// chain step j of lane group g for the group gl of the pass.
template <int E>
__device__ inline int grp_elem(int gl, int g, int j) {
  if constexpr (E == 2)
    return 32 * (2 * gl + (g >> 1)) + 16 * j + 8 * (g & 1);
  else
    return 32 * (4 * gl + g) + 8 * j;
}


// A operands of the wave's BPW blocks in the grouped layout (ap[E gi + j] is
// chain step j of group gi) and the power-of-two unscale of each lane's
// result rows; loads, scaling and hooks as mf_stage with one term.  The
// fp16 rows go through the wave-private area (M x GRP_ROW bytes) one pass of
// 8 blocks at a time.
//
// XT = 2 (E = 2): the activation as two fp16 terms, hi = fp16(x s) and lo =
// fp16(x s - hi).  For M <= 4 the eight A rows of a block carry the hi parts
// of activation rows 0..3, then their lo parts, so lane groups g and g ^ 1
// hold the two halves of the same sums; for M = 5..8 the lo parts are a
// second set of operands (al), a second MFMA chain against the same B
// operand into the same result.  The area holds the hi rows, then the lo
// rows (2 M x GRP_ROW bytes).
//
// KQ (q4_K): ks[gi] receives the block sums S of the activation values the
// MFMAs see (hi + lo with two terms) for the lane's result rows of its block
// in group gi (the min term -dmin m_j S), zero where a result row is not an
// activation row or (lo rows of the M <= 4 two-term layout) would count it
// twice; the sums go through M x BPW floats after the staging rows.
template <int M, int BPW, int E, int XT = 1, bool KQ = false, class Between, class AfterX>
__device__ inline void mf_stage_grp(const MfArgs& a, uint8_t* area, uint32_t blk0, int lane, f16x8 (&ap)[BPW],
                                    f16x8 (&al)[BPW], float (&unscale)[4], f32x4 (&ks)[BPW / E], Between between,
                                    AfterX after_x) {
  static_assert((E == 2 && M <= 8) || (E == 4 && M <= 4), "result rows per block of a group");
  static_assert(XT == 1 || E == 2, "two terms: two blocks per chain");
  static_assert(BPW % 8 == 0, "whole staging passes");
  constexpr int RB = 16 / E;
  constexpr bool LOROWS = XT == 2 && M <= 4;  // lo parts in the block's rows 4..7
  constexpr bool LOCHAIN = XT == 2 && M > 4;  // lo parts as a second chain
  const int g = lane >> 4, c = lane & 15;
  f32x4 xv[M][BPW / 8];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int e = 0; e < BPW / 8; ++e)
      xv[m][e] = *reinterpret_cast<const f32x4*>(a.x + size_t(m) * size_t(a.K) + size_t(blk0) * 32 + 256 * e + 4 * lane);
  __builtin_amdgcn_sched_barrier(0);
  between();
  __builtin_amdgcn_sched_barrier(0);
  float sc[M], us[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < BPW / 8; ++e)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[m][e].x), fabsf(xv[m][e].y)), fmaxf(fabsf(xv[m][e].z), fabsf(xv[m][e].w))));
    mx = wave_max(mx);
    int se = 15 - __builtin_amdgcn_frexp_expf(mx);
    se = se > 126 ? 126 : (se < -126 ? -126 : se);
    sc[m] = __builtin_ldexpf(1.0f, se);
    us[m] = __builtin_ldexpf(1.0f, -se);
  }
  // result rows of lane (g, c): activation rows RB (g % (4 / E)) .. + 3 when
  // RB = 8, rows 0 .. 3 when RB = 4
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (E == 2 && !LOROWS ? 4 * (g & 1) : 0) + i;
    unscale[i] = 1.f;
#pragma unroll
    for (int mm = 0; mm < M; ++mm)
      if (mm == m) unscale[i] = us[mm];
  }
  after_x();
  // A row c of the lane: area row mrow (two terms: the hi rows, then the lo
  // rows)
  const int sub = c % RB;
  const int mrow = LOROWS ? (sub < 4 ? sub : M + sub - 4) : sub;
  const bool on = (c / RB) == (E == 2 ? (g >> 1) : g) && (LOROWS ? (sub & 3) : sub) < M;
  const uint8_t* rd = area + (on ? mrow : 0) * GRP_ROW;
  const uint8_t* rdl = area + (on ? M + mrow : 0) * GRP_ROW;  // LOCHAIN
#pragma unroll
  for (int e = 0; e < BPW / 8; ++e) {
    // a wave's LDS accesses complete in order: this pass's writes are seen by
    // its reads, and its reads finish before the next pass writes
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const f32x4 v = xv[m][e] * sc[m];
      const f16x2 p01 = __builtin_convertvector((f32x2{v.x, v.y}), f16x2);
      const f16x2 p23 = __builtin_convertvector((f32x2{v.z, v.w}), f16x2);
      *reinterpret_cast<u32x2*>(area + m * GRP_ROW + 8 * lane) = u32x2{bits(p01), bits(p23)};
      float part = (float(p01[0]) + float(p01[1])) + (float(p23[0]) + float(p23[1]));
      if constexpr (XT == 2) {
        const f16x2 l01 = __builtin_convertvector((f32x2{v.x, v.y} - __builtin_convertvector(p01, f32x2)), f16x2);
        const f16x2 l23 = __builtin_convertvector((f32x2{v.z, v.w} - __builtin_convertvector(p23, f32x2)), f16x2);
        *reinterpret_cast<u32x2*>(area + (M + m) * GRP_ROW + 8 * lane) = u32x2{bits(l01), bits(l23)};
        part += (float(l01[0]) + float(l01[1])) + (float(l23[0]) + float(l23[1]));
      }
      if constexpr (KQ) {
        // the 8 lanes of a block (lane / 8) add their shares; lane 8 bl keeps
        // row m's sum of block 8 e + bl
        part += dpp_f<SKG_DPP_QUAD_XOR1>(part);
        part += dpp_f<SKG_DPP_QUAD_XOR2>(part);
        part += dpp_f<SKG_DPP_ROW_HALF_MIRROR>(part);
        if ((lane & 7) == 0)
          reinterpret_cast<float*>(area + XT * M * GRP_ROW)[m * BPW + 8 * e + (lane >> 3)] = part;
      }
    }
#pragma unroll
    for (int gl = 0; gl < 8 / E; ++gl)
#pragma unroll
      for (int j = 0; j < E; ++j) {
        // elements 0..7 in order -> slots 0, 2, 1, 3, 4, 6, 5, 7
        auto slots = [&](const uint8_t* src) {
          const u32x4 r = *reinterpret_cast<const u32x4*>(src + 2 * grp_elem<E>(gl, g, j));
          const u32x4 s = {__builtin_amdgcn_perm(r.y, r.x, 0x05040100u), __builtin_amdgcn_perm(r.y, r.x, 0x07060302u),
                           __builtin_amdgcn_perm(r.w, r.z, 0x05040100u), __builtin_amdgcn_perm(r.w, r.z, 0x07060302u)};
          return __builtin_bit_cast(f16x8, on ? s : u32x4{0u, 0u, 0u, 0u});
        };
        ap[E * (e * (8 / E) + gl) + j] = slots(rd);
        if constexpr (LOCHAIN) al[E * (e * (8 / E) + gl) + j] = slots(rdl);
      }
  }
  if constexpr (KQ) {
    // the wave's own LDS writes are visible to its later reads
    const float* sums = reinterpret_cast<const float*>(area + XT * M * GRP_ROW);
    const int gb = (E == 2) ? (g >> 1) : g;
    const int base = (E == 2 && !LOROWS) ? 4 * (g & 1) : 0;
    const bool live = !(LOROWS && (g & 1));
#pragma unroll
    for (int gi = 0; gi < BPW / E; ++gi) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = base + i;
        v[i] = (live && m < M) ? sums[(m < M ? m : 0) * BPW + E * gi + gb] : 0.f;
      }
      ks[gi] = f32x4{v[0], v[1], v[2], v[3]};
    }
  }
}

// One tile of the weight-ring kernel with grouped blocks (layout above); RR:
// result rows per lane that can be output rows.  On return every lane holds
// the full sums of its result rows (lane groups holding the same activation
// rows have been added).
// LOCHAIN: the lo operands al are a second chain (two terms, M = 5..8).
// KQ (q4_K): the slot's scale rows hold the 16-byte super-block headers; the
// codes enter as the exact fp16 subnormals c 2^-24 (one AND per pair, no
// offset to cancel), and sub-block j of a super-block adds
// 2^24 d sc_j D - dmin m_j S with S the block sums of ks.
template <class G, int BPW, int E, int RR, bool LOROWS = false, bool LOCHAIN = false, bool KQ = false>
__device__ inline void mf_tile_grp(const uint8_t* slot, uint32_t blk0, int g, int c, const f16x8 (&ap)[BPW],
                                   const f16x8 (&al)[BPW], const f32x4 (&ks)[BPW / E], float (&acc)[4], uint32_t mlo,
                                   uint32_t mhi, uint32_t magic) {
  uint32_t scw[(E == 2 || KQ) ? BPW / 2 : 1];
  if constexpr (E == 2 || KQ) {
#pragma unroll
    for (int k = 0; k < BPW / 8; ++k) {
      const u32x4 s4 =
          *reinterpret_cast<const u32x4*>(slot + 16 * G::RB + c * G::SRS + mf_swz(int(blk0) / 8 + k, c) * 16);
      scw[4 * k + 0] = s4.x;
      scw[4 * k + 1] = s4.y;
      scw[4 * k + 2] = s4.z;
      scw[4 * k + 3] = s4.w;
    }
  }
  const uint8_t* row = slot + c * G::RB;
  const int gb = (E == 2) ? (g >> 1) : g;  // this lane's block within a group
  const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const f16x2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  // q4_0 nibbles of two dwords (bytes 0..7 of the eight) as n - 8, low or
  // high nibbles, in slot order
  auto q4lo = [&](uint32_t w0, uint32_t w1) {
    const f16x2 r0 = half2_of((w0 & mlo) | magic) + off, r1 = half2_of(((w0 >> 8) & mlo) | magic) + off;
    const f16x2 r2 = half2_of((w1 & mlo) | magic) + off, r3 = half2_of(((w1 >> 8) & mlo) | magic) + off;
    return f16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  };
  auto q4hi = [&](uint32_t w0, uint32_t w1) {
    const f16x2 r0 = __builtin_elementwise_fma(half2_of((w0 & mhi) | magic), sixteenth, off16);
    const f16x2 r1 = __builtin_elementwise_fma(half2_of(((w0 >> 8) & mhi) | magic), sixteenth, off16);
    const f16x2 r2 = __builtin_elementwise_fma(half2_of((w1 & mhi) | magic), sixteenth, off16);
    const f16x2 r3 = __builtin_elementwise_fma(half2_of(((w1 >> 8) & mhi) | magic), sixteenth, off16);
    return f16x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  };
#pragma unroll
  for (int gi = 0; gi < BPW / E; ++gi) {
    const int b = int(blk0) + E * gi + gb;
    f16x8 bw[E];
    if constexpr (KQ) {
      if constexpr (E == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(row + mf_swz(b, c) * 16 + 8 * (g & 1));
        bw[0] = __builtin_bit_cast(f16x8, u32x4{u.x & mlo, (u.x >> 8) & mlo, u.y & mlo, (u.y >> 8) & mlo});
        bw[1] = __builtin_bit_cast(f16x8, u32x4{(u.x >> 4) & mlo, (u.x >> 12) & mlo, (u.y >> 4) & mlo, (u.y >> 12) & mlo});
      } else {
        const u32x4 u = *reinterpret_cast<const u32x4*>(row + mf_swz(b, c) * 16);
        bw[0] = __builtin_bit_cast(f16x8, u32x4{u.x & mlo, (u.x >> 8) & mlo, u.y & mlo, (u.y >> 8) & mlo});
        bw[1] = __builtin_bit_cast(f16x8, u32x4{u.z & mlo, (u.z >> 8) & mlo, u.w & mlo, (u.w >> 8) & mlo});
        bw[2] = __builtin_bit_cast(f16x8, u32x4{(u.x >> 4) & mlo, (u.x >> 12) & mlo, (u.y >> 4) & mlo, (u.y >> 12) & mlo});
        bw[3] = __builtin_bit_cast(f16x8, u32x4{(u.z >> 4) & mlo, (u.z >> 12) & mlo, (u.w >> 4) & mlo, (u.w >> 12) & mlo});
      }
    } else if constexpr (G::NP == 1) {
      if constexpr (E == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(row + mf_swz(b, c) * 16 + 8 * (g & 1));
        bw[0] = q4lo(u.x, u.y);
        bw[1] = q4hi(u.x, u.y);
      } else {
        const u32x4 u = *reinterpret_cast<const u32x4*>(row + mf_swz(b, c) * 16);
        bw[0] = q4lo(u.x, u.y);
        bw[1] = q4lo(u.z, u.w);
        bw[2] = q4hi(u.x, u.y);
        bw[3] = q4hi(u.z, u.w);
      }
    } else {
      if constexpr (E == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint2 u = *reinterpret_cast<const uint2*>(row + mf_swz(j * G::NB + b, c) * 16 + 8 * (g & 1));
          bw[j] = decode_q8_0(u.x, u.y);
        }
      } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const u32x4 u = *reinterpret_cast<const u32x4*>(row + mf_swz(p * G::NB + b, c) * 16);
          bw[2 * p] = decode_q8_0(u.x, u.y);
          bw[2 * p + 1] = decode_q8_0(u.z, u.w);
        }
      }
    }
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < E; ++j) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[E * gi + j], bw[j], d, 0, 0, 0);
    if constexpr (LOCHAIN) {
#pragma unroll
      for (int j = 0; j < E; ++j) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[E * gi + j], bw[j], d, 0, 0, 0);
    }
    if constexpr (KQ) {
      // header of super-block (E gi + gb) / 8 of the span (E gi / 8: the
      // group never straddles two), sub-block (E gi + gb) % 8
      const int hb = 4 * ((E * gi) >> 3);
      uint32_t sc, mn;
      q4_K_sc_m(scw[hb + 1], scw[hb + 2], scw[hb + 3], uint32_t((E * gi + gb) & 7), sc, mn);
      const float aw = h2f(scw[hb] & 0xFFFFu) * float(sc) * 16777216.0f;  // exact: 2^24 d sc_j
      const float bw = h2f(scw[hb] >> 16) * float(mn);
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i] = fmaf(aw, d[i], fmaf(-bw, ks[gi][i], acc[i]));
    } else {
      // fp16 scale of block b: with E = 2 half gb of word gi of the quads
      // read above; with E = 4 the lane's own 2-byte read (a word chosen per
      // lane would go through scratch)
      uint32_t sw;
      if constexpr (E == 2)
        sw = scw[gi] >> (16u * uint32_t(gb));
      else
        sw = *reinterpret_cast<const uint16_t*>(slot + 16 * G::RB + c * G::SRS + mf_swz(b >> 3, c) * 16 + (b & 7) * 2);
      const float s = h2f(sw & 0xFFFFu);
#pragma unroll
      for (int i = 0; i < RR; ++i) acc[i] = fmaf(s, d[i], acc[i]);
    }
  }
  // lane groups g and g + 2 (and, with E = 4 or two terms, g ^ 1) hold
  // parts of the same sums
#pragma unroll
  for (int i = 0; i < RR; ++i) {
    uint32_t v = __float_as_uint(acc[i]);
    const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    acc[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (E == 4 || LOROWS) {
      v = __float_as_uint(acc[i]);
      const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      acc[i] = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    }
  }
}

// LDS bytes of one launch with up to WAVES waves: per-wave activation
// staging, reused afterwards for the two reduction buffers.
template <int M, int WAVES, int BPW, int XT, int NR>
struct MfLds {
  // one pass of 8 blocks; A entries of (XT M | 1) 16-byte units (the hi rows,
  // then the lo rows), see mf_stage
  static constexpr int WAVE_STAGE = 8 * 4 * ((XT * M) | 1) * 16;
  static constexpr int STAGE = WAVES * WAVE_STAGE;
  static constexpr int RED = 2 * WAVES * NR * MF_ROWS * M * 4;
  static constexpr int BYTES = STAGE > RED ? STAGE : RED;
};

// Activation staging of one wave: loads the wave's span of K of every
// activation row once, calls between() (which may issue weight loads into
// registers, so they are in flight during the arithmetic), picks a
// power-of-two scale per row, calls after_x() once the activation registers
// have been consumed (weight transfers straight into LDS go there: the
// compiler drains those before any later use of a register load), and leaves
// the fp16 A operands of the wave's BPW blocks in ah / al.  Passes of 8
// blocks go through the wave-private LDS area `area`.
//
// SUMS (q4_K): ksum receives the A operand of the min term (mf_tile): lane
// (g, c) the block sums S of activation row c (of the values the MFMA sees),
// times 2^-6 so that they stay inside fp16 (|S| < 32 2^15), for blocks
// 8 (g / 2) .. +7 of the span, as their high fp16 part (g even) or the fp16
// rounding of the rest (g odd); zero past the span.
template <int M, int BPW, int XT, int MS = ((XT * M) | 1), bool SUMS = false, class Between, class AfterX>
__device__ inline void mf_stage(const MfArgs& a, uint8_t* area, uint32_t blk0, int lane, f16x8 (&ah)[BPW],
                                f16x8 (&al)[BPW], float (&unscale)[4], f16x8& ksum, Between between,
                                AfterX after_x) {
  const int g = lane >> 4, c = lane & 15;
  // A entry (block, quarter) holds XT M 16-byte units (the hi rows, then the
  // lo rows) at a stride of MS units; an odd stride (XT M | 1, the default)
  // makes the 32 entries a pass writes
  // (and the 4 a read takes) start on different bank groups: with an even
  // stride such as M = 8 (128 bytes, half the 64 banks) they pile onto two.
  static_assert(MS >= XT * M, "entry stride");
  uint8_t* hi_base = area;
  uint8_t* lo_base = area + M * 16;  // lo rows follow the hi rows of each entry
  const int mr = (c < M) ? c : c % M;
  // two terms: A rows 0..7 take the high parts of activation rows 0..7, rows
  // 8..15 the low parts (rows past M repeat a row; their results are unused)
  const int mp = ((c & 7) < M) ? (c & 7) : (c & 7) % M;
  const uint8_t* a_base = (XT == 2 && c >= 8) ? lo_base : hi_base;
  f32x4 xv[M][BPW / 8];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int e = 0; e < BPW / 8; ++e)
      xv[m][e] = *reinterpret_cast<const f32x4*>(a.x + size_t(m) * size_t(a.K) + size_t(blk0) * 32 + 256 * e + 4 * lane);
  __builtin_amdgcn_sched_barrier(0);
  between();
  __builtin_amdgcn_sched_barrier(0);
  // per activation row: the largest |x| in this wave's span of K
  float sc[M], us[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < BPW / 8; ++e)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[m][e].x), fabsf(xv[m][e].y)), fmaxf(fabsf(xv[m][e].z), fabsf(xv[m][e].w))));
    mx = wave_max(mx);
    // mx = f 2^e with f in [0.5, 1): |x| 2^(15-e) < 2^15; both factors stay
    // normal floats
    int se = 15 - __builtin_amdgcn_frexp_expf(mx);
    se = se > 126 ? 126 : (se < -126 ? -126 : se);
    sc[m] = __builtin_ldexpf(1.0f, se);
    us[m] = __builtin_ldexpf(1.0f, -se);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m0 = i, m1 = 4 + i;
    unscale[i] = (m0 < M) ? us[m0 < M ? m0 : 0] : 1.f;
    if (m1 < M && g == 1) unscale[i] = us[m1 < M ? m1 : 0];
  }
  after_x();
  // A wave's LDS accesses complete in order, so its own writes are visible
  // to its reads without a barrier, and a pass's reads finish before the
  // next pass overwrites.
  float part[SUMS ? BPW / 8 : 1][SUMS ? M : 1];
#pragma unroll
  for (int e = 0; e < BPW / 8; ++e) {
    // element 256 e + 4 lane + i of the wave lies in block 8 e + bl, quarter
    // gq, half h; slots 4h .. 4h+3 of A entry (bl, gq, m) hold elements
    // 0, 2, 1, 3.
    const int bl = lane >> 3, h = (lane >> 2) & 1, gq = lane & 3;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const f32x4 v = xv[m][e] * sc[m];
      const f16x2 h02 = __builtin_convertvector((f32x2{v.x, v.z}), f16x2);
      const f16x2 h13 = __builtin_convertvector((f32x2{v.y, v.w}), f16x2);
      const size_t off = size_t(((bl * 4 + gq) * MS + m) * 16 + 8 * h);
      *reinterpret_cast<u32x2*>(hi_base + off) = u32x2{bits(h02), bits(h13)};
      f16x2 l02 = {(_Float16)0.0f, (_Float16)0.0f}, l13 = l02;
      if constexpr (XT == 2) {
        const f32x2 r02 = f32x2{v.x, v.z} - __builtin_convertvector(h02, f32x2);
        const f32x2 r13 = f32x2{v.y, v.w} - __builtin_convertvector(h13, f32x2);
        l02 = __builtin_convertvector(r02, f16x2);
        l13 = __builtin_convertvector(r13, f16x2);
        *reinterpret_cast<u32x2*>(lo_base + off) = u32x2{bits(l02), bits(l13)};
      }
      if constexpr (SUMS) {
        // this lane's share (4 elements) of the block sum of what the MFMA sees
        float p = (float(h02[0]) + float(h02[1])) + (float(h13[0]) + float(h13[1]));
        if constexpr (XT == 2) p += (float(l02[0]) + float(l02[1])) + (float(l13[0]) + float(l13[1]));
        part[e][m] = p;
      }
    }
#pragma unroll
    for (int jl = 0; jl < 8; ++jl) {
      const size_t off = size_t(((jl * 4 + g) * MS + (XT == 2 ? mp : mr)) * 16);
      ah[8 * e + jl] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(a_base + off));
      al[8 * e + jl] = ah[8 * e + jl];
    }
  }
  if constexpr (SUMS) {
    // the 8 lanes of a block (lane / 8) add their shares (two quad exchanges
    // and the half-row mirror); lane 8 bl stores the sums [m][block] in the
    // area, free now (its last reads are above), and each lane reads its 8
    static_assert(BPW == 8 || BPW == 16, "operand layout");
    static_assert(M * BPW * 4 <= 8 * 4 * MS * 16, "block sums fit the staging area");
    float* sarea = reinterpret_cast<float*>(area);
#pragma unroll
    for (int e = 0; e < BPW / 8; ++e)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float p = part[e][m];
        p += dpp_f<SKG_DPP_QUAD_XOR1>(p);
        p += dpp_f<SKG_DPP_QUAD_XOR2>(p);
        p += dpp_f<SKG_DPP_ROW_HALF_MIRROR>(p);
        if ((lane & 7) == 0) sarea[m * BPW + 8 * e + (lane >> 3)] = p;
      }
    const int sb = g >> 1;
    f16x8 t;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // two terms: the high and low rows share one block sum, carried by rows
      // 0..7 only
      const bool live = 8 * sb < BPW && !(XT == 2 && c >= 8);
      const float sv = live ? sarea[(XT == 2 ? mp : mr) * BPW + (8 * sb) % BPW + j] * 0.015625f : 0.0f;
      const _Float16 hi = (_Float16)sv;
      t[j] = (g & 1) ? (_Float16)(sv - float(hi)) : hi;
    }
    ksum = t;
  }
}

// Launched with nb / BPW waves (at most WAVES), so every wave owns BPW
// blocks; requires nb % BPW == 0.
template <int FMT, int M, int WAVES, int BPW, int XT, int EPI, int PD>
__global__ __launch_bounds__(WAVES * 64) void gemv_mfma_kernel(const MfArgs a) {
  static_assert(PD == 1 || PD == 2, "prefetch depth: tiles in flight per wave");
  static_assert(BPW % 8 == 0, "whole 16-byte scale loads");
  constexpr bool Q8 = (FMT == SKG_Q4_0_Q8_1 || FMT == SKG_Q8_0_Q8_1);
  // q4_K: the q4_0 unit layout, with the 16-byte super-block headers as the
  // scale words (one per 8 blocks)
  constexpr bool KQ = (FMT == SKG_Q4_K_F32);
  static_assert(FMT == SKG_Q4_0_F32 || FMT == SKG_Q8_0_F32 || KQ || Q8, "quantised weight formats only");
  static_assert(!KQ || EPI == SKG_EPI_NONE, "q4_K: plain output");
  static_assert(!Q8 || (XT == 1 && EPI == SKG_EPI_NONE), "Q8_1 activations: one integer term, plain output");
  constexpr int NP = (FMT == SKG_Q8_0_F32 || FMT == SKG_Q8_0_Q8_1) ? 2 : 1;
  constexpr int NR = (EPI == SKG_EPI_SWIGLU) ? 2 : 1;
  constexpr int RR = M < 4 ? M : 4;  // accumulator rows a lane can own
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  // The nibble masks (SGPRs) and fp16 1024.0 in both halves (a VGPR) are
  // made opaque here, before any MFMA, so each q4_0 pair decodes in one
  // v_and_or_b32 (two literals do not fit one instruction).  The empty asm
  // statements emit nothing.
  uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
  asm volatile("" : "+s"(mlo));
  asm volatile("" : "+s"(mhi));
  asm volatile("" : "+v"(magic));
  const int nw = int(blockDim.x) >> 6;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const uint32_t blk0 = uint32_t(wave) * BPW;

  const int t0 = blockIdx.x;
  const int step = int(gridDim.x);
  if (t0 >= a.ntiles) return;  // uniform per workgroup: no barrier is skipped by part of it
  const int nmine = (a.ntiles - t0 + step - 1) / step;

  auto seg_of = [&](int t) {
    MfSeg sg = a.seg[0];
#pragma unroll
    for (int i = 1; i < MAX_SEGS; ++i)
      if (i < a.nseg && t >= a.seg[i].tile_begin) sg = a.seg[i];
    return sg;
  };
  auto next_of = [&](MfNext (&nx)[NR], int t) {
    const MfSeg sg = seg_of(t);
    int64_t n = int64_t(t - sg.tile_begin) * MF_ROWS + c;
    n = (n < sg.N) ? n : sg.N - 1;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const PackedW& P = (r == 0) ? sg.w0 : sg.w1;
      nx[r].rowp = P.payload + size_t(n) * P.row_bytes;
      nx[r].srow = P.scales + size_t(n) * P.nb;
      nx[r].nb = P.nb;
    }
  };
  // ---- activation staging: A operands of this wave's BPW blocks, with the
  // first tiles' weight loads issued between the activation loads and the
  // staging arithmetic ----
  MfW<NP, BPW> w[NR], w2[NR];
  MfNext nx[NR];
  f16x8 ah[Q8 ? 1 : BPW], al[Q8 ? 1 : BPW];
  uint64_t aq[Q8 ? BPW : 1];
  f32x4 da[Q8 ? BPW : 1];
  float unscale[4] = {1.f, 1.f, 1.f, 1.f};  // 2^e of the activation rows this lane's outputs belong to
  f16x8 ksum = {};                            // q4_K: block sums, the A operand of the min term
  auto first_loads = [&] {
    next_of(nx, t0);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int q = 0; q < BPW / 4; ++q)
        mf_load_quad<NP, BPW>(w[r], q, nx[r].rowp, nx[r].nb, blk0, g);
      mf_load_scales<NP, BPW>(w[r], nx[r].srow, blk0);
    }
    if constexpr (PD == 2) {
      // second tile (the first again when there is none:
      // unconditional loads keep the compiler's waits exact)
      next_of(nx, nmine > 1 ? t0 + step : t0);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int q = 0; q < BPW / 4; ++q)
          mf_load_quad<NP, BPW>(w2[r], q, nx[r].rowp, nx[r].nb, blk0, g);
        mf_load_scales<NP, BPW>(w2[r], nx[r].srow, blk0);
      }
    }
  };
  if constexpr (Q8)
    mf_stage_q8<M, BPW>(a, reinterpret_cast<uint32_t*>(lds) + size_t(wave) * (M * q8_stage_row<BPW>()), blk0, lane,
                        aq, da,
                        first_loads, [] {});
  else
    mf_stage<M, BPW, XT, ((XT * M) | 1), KQ>(a, lds + size_t(wave) * MfLds<M, WAVES, BPW, XT, 1>::WAVE_STAGE, blk0, lane, ah, al,
                                      unscale, ksum, first_loads, [] {});
  __syncthreads();  // the staging area becomes the reduction buffers

  float* red = reinterpret_cast<float*>(lds);
  int parity = 0;

  auto process = [&](MfW<NP, BPW>(&w)[NR], int t, auto reload, const MfNext (&nx)[NR]) {
    constexpr bool RELOAD = decltype(reload)::value;
    float acc[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r][i] = 0.f;
      if constexpr (Q8)
        mf_tile_q8<NP, BPW, RR, RELOAD>(w[r], aq, da, acc[r], nx[r], blk0, g);
      else
        mf_tile<NP, BPW, RR, XT, RELOAD, KQ>(w[r], ah, al, acc[r], mlo, mhi, magic, nx[r], blk0, g, ksum);
    }
    // partial sums: lane (g, c) holds rows m = 4g + i of output row c
    float* rb = red + size_t(parity) * (WAVES * NR * MF_ROWS * M);
    parity ^= 1;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < RR; ++i) {
        const int m = 4 * g + i;
        if (m < M) rb[((wave * NR + r) * MF_ROWS + c) * M + m] = acc[r][i] * unscale[i];
      }
    // One barrier per tile: the buffer written here is rewritten two tiles
    // later, after the next tile's barrier, which its readers pass only once
    // they are done.
    __syncthreads();
    // 16 M outputs; a launch may have a single wave (K = 32 BPW)
    for (int o = int(threadIdx.x); o < MF_ROWS * M; o += int(blockDim.x)) {
      const int cc = o / M, m = o % M;
      float v[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float s = 0.f;
        for (int ww = 0; ww < nw; ++ww) s += rb[((ww * NR + r) * MF_ROWS + cc) * M + m];
        v[r] = s;
      }
      const MfSeg sg = seg_of(t);
      const int64_t n = int64_t(t - sg.tile_begin) * MF_ROWS + cc;
      float out = v[0];
      if constexpr (NR == 2) out = silu_f32(v[0]) * v[1];
      if (n < sg.N) sg.y[size_t(m) * size_t(sg.N) + size_t(n)] = out;
    }
  };

  // Tiles blockIdx.x, + gridDim.x, ...: while a tile is decoded its
  // registers are refilled with the tile PD steps ahead, so PD tiles of loads
  // stay in flight.  Inside the loops every load is unconditional (the
  // compiler's waits stay exact); the last PD tiles are peeled off.
  if constexpr (PD == 1) {
    int t = t0;
    for (int i = 0; i + 1 < nmine; ++i, t += step) {
      next_of(nx, t + step);
      process(w, t, std::true_type{}, nx);
    }
    process(w, t, std::false_type{}, nx);
  } else {
    int i = 0;
    for (; i + 3 < nmine; i += 2) {
      next_of(nx, t0 + (i + 2) * step);
      process(w, t0 + i * step, std::true_type{}, nx);
      next_of(nx, t0 + (i + 3) * step);
      process(w2, t0 + (i + 1) * step, std::true_type{}, nx);
    }
    const int left = nmine - i;
    if (left == 3) {
      next_of(nx, t0 + (i + 2) * step);
      process(w, t0 + i * step, std::true_type{}, nx);
      process(w2, t0 + (i + 1) * step, std::false_type{}, nx);
      process(w, t0 + (i + 2) * step, std::false_type{}, nx);
    } else if (left == 2) {
      process(w, t0 + i * step, std::false_type{}, nx);
      process(w2, t0 + (i + 1) * step, std::false_type{}, nx);
    } else {
      process(w, t0 + i * step, std::false_type{}, nx);
    }
  }
}

// ---------------------------------------------------------------------------
// K = 4096 variant with the weights streamed into LDS.  The loads of the
// register-fed kernel above touch 16 rows x 64 bytes per wave instruction;
// here each wave instruction moves 1 KB of one row straight from HBM into LDS
// (global_load_lds_dwordx4), so every request is whole cache lines and no
// weight registers are held.  A ring of R tile slots (16 rows x all of K,
// plus scales) keeps R - 1 tiles in flight while one is decoded; one barrier
// per tile.  With R = 4 (q4_0 only: four 37 KB slots fit the 160 KB) every
// tile a workgroup owns is requested before the first is decoded, so no
// transfer waits for a slot to drain.  Q8_1 activations take two blocks per
// 64-deep integer MFMA (mf_stage_q8p / mf_tile_q8p above), with the B
// operand read from the slot in its final layout.
//
// LDS rows are not padded: a row's 16-byte chunks are permuted within each
// aligned group of 16 (chunk j of row r sits at position j ^ (r % 16)), so the
// 16 rows a B-operand group reads at one chunk index land on 16 different
// 4-bank groups.  Each lane of a transfer fetches the chunk its destination
// position holds.  (Two workgroups per CU would fit the LDS of the q4_0
// variants with aliased staging, but not their registers: held to 128 VGPRs
// they spill, and ran 2.4-3.3x slower.)

constexpr int MF_DMA_TILES = 4;  // most tiles one workgroup processes

template <int FMT>
struct MfDmaGeom {
  static constexpr int NP = (FMT == SKG_Q8_0_F32 || FMT == SKG_Q8_0_Q8_1) ? 2 : 1;
  static constexpr bool Q6 = FMT == SKG_Q6_K_Q8_1 || FMT == SKG_Q6_K_F32;  // low + high units per row, d rows
  static constexpr int NB = 128;                     // blocks per row (K = 4096)
  static constexpr int RB = Q6 ? NB * 24 : NB * 16 * NP;  // payload bytes per row (LDS row stride)
  static constexpr int SRS = NB * 2;                 // scale bytes per row (16 chunks)
  // q6_K: the rows' fp16 super-block d (32 bytes per row), copied by one
  // 64-lane transfer whose upper half repeats the lower into a pad
  static constexpr int DOFF = 16 * RB + 16 * SRS;
  static constexpr int DREG = Q6 ? 1024 : 0;
  // one tile, plus 256 bytes so that the aliased Q8_1 staging of 8 rows keeps
  // its bank-spreading row stride (8 waves x 8 rows x 145 dwords)
  static constexpr int SLOT = 16 * RB + 16 * SRS + DREG + 256;
  static constexpr int CH = RB / 1024;               // 1 KB transfers per row
  // transfers per wave per tile (2 rows + 4 scale rows [+ the d rows])
  static constexpr int P = 2 * CH + 1 + (Q6 ? 1 : 0);
};


// R: ring slots; ALIAS: the activation staging area shares the last slot
// (its first load is issued after staging); E: 0 for one block per MFMA, or
// 2 / 4 blocks per chain of MFMAs (fp32 activations as one fp16 term; see
// mf_stage_grp); DEFER: the partial sums of all the workgroup's tiles stay
// in LDS and meet once after the last tile, instead of after each tile's
// barrier (faster for the q6_K kernels, slower for the others).
template <int FMT, int M, int XT, int R, bool ALIAS, int E = 0, bool DEFER = false>
__global__ __launch_bounds__(512) void gemv_mfma_dma_kernel(const MfArgs a) {
  constexpr bool Q6 = FMT == SKG_Q6_K_Q8_1;
  constexpr bool Q8 = (FMT == SKG_Q4_0_Q8_1 || FMT == SKG_Q8_0_Q8_1 || FMT == SKG_Q4_K_Q8_1 || Q6);
  constexpr bool Q6F = FMT == SKG_Q6_K_F32;
  static_assert(FMT == SKG_Q4_0_F32 || FMT == SKG_Q8_0_F32 || FMT == SKG_Q4_K_F32 || Q6F || Q8,
                "quantised weight formats only");
  static_assert(!Q6F || XT == 1, "q6_K x fp32: one fp16 term");
  constexpr bool KQF = FMT == SKG_Q4_K_F32;
  static_assert(!KQF || E > 0, "q4_K x fp32: grouped blocks only");
  constexpr int WKQ = FMT == SKG_Q4_0_Q8_1 ? WK_Q4_0 : FMT == SKG_Q4_K_Q8_1 ? WK_Q4_K : WK_Q8_0;
  static_assert(!Q8 || XT == 1, "Q8_1 activations: one integer term");
  static_assert(E == 0 || (!Q8 && (XT == 1 || E == 2)), "grouped blocks: fp32 activations");
  static_assert(R >= 2 && R <= MF_DMA_TILES, "ring slots");
  static_assert(R * MfDmaGeom<FMT>::SLOT <= 160 * 1024, "ring exceeds the LDS");
  using G = MfDmaGeom<FMT>;
  constexpr int NP = G::NP, BPW = 16, WAVES = 8, P = G::P;
  constexpr int RR = M < 4 ? M : 4;
  // per-wave activation staging: fp16 A operands, or the raw Q8_1 blocks;
  // the bank-spreading strides where the staging still fits the shared slot
  constexpr int MSO = (XT * M) | 1;
  constexpr int MSD = (!ALIAS || WAVES * (8 * 4 * MSO * 16) <= G::SLOT) ? MSO : XT * M;
  constexpr int QRP = (!ALIAS || WAVES * M * q8_stage_row<BPW>() * 4 <= G::SLOT) ? q8_stage_row<BPW>() : 9 * BPW;
  constexpr int WAVE_STAGE = Q8 ? M * QRP * 4
                             : (E > 0 || Q6F) ? XT * M * GRP_ROW + (KQF ? M * BPW * 4 : 0)
                                              : 8 * 4 * MSD * 16;
  static_assert(!ALIAS || WAVES * WAVE_STAGE <= G::SLOT, "staging must fit the shared slot");
  // one LDS array, carved: R slots, the own staging area, the partial sums
  constexpr int RED_BYTES = (DEFER ? MF_DMA_TILES : 2) * WAVES * MF_ROWS * M * 4;
  constexpr int STAGE_BYTES = ALIAS ? 0 : WAVES * WAVE_STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[R * G::SLOT + STAGE_BYTES + RED_BYTES];
  uint8_t* const slot0 = lds_all;
  uint8_t* const slot1 = lds_all + G::SLOT;
  uint8_t* const slot2 = lds_all + (R >= 3 ? 2 * G::SLOT : 0);
  uint8_t* const slot3 = lds_all + (R == 4 ? 3 * G::SLOT : 0);
  uint8_t* const stage_own = lds_all + R * G::SLOT;
  float* const red = reinterpret_cast<float*>(lds_all + R * G::SLOT + STAGE_BYTES);

  uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
  asm volatile("" : "+s"(mlo));
  asm volatile("" : "+s"(mhi));
  asm volatile("" : "+v"(magic));
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const uint32_t blk0 = uint32_t(wave) * BPW;
  const int t0 = blockIdx.x;
  const int step = int(gridDim.x);
  if (t0 >= a.ntiles) return;  // uniform per workgroup
  const int nmine = (a.ntiles - t0 + step - 1) / step;

  auto seg_of = [&](int t) {
    MfSeg sg = a.seg[0];
#pragma unroll
    for (int i = 1; i < MAX_SEGS; ++i)
      if (i < a.nseg && t >= a.seg[i].tile_begin) sg = a.seg[i];
    return sg;
  };
  // This wave's share of tile i: rows 2 wave and 2 wave + 1, payload and scales.
  auto dma_tile = [&](uint8_t* slot, int i) {
    const int t = t0 + i * step;
    const MfSeg sg = seg_of(t);
    const int64_t rbase = int64_t(t - sg.tile_begin) * MF_ROWS;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 2 * wave + k;
      const int64_t n = (rbase + r < sg.N) ? rbase + r : sg.N - 1;
      const uint8_t* rowp = sg.w0.payload + size_t(n) * sg.w0.row_bytes;
#pragma unroll
      for (int ch = 0; ch < G::CH; ++ch)
        dma16_stream(rowp + mf_swz(ch * 64 + lane, r) * 16, lds_addr(slot) + uint32_t(r * G::RB + ch * 1024));
    }
    // Scales of rows 4 (wave % 4) .. +3, all 64 lanes (waves 4..7 repeat the
    // identical copies of waves 0..3, so every wave issues the same number of
    // transfers per tile); lane l fills position l % 16 of row 4 (wave % 4) +
    // l / 16.
    {
      const int r = 4 * (wave & 3) + (lane >> 4);
      const int64_t n = (rbase + r < sg.N) ? rbase + r : sg.N - 1;
      const uint16_t* srow = sg.w0.scales + size_t(n) * sg.w0.nb;
      dma16_stream(srow + mf_swz(lane & 15, r) * 8, lds_addr(slot) + uint32_t(16 * G::RB + 4 * (wave & 3) * G::SRS));
    }
    if constexpr (G::Q6) {
      // d rows: lane l copies 16 bytes (chunk l % 2) of row (l / 2) % 16; every
      // wave issues the same copy
      const int r = (lane >> 1) & 15;
      const int64_t n = (rbase + r < sg.N) ? rbase + r : sg.N - 1;
      const uint16_t* drow = sg.w0.dsup + size_t(n) * (sg.w0.nb / 8);
      dma16_stream(drow + 8 * (lane & 1), lds_addr(slot) + uint32_t(G::DOFF));
    }
  };

  uint8_t* stage_area = ALIAS ? (R == 4 ? slot3 : R == 3 ? slot2 : slot1) : stage_own;
  f16x8 ah[Q8 ? 1 : BPW], al[Q8 ? 1 : BPW];
  i32x4 aq[Q8 ? BPW / 2 : 1];
  f32x4 da[Q8 ? BPW / 2 : 1], sa[Q8 ? BPW / 2 : 1];
  i32x4 aq6[Q6 ? 2 : 1][Q6 ? BPW / 2 : 1];
  f32x4 da6[Q6 ? 2 : 1][Q6 ? BPW / 2 : 1];
  f16x8 ap6[Q6F ? 2 : 1][Q6F ? BPW : 1];
  f32x4 ks[E > 0 ? BPW / (E > 0 ? E : 1) : 1];  // q4_K block sums (grouped kernel)
  float unscale[4] = {1.f, 1.f, 1.f, 1.f};
  f16x8 ksum = {};  // unused: no q4_K here
  // The first R tiles' transfers are unconditional (a workgroup with fewer
  // tiles copies its last one again): conditional transfers here would make
  // the compiler drain them all before the staging arithmetic.
  auto clamp = [&](int i) { return i < nmine ? i : nmine - 1; };
  auto first_dma = [&] {
    dma_tile(slot0, 0);
    if constexpr (!(R == 2 && ALIAS)) dma_tile(slot1, clamp(1));
    if constexpr ((R == 3 && !ALIAS) || R == 4) dma_tile(slot2, clamp(2));
    if constexpr (R == 4 && !ALIAS) dma_tile(slot3, clamp(3));
  };
  if constexpr (Q6F)
    mf_stage_q6f<M, BPW>(a, stage_area + size_t(wave) * WAVE_STAGE, blk0, lane, ap6, unscale, [] {}, first_dma);
  else if constexpr (Q6)
    mf_stage_q6q8<M, BPW, QRP>(a, reinterpret_cast<uint32_t*>(stage_area + size_t(wave) * WAVE_STAGE), blk0, lane, aq6,
                               da6, [] {}, first_dma);
  else if constexpr (Q8)
    mf_stage_q8p<M, BPW, WKQ, QRP>(a, reinterpret_cast<uint32_t*>(stage_area + size_t(wave) * WAVE_STAGE), blk0, lane,
                                   aq, da, sa, [] {}, first_dma);
  else if constexpr (E > 0)
    mf_stage_grp<M, BPW, E, XT, KQF>(a, stage_area + size_t(wave) * WAVE_STAGE, blk0, lane, ah, al, unscale, ks,
                                     [] {}, first_dma);
  else
    mf_stage<M, BPW, XT, MSD>(a, stage_area + size_t(wave) * WAVE_STAGE, blk0, lane, ah, al, unscale, ksum, [] {},
                              first_dma);
  if constexpr (ALIAS) {
    // every wave has read its staged operands before the shared slot refills
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (R == 2) dma_tile(slot1, clamp(1));
    if constexpr (R == 3) dma_tile(slot2, clamp(2));
    if constexpr (R == 4) dma_tile(slot3, clamp(3));
  }

  // Waits until this wave's transfers of tile i have landed: tiles
  // i+1 .. min(issued, nmine) - 1 may stay in flight.
  // `issued`: tiles 0 .. issued - 1 have been requested (the first R always).
  auto wait_tile = [&](int i, int issued) {
    const int last = (issued > R ? (issued < nmine ? issued : nmine) : R) - 1;
    const int after = last - i;
    if (after >= 3)
      wait_vmcnt<3 * P>();
    else if (after == 2)
      wait_vmcnt<2 * P>();
    else if (after == 1)
      wait_vmcnt<P>();
    else
      wait_vmcnt<0>();
  };
  auto sync = [] {
    asm volatile("" ::: "memory");       // no LDS access moves past the barrier
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  wait_tile(0, R);
  sync();

  int parity = 0;
  auto run = [&](uint8_t* slot, int i) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Q6F) {
      float a6[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      mf_tile_q6f<G, BPW, M>(slot, blk0, g, c, ap6, a6, magic, 0x00FF00FFu);
      // lane group 0 writes rows 0..3, group 1 rows 4..7 (below, times unscale)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = (g == 1) ? a6[1][k] : a6[0][k];
    } else if constexpr (Q6) {
      float a6[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      mf_tile_q6q8<G, BPW, M>(slot, blk0, g, c, aq6, da6, a6);
      // lane group 0 writes rows 0..3, group 1 rows 4..7 (below)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = (g == 1) ? a6[1][i] : a6[0][i];
    } else if constexpr (Q8) {
      mf_tile_q8p<G, BPW, (M > 4 ? 4 : M), FMT == SKG_Q4_K_Q8_1>(slot, blk0, g, c, aq, da, sa, acc);
    } else if constexpr (E > 0) {
      constexpr bool LOROWS = XT == 2 && M <= 4, LOCHAIN = XT == 2 && !LOROWS;
      mf_tile_grp<G, BPW, E, RR, LOROWS, LOCHAIN, KQF>(slot, blk0, g, c, ah, al, ks, acc, mlo, mhi, magic);
    } else {
      MfW<NP, BPW> w;
#pragma unroll
      for (int q = 0; q < BPW / 4; ++q)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          w.u[q][p] = *reinterpret_cast<const u32x4*>(slot + c * G::RB + mf_swz(p * G::NB + int(blk0) + 4 * q + g, c) * 16);
#pragma unroll
      for (int k = 0; k < BPW / 8; ++k)
        w.sc[k] = *reinterpret_cast<const u32x4*>(slot + 16 * G::RB + c * G::SRS + mf_swz(int(blk0) / 8 + k, c) * 16);
      const MfNext none{};
      mf_tile<NP, BPW, RR, XT, false>(w, ah, al, acc, mlo, mhi, magic, none, blk0, g);
    }
    float* rb = red + (DEFER ? i : parity) * (WAVES * MF_ROWS * M);
    parity ^= 1;
#pragma unroll
    for (int k = 0; k < RR; ++k) {
      const int m = 4 * g + k;
      if (m < M) rb[(wave * MF_ROWS + c) * M + m] = acc[k] * unscale[k];
    }
    // next tile's transfers landed (this wave's), partial sums written;
    // after the barrier every wave is past this slot and the next is full
    if (i + 1 < nmine) wait_tile(i + 1, i + R);
    sync();
    if (i + R < nmine) dma_tile(slot, i + R);
    if constexpr (DEFER) return;
    const int t = t0 + i * step;
    for (int o = int(threadIdx.x); o < MF_ROWS * M; o += 512) {
      const int cc = o / M, m = o % M;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) v += rb[(ww * MF_ROWS + cc) * M + m];
      const MfSeg sg = seg_of(t);
      const int64_t n = int64_t(t - sg.tile_begin) * MF_ROWS + cc;
      if (n < sg.N) sg.y[size_t(m) * size_t(sg.N) + size_t(n)] = v;
    }
  };
  // Straight-line over at most MF_DMA_TILES tiles (the launch sizes the grid
  // so no workgroup gets more): inside a loop the compiler could not tell
  // which slot's transfers had landed and would drain them all per tile.
  static_assert(MF_DMA_TILES == 4, "unrolled for four tiles");
  run(slot0, 0);
  if (1 < nmine) run(slot1, 1);
  if constexpr (R == 4) {
    if (2 < nmine) run(slot2, 2);
    if (3 < nmine) run(slot3, 3);
  } else if constexpr (R == 3) {
    if (2 < nmine) run(slot2, 2);
    if (3 < nmine) run(slot0, 3);
  } else {
    if (2 < nmine) run(slot0, 2);
    if (3 < nmine) run(slot1, 3);
  }
  if constexpr (DEFER) {
    for (int o = int(threadIdx.x); o < nmine * MF_ROWS * M; o += 512) {
      const int i = o / (MF_ROWS * M), cc = (o / M) % MF_ROWS, m = o % M;
      const float* rb = red + i * (WAVES * MF_ROWS * M);
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) v += rb[(ww * MF_ROWS + cc) * M + m];
      const int t = t0 + i * step;
      const MfSeg sg = seg_of(t);
      const int64_t n = int64_t(t - sg.tile_begin) * MF_ROWS + cc;
      if (n < sg.N) sg.y[size_t(m) * size_t(sg.N) + size_t(n)] = v;
    }
  }
  // a workgroup with fewer tiles than slots still has its repeated first
  // transfers in flight: none may outlive the workgroup's LDS
  wait_vmcnt<0>();
}

template <int FMT, int M, int XT, int R, bool ALIAS, bool DEFER = false>
inline GemvEntry gemv_mfma_dma_entry() {
  GemvEntry e{reinterpret_cast<const void*>(&gemv_mfma_dma_kernel<FMT, M, XT, R, ALIAS, 0, DEFER>),
              FMT, M, SKG_EPI_NONE, MF_ROWS, XT, 3, 8, 16};
  e.lds = 0;
  e.max_nb = MfDmaGeom<FMT>::NB;
  e.depth = R;
  return e;
}

// The ring kernel with grouped blocks (x_lds = 5): one fp16 activation term
// with two blocks per MFMA chain for M = 5..8 and four for M <= 4, or two
// terms (XT = 2) with two blocks per chain.
// q6_K x fp32 on the ring kernel (block-halves; x_lds = 5 like the grouped
// kernels, one fp16 term).
template <int M, int R, bool ALIAS, bool DEFER = false>
inline GemvEntry gemv_mfma_q6f_entry() {
  GemvEntry e{reinterpret_cast<const void*>(&gemv_mfma_dma_kernel<SKG_Q6_K_F32, M, 1, R, ALIAS, 0, DEFER>),
              SKG_Q6_K_F32, M, SKG_EPI_NONE, MF_ROWS, 1, 5, 8, 16};
  e.lds = 0;
  e.max_nb = MfDmaGeom<SKG_Q6_K_F32>::NB;
  e.depth = R;
  return e;
}

template <int FMT, int M, int R, bool ALIAS, int XT = 1>
inline GemvEntry gemv_mfma_grp_entry() {
  constexpr int E = (M <= 4 && XT == 1) ? 4 : 2;
  GemvEntry e{reinterpret_cast<const void*>(&gemv_mfma_dma_kernel<FMT, M, XT, R, ALIAS, E>),
              FMT, M, SKG_EPI_NONE, MF_ROWS, XT, 5, 8, 16};
  e.lds = 0;
  e.max_nb = MfDmaGeom<FMT>::NB;
  e.depth = R;
  return e;
}

// Registry entry: ro = output rows per tile, j = fp16 activation terms,
// x_lds = 2 (matrix cores), waves = most waves per workgroup, kw = blocks per
// wave.  The prefetch depth is not part of the key (one depth per instance).
template <int FMT, int M, int WAVES, int BPW, int XT, int EPI, int PD>
inline GemvEntry gemv_mfma_entry() {
  constexpr int NR = (EPI == SKG_EPI_SWIGLU) ? 2 : 1;
  GemvEntry e{reinterpret_cast<const void*>(&gemv_mfma_kernel<FMT, M, WAVES, BPW, XT, EPI, PD>),
              FMT, M, EPI, MF_ROWS, XT, 2, WAVES, BPW};
  e.lds = MfLds<M, WAVES, BPW, XT, NR>::BYTES;
  if constexpr (FMT == SKG_Q4_0_Q8_1 || FMT == SKG_Q8_0_Q8_1) {
    constexpr int q8_stage = WAVES * M * q8_stage_row<BPW>() * 4;  // each wave's Q8_1 blocks
    if (e.lds < q8_stage) e.lds = q8_stage;
  }
  e.max_nb = WAVES * BPW;
  e.depth = PD;
  return e;
}

}  // namespace skg
