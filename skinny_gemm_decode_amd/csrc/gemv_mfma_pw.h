// Small-batch GEMV on the matrix cores with a private weight ring per wave:
// y[m][n] = sum_k W[n][k] x[m][k] for q4_0 / q8_0 weights and fp32
// activations, 2 <= M <= 8, K a multiple of 512 up to 4096.
//
// The arithmetic is that of gemv_mfma.h (one v_mfma_f32_16x16x32_f16 per
// 32-element block of 16 weight rows, codes decoded exactly to fp16, the
// block's fp16 scale applied to the fp32 result, the activation as one or two
// fp16 terms under a power-of-two scale); what differs is how the waves are
// fed and synchronised:
//
// * Wave w owns blocks 16 w .. 16 w + 15 of every row, for the whole launch.
//   It copies its own slice of each 16-row tile (16 rows x 16 blocks, plus
//   the 16 x 16 fp16 scales) straight from HBM into a ring of R slots in LDS
//   that no other wave reads, so no wave ever waits at a workgroup barrier
//   until the last tile is done: each wave refills a slot as soon as it has
//   read it, and the weight stream never stalls behind the slowest wave.
// * In a slot the 16-byte units sit block-major ([plane][block][row]), so
//   lane (g, c) reads dword g of block j of row c with one 4-byte LDS load
//   (64 lanes, 64 distinct banks) and holds the MFMA B operand directly: no
//   cross-lane transpose.  A copy instruction moves four blocks of 16 rows
//   (64-byte pieces of each row), and a second wave instruction the rest of
//   the same cache lines right after it.
// * The activation needs no LDS: lane (g, c) loads elements 4g..4g+3 and
//   16+4g..16+4g+3 of each of its 16 blocks of activation row c, exactly the
//   A operand, and the power-of-two scale of each half of the wave's span
//   (eight blocks) comes from a four-lane max.
// * A workgroup owns a contiguous range of rows (all of N spread over every
//   CU: 56 rows per CU at N = 14336, i.e. three full tiles and one of 8 rows,
//   whose missing rows are neither copied nor stored).  Partial sums of all
//   its tiles stay in LDS and meet after one barrier at the end.
#pragma once

#include "gemv_mfma.h"

namespace skg {

constexpr int PW_BPW = 16;   // blocks per wave
constexpr int PW_MAXT = 4;   // most 16-row tiles per workgroup (64 rows)

// Slot layout (per wave, per tile): for plane p and row half h (rows 8h ..
// 8h + 7), a group of 16 blocks x 8 rows of 16-byte units, unit (j, r) at
// 16 (8 j + r); the groups of a plane 2176 bytes apart (2048 + a 128-byte
// pad, so the two row halves fall on opposite halves of the LDS banks) and
// the planes 4224 bytes apart; then the fp16 scales [16 rows][16 blocks].
template <int FMT>
struct PwGeom {
  static constexpr int NP = (FMT == SKG_Q8_0_F32 || FMT == SKG_Q8_0_Q8_1) ? 2 : 1;
  static constexpr int GRP = 2048 + 128;             // one (plane, row half) group, padded
  static constexpr int PLANE = 2 * GRP - 128;        // 4224
  static constexpr int SCL_OFF = NP * PLANE;
  static constexpr int SLOT = SCL_OFF + 16 * PW_BPW * 2;
  static constexpr int PI = NP * 4;                  // payload copy instructions per tile (1 KB each)
  static constexpr int P = PI + 1;                   // copy instructions per tile (with the scales)
};

// Rows of a launch: the concatenated rows of up to MAX_SEGS matrices.
struct PwSeg {
  PackedW w;
  float* y;
  int64_t row_begin;  // first row of this matrix in the concatenation
  int64_t N;
};

struct PwArgs {
  PwSeg seg[MAX_SEGS];
  int nseg;
  int64_t ntot;         // rows in all
  int64_t rows_per_wg;  // 1 .. 16 * PW_MAXT
  int64_t K;
  uint32_t nb;
  const float* x;
};

template <int FMT, int M, int R>
inline size_t pw_lds_bytes(int waves) {
  return size_t(waves) * R * PwGeom<FMT>::SLOT + size_t(PW_MAXT) * waves * 16 * M * 4;
}

// One 16-byte activation load straight into registers, left to the caller
// to wait for (s_waitcnt vmcnt): written as asm so that the compiler, which
// cannot see the asm copies into LDS issued after it, does not wait for
// those as well before the activation is used.
__device__ inline void ld_x_async(f32x4& v, const float* p) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p) : "memory");
}

// Launched with nb / 16 waves (nb % 16 == 0, nb <= 128) and
// pw_lds_bytes<FMT, M, R>(waves) bytes of dynamic LDS.
template <int FMT, int M, int XT, int R>
__global__ __launch_bounds__(512, 1) void gemv_mfma_pw_kernel(const PwArgs a) {
  static_assert(FMT == SKG_Q4_0_F32 || FMT == SKG_Q8_0_F32, "fp32-activation quantised formats");
  static_assert(M >= 1 && M <= 8 && (XT == 1 || XT == 2) && R >= 2 && R <= 3, "configuration");
  using G = PwGeom<FMT>;
  constexpr int NP = G::NP, BPW = PW_BPW;
  constexpr int RR = M < 4 ? M : 4;  // accumulator rows a lane can own
  static_assert(R * G::P <= 63, "copies in flight must fit the vmcnt field");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u, magic = 0x64006400u;
  asm volatile("" : "+s"(mlo));
  asm volatile("" : "+s"(mhi));
  asm volatile("" : "+v"(magic));
  const int nw = int(blockDim.x) >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const uint32_t blk0 = uint32_t(wave) * BPW;

  const int64_t r0 = int64_t(blockIdx.x) * a.rows_per_wg;
  const int64_t r1 = (r0 + a.rows_per_wg < a.ntot) ? r0 + a.rows_per_wg : a.ntot;
  if (r0 >= r1) return;  // uniform per workgroup
  const int nt = int((r1 - r0 + 15) / 16);  // <= PW_MAXT; every tile holds row r0 + 16 t

  uint8_t* ring = lds + size_t(wave) * R * G::SLOT;
  float* red = reinterpret_cast<float*>(lds + size_t(nw) * R * G::SLOT);  // [PW_MAXT][nw][16][M]

  // Segment of a global row (rows of the first segment start at 0).
  auto seg_of = [&](int64_t row) {
    PwSeg s = a.seg[0];
#pragma unroll
    for (int i = 1; i < MAX_SEGS; ++i)
      if (i < a.nseg && row >= a.seg[i].row_begin) s = a.seg[i];
    return s;
  };

  // This wave's copy instructions of tile i into slot i % R.  Payload
  // instruction (p, h, b) moves blocks 8b .. 8b + 7 of plane p of rows
  // 8h .. 8h + 7: one whole 128-byte line per row.  Lanes of rows past the
  // end are masked off, except lane 0, which then copies 16 bytes of the
  // tile's first row (which always exists) into the unit of a row that is
  // never stored: every instruction executes, so each counts once in vmcnt.
  auto dma_tile = [&](int i) {
    const uint32_t slot = lds_addr(ring + (i % R) * G::SLOT);
    const int64_t rbase = r0 + 16 * int64_t(i);
    const int rl = lane & 7, jb = lane >> 3;  // row within the half, block within the eight
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t row = rbase + 8 * h + rl;
      const bool valid = row < r1;
      const PwSeg s = seg_of(valid ? row : rbase);
      const uint8_t* pay = s.w.payload + size_t((valid ? row : rbase) - s.row_begin) * s.w.row_bytes;
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          if (valid || lane == 0)
            dma16_stream(pay + (size_t(p) * a.nb + blk0 + uint32_t(8 * b + jb)) * 16,
                  slot + uint32_t(p * G::PLANE + h * G::GRP + 1024 * b));
    }
    // scales: lane 2 r + e copies the eight scales of blocks 8e .. 8e + 7 of row r
    const int64_t srow = rbase + (lane >> 1);
    const bool svalid = lane < 32 && srow < r1;
    const PwSeg s = seg_of(svalid ? srow : rbase);
    const uint16_t* sc = s.w.scales + size_t((svalid ? srow : rbase) - s.row_begin) * s.w.nb;
    if (svalid) dma16_stream(sc + blk0 + uint32_t(8 * (lane & 1)), slot + uint32_t(G::SCL_OFF));
  };

  // ---- the activation slice (asm loads), then the first R tiles, then one
  // wait for the activation alone: the copies stay in flight ----
  const bool xrow = c < M;
  f32x4 xl[BPW], xh[BPW];  // elements 4g..4g+3 and 16+4g..16+4g+3 of each block of row c
  {
    const float* xr = a.x + size_t(xrow ? c : 0) * size_t(a.K) + size_t(blk0) * 32 + 4 * g;
    if (xrow) {
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        ld_x_async(xl[j], xr + 32 * j);
        ld_x_async(xh[j], xr + 32 * j + 16);
      }
    }
  }
  for (int i = 0; i < R; ++i)
    if (i < nt) dma_tile(i);
  // outstanding after the activation: the copies of min(R, nt) tiles
  {
    const int issued = nt < R ? nt : R;
    if (issued >= 3)
      wait_vmcnt<3 * G::P>();
    else if (issued == 2)
      wait_vmcnt<2 * G::P>();
    else
      wait_vmcnt<G::P>();
  }
  // the registers written by the activation loads are read only from here on
#pragma unroll
  for (int j = 0; j < BPW; ++j) asm volatile("" : "+v"(xl[j]), "+v"(xh[j]));

  f16x8 ah[BPW], al[BPW];
  float us[2][4];  // unscale of this lane's output rows 4g + i, per half of the span
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float mx = 0.f;
#pragma unroll
    for (int jl = 0; jl < 8; ++jl) {
      const f32x4 vl = xl[8 * h + jl], vh = xh[8 * h + jl];
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(vl.x), fabsf(vl.y)), fmaxf(fabsf(vl.z), fabsf(vl.w))));
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(vh.x), fabsf(vh.y)), fmaxf(fabsf(vh.z), fabsf(vh.w))));
    }
    mx = xrow ? mx : 0.f;  // lanes past M never loaded
    // the four lanes of row c (g = 0..3) sit 16 lanes apart
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // mx = f 2^e, f in [0.5, 1): |x| 2^(15-e) < 2^15, both factors normal
    int se = 15 - __builtin_amdgcn_frexp_expf(mx);
    se = se > 126 ? 126 : (se < -126 ? -126 : se);
    const float sc = xrow ? __builtin_ldexpf(1.0f, se) : 0.f;
    const float u = __builtin_ldexpf(1.0f, -se);
#pragma unroll
    for (int jl = 0; jl < 8; ++jl) {
      const f32x4 vl = xl[8 * h + jl] * sc, vh = xh[8 * h + jl] * sc;
      // slot order of the B operand: elements 4g, 4g+2, 4g+1, 4g+3, then +16
      const f16x2 h0 = __builtin_convertvector((f32x2{vl.x, vl.z}), f16x2);
      const f16x2 h1 = __builtin_convertvector((f32x2{vl.y, vl.w}), f16x2);
      const f16x2 h2 = __builtin_convertvector((f32x2{vh.x, vh.z}), f16x2);
      const f16x2 h3 = __builtin_convertvector((f32x2{vh.y, vh.w}), f16x2);
      ah[8 * h + jl] = f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      if constexpr (XT == 2) {
        const f16x2 l0 = __builtin_convertvector((f32x2{vl.x, vl.z} - __builtin_convertvector(h0, f32x2)), f16x2);
        const f16x2 l1 = __builtin_convertvector((f32x2{vl.y, vl.w} - __builtin_convertvector(h1, f32x2)), f16x2);
        const f16x2 l2 = __builtin_convertvector((f32x2{vh.x, vh.z} - __builtin_convertvector(h2, f32x2)), f16x2);
        const f16x2 l3 = __builtin_convertvector((f32x2{vh.y, vh.w} - __builtin_convertvector(h3, f32x2)), f16x2);
        al[8 * h + jl] = f16x8{l0[0], l0[1], l1[0], l1[1], l2[0], l2[1], l3[0], l3[1]};
      } else {
        al[8 * h + jl] = ah[8 * h + jl];
      }
    }
    // this lane's output rows are 4g + i: fetch their unscale from lane 4g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const float v = __shfl(u, m & 15, 64);
      us[h][i] = (m < M) ? v : 0.f;
    }
  }

  for (int i = 0; i < nt; ++i) {
    // copies issued after tile i's: tiles i + 1 .. min(i + R, nt) - 1
    const int after = ((i + R < nt) ? i + R : nt) - 1 - i;
    if (after >= 2)
      wait_vmcnt<2 * G::P>();
    else if (after == 1)
      wait_vmcnt<G::P>();
    else
      wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    const uint8_t* slot = ring + (i % R) * G::SLOT;
    uint32_t scw[8];  // the 16 fp16 scales of row c
    {
      const u32x4 s0 = *reinterpret_cast<const u32x4*>(slot + G::SCL_OFF + c * 32);
      const u32x4 s1 = *reinterpret_cast<const u32x4*>(slot + G::SCL_OFF + c * 32 + 16);
      scw[0] = s0.x; scw[1] = s0.y; scw[2] = s0.z; scw[3] = s0.w;
      scw[4] = s1.x; scw[5] = s1.y; scw[6] = s1.z; scw[7] = s1.w;
    }
    // unit (j, row c) of plane p: group (p, c / 8), unit 8 j + c % 8
    const uint32_t* u0 = reinterpret_cast<const uint32_t*>(slot + (c >> 3) * G::GRP + (c & 7) * 16) + g;
    float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      // dword g of block j, row c (and of its second plane for q8_0)
      const uint32_t w0 = u0[32 * j];
      f16x8 bw;
      if constexpr (NP == 1) {
        bw = decode_q4_0(w0, mlo, mhi, magic);
      } else {
        const uint32_t w1 = u0[G::PLANE / 4 + 32 * j];
        bw = decode_q8_0(w0, w1);
      }
      f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[j], bw, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      if constexpr (XT == 2) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[j], bw, d, 0, 0, 0);
      const uint32_t sw = scw[j >> 1];
      const float s = h2f((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
      for (int r = 0; r < RR; ++r) acc[j >> 3][r] = fmaf(s, d[r], acc[j >> 3][r]);
    }
    // this wave's partial sums of tile i: lane (g, c) holds rows m = 4g + r of output row c
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const int m = 4 * g + r;
      if (m < M) red[((i * nw + wave) * 16 + c) * M + m] = acc[0][r] * us[0][r] + acc[1][r] * us[1][r];
    }
    if (i + R < nt) {
      // every LDS read of this slot has returned before it is refilled
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      dma_tile(i + R);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  // partial sums of every tile meet: one output (tile, row, m) per thread
  for (int o = int(threadIdx.x); o < nt * 16 * M; o += int(blockDim.x)) {
    const int t = o / (16 * M), cc = (o / M) % 16, m = o % M;
    const int64_t row = r0 + 16 * int64_t(t) + cc;
    if (row >= r1) continue;
    float v = 0.f;
    for (int ww = 0; ww < nw; ++ww) v += red[((t * nw + ww) * 16 + cc) * M + m];
    const PwSeg s = seg_of(row);
    s.y[size_t(m) * size_t(s.N) + size_t(row - s.row_begin)] = v;
  }
}

// Registry entry: ro = 16 rows per tile, j = fp16 activation terms, x_lds = 4
// (per-wave ring), waves = 8 (most), kw = 16 blocks per wave, depth = R.
template <int FMT, int M, int XT, int R>
inline GemvEntry gemv_mfma_pw_entry() {
  GemvEntry e{reinterpret_cast<const void*>(&gemv_mfma_pw_kernel<FMT, M, XT, R>), FMT, M, SKG_EPI_NONE, MF_ROWS, XT,
              4, 8, PW_BPW};
  e.lds = int(pw_lds_bytes<FMT, M, R>(8));
  e.max_nb = 8 * PW_BPW;
  e.depth = R;
  return e;
}

// Dynamic LDS bytes of a per-wave-ring launch with `waves` waves.
inline size_t pw_lds_bytes_of(const GemvEntry& e, int waves) {
  const int slot = e.fmt == SKG_Q8_0_F32 ? PwGeom<SKG_Q8_0_F32>::SLOT : PwGeom<SKG_Q4_0_F32>::SLOT;
  return size_t(waves) * e.depth * slot + size_t(PW_MAXT) * waves * 16 * e.M * 4;
}

}  // namespace skg
