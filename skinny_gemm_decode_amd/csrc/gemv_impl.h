// Skinny GEMM / GEMV kernels: y[m][n] = sum_k W[n][k] x[m][k], 1 <= M <= 8.
//
// The decode product streams every weight once from HBM ("The Shape That
// Actually Matters", The shape a decode step actually runs), so the kernel is
// organised around the weight stream:
//
// * A wave owns RO output rows (2*RO weight rows for the SwiGLU epilogue).
//   Its 64 lanes split K into 16-byte units: lane l takes units l, l+64, ...
//   so each wave-wide 16-byte load reads 1 KB of one row contiguously, and a
//   lane always owns whole q4_0 / q8_0 blocks ("Six hypotheses, four
//   refutations", What the failure left behind: a full data block per lane
//   through wide loads, several output rows per workgroup).
// * K is walked in chunks of 64*J units per lane-row; all RT*J weight loads of
//   a chunk are issued before any of them is consumed.
// * The activation is fetched once per wave per chunk and reused for every
//   row the wave owns: from global memory into registers (XLDS = false), or
//   staged once per workgroup in LDS (XLDS = true) for larger M.  Re-fetching
//   an already cached activation per row is exactly the waste the MI50 case
//   study found (Hypothesis ledger: 3 of 5 memory instructions per iteration).
// * Products accumulate in fp32 (int32 within a block for the Q8_1 formats),
//   then one DPP/shuffle reduction per output over the 64 lanes.
#pragma once

#include "common.h"

namespace skg {

template <int FMT>
struct Fmt;

// E: elements per 16-byte weight unit; WV: payload dwords per unit; XB, XF:
// activation bytes and floats per unit; KQ: 4 or 6 for the K-quant
// super-block formats q4_K / q6_K, else 0.
template <>
struct Fmt<SKG_BF16_BF16> {
  static constexpr int E = 8, WV = 4, XB = 16, XF = 8, KQ = 0;
  static constexpr bool SCALE = false, XQ8 = false, XSUM = false;
};
template <>
struct Fmt<SKG_Q8_0_F32> {
  static constexpr int E = 32, WV = 8, XB = 128, XF = 32, KQ = 0;
  static constexpr bool SCALE = true, XQ8 = false, XSUM = false;
};
template <>
struct Fmt<SKG_Q4_0_F32> {
  static constexpr int E = 32, WV = 4, XB = 128, XF = 32, KQ = 0;
  static constexpr bool SCALE = true, XQ8 = false, XSUM = false;
};
template <>
struct Fmt<SKG_Q4_0_Q8_1> {
  static constexpr int E = 32, WV = 4, XB = 36, XF = 0, KQ = 0;
  static constexpr bool SCALE = true, XQ8 = true, XSUM = false;
};
template <>
struct Fmt<SKG_Q8_0_Q8_1> {
  static constexpr int E = 32, WV = 8, XB = 36, XF = 0, KQ = 0;
  static constexpr bool SCALE = true, XQ8 = true, XSUM = false;
};
// K-quant super-block weights (256 elements): one unit per 32-element
// sub-block; their scales are decoded per unit from the super-block header
// (q4_K) or the int8 scale and fp16 d streams (q6_K).
template <>
struct Fmt<SKG_Q4_K_F32> {
  static constexpr int E = 32, WV = 4, XB = 128, XF = 32, KQ = 4;
  static constexpr bool SCALE = false, XQ8 = false, XSUM = true;
};
template <>
struct Fmt<SKG_Q6_K_F32> {
  static constexpr int E = 32, WV = 4, XB = 128, XF = 32, KQ = 6;
  static constexpr bool SCALE = false, XQ8 = false, XSUM = false;
};
template <>
struct Fmt<SKG_Q4_K_Q8_1> {
  static constexpr int E = 32, WV = 4, XB = 36, XF = 0, KQ = 4;
  static constexpr bool SCALE = false, XQ8 = true, XSUM = false;
};
template <>
struct Fmt<SKG_Q6_K_Q8_1> {
  static constexpr int E = 32, WV = 4, XB = 36, XF = 0, KQ = 6;
  static constexpr bool SCALE = false, XQ8 = true, XSUM = false;
};

// One 16-byte (bf16, q4_0) or 2x16-byte (q8_0) weight unit and its scale.
// The K-quant units keep their scale words raw until the unit is consumed, so
// that no load result is needed while the chunk's loads are being issued.
template <int FMT, int KQ = Fmt<FMT>::KQ>
struct WUnit {
  uint32_t w[Fmt<FMT>::WV];
  float d;
};
// q4_K: lane l always owns units u with u = l (mod 64), so the eight lanes
// 8s .. 8s+7 hold the eight sub-blocks of one super-block and each quad of
// them can hold its whole 16-byte header: lane l loads header dword l & 3 and
// the quad exchanges them (DPP) when the unit is consumed.
template <int FMT>
struct WUnit<FMT, 4> {
  uint32_t w[4];  // codes, q4_0 order
  uint32_t hd;    // header dword (lane & 3): d | dmin << 16, or 4 of the 12 scale/min bytes
  float a, b;     // d * sc and dmin * m of the unit's sub-block (set by prep_w)
};
template <int FMT>
struct WUnit<FMT, 6> {
  uint32_t w[4];  // low four bits of the codes, q4_0 order
  uint32_t h[2];  // top two bits (crumbs, see the packed layout)
  uint32_t sc;    // int8 scales of elements 0..15 (low byte) and 16..31
  uint32_t d;     // fp16 bits of the super-block's d
  float alo, ahi;  // d * scale of each half (set by prep_w)
};

// One activation unit in compute form.
template <int FMT, bool Q8 = Fmt<FMT>::XQ8>
struct XUnit;
template <int FMT>
struct XUnit<FMT, false> {
  float v[Fmt<FMT>::XF];
  float sum;   // sum of the block (q6_K: of elements 0..15)
  float sum2;  // q6_K: sum of elements 16..31
};
template <int FMT>
struct XUnit<FMT, true> {
  uint32_t q[8];
  float d, s;
  int qs_lo, qs_hi;  // q6_K: integer sums of codes 0..15 and 16..31
};

template <int FMT>
__device__ inline void zero_w(WUnit<FMT>& u) {
#pragma unroll
  for (int k = 0; k < Fmt<FMT>::WV; ++k) u.w[k] = 0;
  u.d = 0.f;
}

// Weights are read exactly once per launch, so they are loaded non-temporally
// (streamed past the caches that hold the reused activation); measured on
// MI355X this moves the bf16 M=1 GEMV from 17.1 to 15.9 us.
__device__ inline u32x4 ld_u32x4_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// rowp: start of the row's payload; srow: the row's scale stream (fp16
// scales; q4_K super-block headers; q6_K int8 scale pairs); drow: the row's
// q6_K d stream.
template <int FMT>
__device__ inline void load_w(WUnit<FMT>& u, const uint8_t* rowp, const uint16_t* srow, uint32_t nb,
                              uint32_t unit, const uint16_t* drow = nullptr) {
  const u32x4 p = ld_u32x4_stream(rowp + size_t(unit) * 16);
  if constexpr (Fmt<FMT>::KQ == 4) {
    u.w[0] = p.x;
    u.w[1] = p.y;
    u.w[2] = p.z;
    u.w[3] = p.w;
    // dword lane & 3 (= unit & 3, also for a clamped unit past the row's end,
    // so the quad always exchanges one whole header)
    u.hd = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(srow + size_t(unit >> 3) * 8) +
                                      (threadIdx.x & 3u));
  } else if constexpr (Fmt<FMT>::KQ == 6) {
    u.w[0] = p.x;
    u.w[1] = p.y;
    u.w[2] = p.z;
    u.w[3] = p.w;
    const u32x2 h = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rowp + size_t(nb) * 16 + size_t(unit) * 8));
    u.h[0] = h.x;
    u.h[1] = h.y;
    u.sc = __builtin_nontemporal_load(srow + unit);
    u.d = __builtin_nontemporal_load(drow + (unit >> 3));
  } else {
    u.w[0] = p.x;
    u.w[1] = p.y;
    u.w[2] = p.z;
    u.w[3] = p.w;
    if constexpr (Fmt<FMT>::WV == 8) {
      const u32x4 q = ld_u32x4_stream(rowp + (size_t(nb) + unit) * 16);
      u.w[4] = q.x;
      u.w[5] = q.y;
      u.w[6] = q.z;
      u.w[7] = q.w;
    }
    if constexpr (Fmt<FMT>::SCALE) {
      u.d = h2f(__builtin_nontemporal_load(srow + unit));
    } else {
      u.d = 0.f;
    }
  }
}

typedef _Float16 q4h __attribute__((ext_vector_type(2)));
__device__ inline q4h q4h_of(uint32_t v) { return __builtin_bit_cast(q4h, v); }

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ inline float ubyte(uint32_t w, int i) { return float((w >> (8 * i)) & 0xFFu); }

template <int FMT>
__device__ inline void zero_x(XUnit<FMT>& x) {
  if constexpr (Fmt<FMT>::XQ8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x.q[k] = 0;
    x.d = 0.f;
    x.s = 0.f;
  } else {
#pragma unroll
    for (int k = 0; k < Fmt<FMT>::XF; ++k) x.v[k] = 0.f;
    x.sum = 0.f;
  }
}

// Activation unit from raw 16-byte pieces (bf16 / fp32 layouts).
template <int FMT>
__device__ inline void x_from_pieces(XUnit<FMT>& x, const u32x4* pc) {
  if constexpr (FMT == SKG_BF16_BF16) {
    const u32x4 p = pc[0];
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x.v[2 * k] = bf16_lo(w[k]);
      x.v[2 * k + 1] = bf16_hi(w[k]);
    }
    x.sum = 0.f;
  } else {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const u32x4 v = pc[p];
      x.v[4 * p + 0] = __uint_as_float(v.x);
      x.v[4 * p + 1] = __uint_as_float(v.y);
      x.v[4 * p + 2] = __uint_as_float(v.z);
      x.v[4 * p + 3] = __uint_as_float(v.w);
    }
    // The block sum is accumulated in the same element order as the code x
    // activation chain of unit_acc, so that a block whose codes are all 0
    // (q8_0) cancels to exactly zero: scaling every term by a power of two
    // commutes with each rounding.
    if constexpr (Fmt<FMT>::KQ == 6 && Fmt<FMT>::XSUM) {
      // half-block sums, each in the element order of its product chain
      float s2 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += x.v[i];
#pragma unroll
      for (int i = 16; i < 32; ++i) s2 += x.v[i];
      x.sum2 = s2;
    } else if constexpr (Fmt<FMT>::XSUM) {
#pragma unroll
      for (int i = 0; i < 32; ++i) s += x.v[i];
    }
    x.sum = s;
  }
}

// Raw activation unit as loaded from global memory: 16-byte pieces (bf16,
// fp32) or the nine dwords of a Q8_1 block.
template <int FMT, bool Q8 = Fmt<FMT>::XQ8>
struct XRaw;
template <int FMT>
struct XRaw<FMT, false> {
  u32x4 pc[Fmt<FMT>::XB / 16];
};
template <int FMT>
struct XRaw<FMT, true> {
  uint32_t w[9];
};

// Loads activation unit u of row m (u must be in range).
template <int FMT>
__device__ inline void load_x_raw(XRaw<FMT>& r, const uint8_t* xb, int64_t K, uint32_t nb, int m, uint32_t u) {
  if constexpr (Fmt<FMT>::XQ8) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(xb + (size_t(m) * nb + u) * 36);
#pragma unroll
    for (int k = 0; k < 9; ++k) r.w[k] = p[k];
  } else {
    constexpr int PP = Fmt<FMT>::XB / 16;
    constexpr int ESZ = Fmt<FMT>::XB / Fmt<FMT>::E;
    const u32x4* src = reinterpret_cast<const u32x4*>(xb + (size_t(m) * size_t(K) + size_t(u) * Fmt<FMT>::E) * ESZ);
#pragma unroll
    for (int p = 0; p < PP; ++p) r.pc[p] = src[p];
  }
}

// Compute form of a raw unit; ok == false yields the all-zero unit (selects,
// no branch).
template <int FMT>
__device__ inline void x_from_raw(XUnit<FMT>& x, const XRaw<FMT>& r, bool ok) {
  if constexpr (Fmt<FMT>::XQ8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x.q[k] = ok ? r.w[1 + k] : 0u;
    const uint32_t ds = ok ? r.w[0] : 0u;
    x.d = h2f(ds & 0xFFFFu);
    x.s = h2f(ds >> 16);
    if constexpr (Fmt<FMT>::KQ == 6) {
      int lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo = __builtin_amdgcn_sdot4(int(x.q[k]), 0x01010101, lo, false);
        hi = __builtin_amdgcn_sdot4(int(x.q[4 + k]), 0x01010101, hi, false);
      }
      x.qs_lo = lo;
      x.qs_hi = hi;
    }
  } else {
    constexpr int PP = Fmt<FMT>::XB / 16;
    u32x4 pc[PP];
#pragma unroll
    for (int p = 0; p < PP; ++p) pc[p] = ok ? r.pc[p] : u32x4{0u, 0u, 0u, 0u};
    x_from_pieces<FMT>(x, pc);
  }
}

// Activation unit straight from global memory (row m, unit index u).
template <int FMT>
__device__ inline void fetch_x_global(XUnit<FMT>& x, const uint8_t* xb, int64_t K, uint32_t nb, int m,
                                      uint32_t u) {
  XRaw<FMT> r;
  load_x_raw<FMT>(r, xb, K, nb, m, u);
  x_from_raw<FMT>(x, r, true);
}

// Integer block dot of the Q8_1 formats (exact int32).
template <int FMT>
__device__ inline int unit_idot(const WUnit<FMT>& w, const XUnit<FMT, true>& x) {
  int si = 0;
  if constexpr (FMT == SKG_Q4_0_Q8_1 || FMT == SKG_Q4_K_Q8_1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      si = __builtin_amdgcn_sdot4(int(w.w[k] & 0x0F0F0F0Fu), int(x.q[k]), si, false);
      si = __builtin_amdgcn_sdot4(int((w.w[k] >> 4) & 0x0F0F0F0Fu), int(x.q[4 + k]), si, false);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) si = __builtin_amdgcn_sdot4(int(w.w[k]), int(x.q[k]), si, false);
  }
  return si;
}

// Decode constants of the q4_0 fp16 path, made opaque once per kernel
// (SGPR masks, fp16 1024.0 pair in a VGPR) so each code pair decodes in one
// v_and_or_b32: an instruction of that encoding takes at most one literal.
struct DecodeK {
  uint32_t mlo, mhi, magic, mbyte;
};
__device__ inline DecodeK decode_consts() {
  DecodeK k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x00FF00FFu};
  asm volatile("" : "+s"(k.mlo));
  asm volatile("" : "+s"(k.mhi));
  asm volatile("" : "+v"(k.magic));
  asm volatile("" : "+s"(k.mbyte));
  return k;
}

// d * sc_j and dmin * m_j of the calling lane's q4_K sub-block j = lane & 7
// (both exact in binary32: 11-bit by 6-bit products).  The quad's header
// dwords arrive by DPP broadcast (all 64 lanes take part).
template <int CTRL>
__device__ inline uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline void q4_K_scales(uint32_t hd, float& a, float& b) {
  const uint32_t dd = dpp_u<0x00>(hd);  // quad_perm [0,0,0,0]
  const uint32_t s0 = dpp_u<0x55>(hd);  // [1,1,1,1]: s[0..3]
  const uint32_t s1 = dpp_u<0xAA>(hd);  // [2,2,2,2]: s[4..7]
  const uint32_t s2 = dpp_u<0xFF>(hd);  // [3,3,3,3]: s[8..11]
  uint32_t sc, m;
  q4_K_sc_m(s0, s1, s2, threadIdx.x & 7u, sc, m);
  a = h2f(dd & 0xFFFFu) * float(sc);
  b = h2f(dd >> 16) * float(m);
}

// Once per loaded unit, before it meets the M activation rows: the K-quant
// scales are decoded here rather than once per row of the activation.
template <int FMT>
__device__ inline void prep_w(WUnit<FMT>& w) {
  if constexpr (Fmt<FMT>::KQ == 4) {
    q4_K_scales(w.hd, w.a, w.b);
  } else if constexpr (Fmt<FMT>::KQ == 6) {
    const float d = h2f(w.d);
    w.alo = d * float(int8_t(w.sc & 0xFFu));  // exact: 11 x 8 bits
    w.ahi = d * float(int8_t(w.sc >> 8));
  }
}

// acc + (contribution of one weight unit against one activation unit).
template <int FMT>
__device__ inline float unit_acc(const WUnit<FMT>& w, const XUnit<FMT>& x, float acc, const DecodeK& dk) {
  if constexpr (FMT == SKG_BF16_BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = fmaf(bf16_lo(w.w[k]), x.v[2 * k], acc);
      acc = fmaf(bf16_hi(w.w[k]), x.v[2 * k + 1], acc);
    }
    return acc;
  } else if constexpr (FMT == SKG_Q4_0_F32) {
    // Codes decode exactly to fp16 pairs c - 8 (two per v_and_or_b32 and one
    // packed add or fma), and each product takes the fp16 weight and the fp32
    // activation in one mixed-precision fma: exact products, one rounding per
    // element, and a code of 8 contributes exactly zero.
    // two chains (low and high nibbles) halve the dependent-fma depth
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t v = w.w[k], v8 = v >> 8;
      // elements 4k, 4k+2 | 4k+1, 4k+3 (low nibbles) as 1024 + c
      const q4h lo02 = q4h_of((v & dk.mlo) | dk.magic);
      const q4h lo13 = q4h_of((v8 & dk.mlo) | dk.magic);
      // elements 16+4k, 16+4k+2 | 16+4k+1, 16+4k+3 (high nibbles) as 1024 + 16 c
      const q4h hi02 = q4h_of((v & dk.mhi) | dk.magic);
      const q4h hi13 = q4h_of((v8 & dk.mhi) | dk.magic);
      const q4h off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
      const q4h sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
      const q4h off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
      const q4h a = lo02 + off, b = lo13 + off;
      const q4h c = __builtin_elementwise_fma(hi02, sixteenth, off16);
      const q4h e = __builtin_elementwise_fma(hi13, sixteenth, off16);
      s = fmaf(float(a[0]), x.v[4 * k + 0], s);
      s = fmaf(float(b[0]), x.v[4 * k + 1], s);
      s = fmaf(float(a[1]), x.v[4 * k + 2], s);
      s = fmaf(float(b[1]), x.v[4 * k + 3], s);
      t = fmaf(float(c[0]), x.v[16 + 4 * k + 0], t);
      t = fmaf(float(e[0]), x.v[16 + 4 * k + 1], t);
      t = fmaf(float(c[1]), x.v[16 + 4 * k + 2], t);
      t = fmaf(float(e[1]), x.v[16 + 4 * k + 3], t);
    }
    return fmaf(w.d, s + t, acc);
  } else if constexpr (FMT == SKG_Q8_0_F32) {
    // The codes as exact fp16 pairs: q ^ 0x80 is the unsigned byte q + 128, a
    // byte permute puts two of them under the exponent of 1024 (1024 + q +
    // 128) and one packed subtraction of 1152 leaves q; each product takes
    // the fp16 code and the fp32 activation in one mixed-precision fma.  A
    // code of 0 then contributes exactly zero whatever its activation (taking
    // sum (q + 128) x - 128 sum x instead, an activation outlier with a zero
    // weight cancels against itself and erases the rest of its block).
    const q4h off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t u = w.w[k] ^ 0x80808080u;
      const q4h e02 = q4h_of(__builtin_amdgcn_perm(dk.magic | 0x00640064u, u, 0x04020400u)) + off;
      const q4h e13 = q4h_of(__builtin_amdgcn_perm(dk.magic | 0x00640064u, u, 0x04030401u)) + off;
      s = fmaf(float(e02[0]), x.v[4 * k + 0], s);
      s = fmaf(float(e13[0]), x.v[4 * k + 1], s);
      s = fmaf(float(e02[1]), x.v[4 * k + 2], s);
      s = fmaf(float(e13[1]), x.v[4 * k + 3], s);
    }
    return fmaf(w.d, s, acc);
  } else if constexpr (FMT == SKG_Q4_0_Q8_1) {
    const int si = unit_idot<FMT>(w, x);
    return fmaf(w.d, fmaf(x.d, float(si), -8.f * x.s), acc);
  } else if constexpr (FMT == SKG_Q4_K_F32) {
    // w = d sc q - dmin m: the codes decode exactly to fp16 (as for q4_0,
    // without the offset) and the min term takes the block sum of x.
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t v = w.w[k], v8 = v >> 8;
      const q4h lo02 = q4h_of((v & dk.mlo) | dk.magic);
      const q4h lo13 = q4h_of((v8 & dk.mlo) | dk.magic);
      const q4h hi02 = q4h_of((v & dk.mhi) | dk.magic);
      const q4h hi13 = q4h_of((v8 & dk.mhi) | dk.magic);
      const q4h off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
      const q4h sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
      const q4h off16 = {(_Float16)-64.0f, (_Float16)-64.0f};
      const q4h a = lo02 + off, b = lo13 + off;
      const q4h c = __builtin_elementwise_fma(hi02, sixteenth, off16);
      const q4h e = __builtin_elementwise_fma(hi13, sixteenth, off16);
      s = fmaf(float(a[0]), x.v[4 * k + 0], s);
      s = fmaf(float(b[0]), x.v[4 * k + 1], s);
      s = fmaf(float(a[1]), x.v[4 * k + 2], s);
      s = fmaf(float(b[1]), x.v[4 * k + 3], s);
      t = fmaf(float(c[0]), x.v[16 + 4 * k + 0], t);
      t = fmaf(float(e[0]), x.v[16 + 4 * k + 1], t);
      t = fmaf(float(c[1]), x.v[16 + 4 * k + 2], t);
      t = fmaf(float(e[1]), x.v[16 + 4 * k + 3], t);
    }
    return fmaf(w.a, s + t, fmaf(-w.b, x.sum, acc));
  } else if constexpr (FMT == SKG_Q4_K_Q8_1) {
    const int si = unit_idot<FMT>(w, x);
    return fmaf(w.a, x.d * float(si), fmaf(-w.b, x.s, acc));
  } else if constexpr (FMT == SKG_Q6_K_F32) {
    // w = d sc (q - 32) per 16 elements.  The 6-bit codes decode exactly to
    // the fp16 pairs q - 32 (one mask-and-or to 1024 + q, one packed
    // subtraction of 1056) and each product takes the fp16 code and the fp32
    // activation in one mixed-precision fma, so a code of 32 contributes
    // exactly zero whatever its activation (taking sum q x - 32 sum x
    // instead, an activation outlier with a zero weight cancels against
    // itself and erases the rest of its half).
    const q4h off = {(_Float16)-1056.0f, (_Float16)-1056.0f};
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t ca, cb;
      q6_K_codes(w.w, w.h, k, ca, cb);
      // elements 4k, 4k+2 | 4k+1, 4k+3 of each half
      const q4h a02 = q4h_of((ca & dk.mbyte) | dk.magic) + off;
      const q4h a13 = q4h_of(((ca >> 8) & dk.mbyte) | dk.magic) + off;
      const q4h b02 = q4h_of((cb & dk.mbyte) | dk.magic) + off;
      const q4h b13 = q4h_of(((cb >> 8) & dk.mbyte) | dk.magic) + off;
      s = fmaf(float(a02[0]), x.v[4 * k + 0], s);
      s = fmaf(float(a13[0]), x.v[4 * k + 1], s);
      s = fmaf(float(a02[1]), x.v[4 * k + 2], s);
      s = fmaf(float(a13[1]), x.v[4 * k + 3], s);
      t = fmaf(float(b02[0]), x.v[16 + 4 * k + 0], t);
      t = fmaf(float(b13[0]), x.v[16 + 4 * k + 1], t);
      t = fmaf(float(b02[1]), x.v[16 + 4 * k + 2], t);
      t = fmaf(float(b13[1]), x.v[16 + 4 * k + 3], t);
    }
    acc = fmaf(w.alo, s, acc);
    return fmaf(w.ahi, t, acc);
  } else if constexpr (FMT == SKG_Q6_K_Q8_1) {
    // codes 0..63 are non-negative int8, so the signed 4x8-bit dot is exact
    int sa = 0, sb = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t ca, cb;
      q6_K_codes(w.w, w.h, k, ca, cb);
      sa = __builtin_amdgcn_sdot4(int(ca), int(x.q[k]), sa, false);
      sb = __builtin_amdgcn_sdot4(int(cb), int(x.q[4 + k]), sb, false);
    }
    // d * sc * dA * (sum q qa - 32 sum qa) per half: the integer parts are exact
    acc = fmaf(w.alo * x.d, float(sa - 32 * x.qs_lo), acc);
    return fmaf(w.ahi * x.d, float(sb - 32 * x.qs_hi), acc);
  } else {
    const int si = unit_idot<FMT>(w, x);
    return fmaf(w.d * x.d, float(si), acc);
  }
}

__device__ inline float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Units per activation piece plane in LDS for PP pieces of UC units (see
// gemv_kernel).
__host__ __device__ constexpr int gemv_x_plane_stride(int pp, int uc) { return pp > 1 ? uc + 2 : uc; }

// One output segment of a launch: a matrix (two for SwiGLU) and its output
// (plus the Q8_1 form of the SwiGLU output for SKG_EPI_SWIGLU_Q8_1).
struct Seg {
  PackedW w0, w1;
  float* y;
  uint8_t* yq;
  int64_t N;
  int blk_begin;
};

constexpr int MAX_SEGS = 4;

struct GemvArgs {
  Seg seg[MAX_SEGS];
  int nseg;
  int64_t K;
  uint32_t nu;  // 16-byte weight units per row (K/8 bf16, K/32 quantised)
  const uint8_t* x;
};

// Reductions over each 32-lane half of a wave, every lane receiving its
// half's result: DPP within 16-lane rows (pairs, quads, mirrored eights, the
// two mirrored halves of a row), then one swizzle that swaps the two rows of
// each half (bit-mask mode, lane ^ 16).
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int SKG_SWZ_XOR16 = 0x1F | (0x10 << 10);

__device__ inline float half_max(float v) {
  v = fmaxf(v, dpp_f<SKG_DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_ROW_MIRROR>(v));
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), SKG_SWZ_XOR16)));
}
__device__ inline int half_sum(int v) {
  v += dpp_i<SKG_DPP_QUAD_XOR1>(v);
  v += dpp_i<SKG_DPP_QUAD_XOR2>(v);
  v += dpp_i<SKG_DPP_ROW_HALF_MIRROR>(v);
  v += dpp_i<SKG_DPP_ROW_MIRROR>(v);
  return v + __builtin_amdgcn_ds_swizzle(v, SKG_SWZ_XOR16);
}

// One Q8_1 block from 32 values held one per lane by a 32-lane half-wave
// (lane e holds element e), written to dst (36 bytes, 4-byte aligned) when
// `store`.  The per-block steps are those of the standalone quantiser, and
// the cross-lane max and integer sum are exact, so the bits are its bits.
__device__ inline void quantise_half_q8_1(float v, uint8_t* dst, bool store) {
  const uint32_t e = threadIdx.x & 31;
  const float d = q8_1_d(half_max(fabsf(v)));
  const int q = q8_1_code(v, q8_1_id(d));
  const int sum = half_sum(q);
  // codes of lanes 4k .. 4k+3 into one word (quad_perm broadcasts of lanes 1, 2, 3 of each quad)
  const uint32_t b = uint32_t(q) & 0xFFu;
  const uint32_t word = b | (uint32_t(dpp_i<0x55>(int(b))) << 8) | (uint32_t(dpp_i<0xAA>(int(b))) << 16) |
                        (uint32_t(dpp_i<0xFF>(int(b))) << 24);
  const uint32_t ds = q8_1_d16(d) | (q8_1_s16(d, sum) << 16);
  if (store) {
    uint32_t* w = reinterpret_cast<uint32_t*>(dst);
    if ((e & 3) == 0) w[1 + (e >> 2)] = word;
    if (e == 0) w[0] = ds;
  }
}

template <int FMT, int M, int RO, int J, bool XLDS, int WAVES, int EPI, int KW>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const GemvArgs a) {
  using F = Fmt<FMT>;
  constexpr int NR = (EPI == SKG_EPI_NONE) ? 1 : 2;
  constexpr int RT = RO * NR;
  constexpr int UC = 64 * J;
  constexpr int PP = F::XB / 16;
  constexpr int GROUPS = WAVES / KW;  // row groups per workgroup
  static_assert(WAVES % KW == 0, "KW must divide WAVES");
  // With the activation in LDS and K split across waves, the waves of one
  // K class (kw) stage their chunk into LDS region kw; the host launches such
  // a variant only when every class has the same number of chunks.
  constexpr int XCLS = XLDS ? KW : 1;  // LDS chunk regions
  // Stride (16-byte units) of an activation piece plane in LDS.  The staging
  // threads write the PP pieces of a unit with consecutive lanes (so the
  // global loads stay contiguous); a plane stride of UC + 2 units puts the 16
  // stores of 16 lanes (8 pieces x 2 units) on 16 different bank groups,
  // where a stride of UC (a multiple of the 64 banks) put a unit's 8 pieces
  // on one.  The lanes reading a plane take consecutive units either way.
  constexpr int XPS = gemv_x_plane_stride(PP, UC);
  extern __shared__ u32x4 xlds[];
  __shared__ float red[KW > 1 ? WAVES : 1][KW > 1 ? RT * M : 1];
  // SwiGLU outputs of the workgroup's rows, gathered for their Q8_1 blocks
  constexpr int RWG = GROUPS * RO;
  static_assert(EPI != SKG_EPI_SWIGLU_Q8_1 || RWG % QK == 0, "Q8_1 output needs whole 32-row blocks per workgroup");
  __shared__ float hq[EPI == SKG_EPI_SWIGLU_Q8_1 ? M * RWG : 1];

  const int blk = blockIdx.x;
  // Segment of this workgroup; selected with compile-time indices so the
  // argument block is read with scalar loads, never copied to scratch.
  Seg sg = a.seg[0];
#pragma unroll
  for (int i = 1; i < MAX_SEGS; ++i)
    if (i < a.nseg && blk >= a.seg[i].blk_begin) sg = a.seg[i];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // Waves g*KW .. g*KW+KW-1 share row group g and take its K chunks in turn.
  const int kw = wave % KW;
  const int64_t n0 = (int64_t(blk - sg.blk_begin) * GROUPS + wave / KW) * RO;

  const uint8_t* rowp[RT];
  const uint16_t* srow[RT];
  const uint16_t* drow[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const PackedW& P = (r < RO) ? sg.w0 : sg.w1;
    const int64_t n = n0 + (r % RO);
    const int64_t nn = (n < sg.N) ? n : 0;
    rowp[r] = P.payload + size_t(nn) * P.row_bytes;
    srow[r] = P.scales + size_t(nn) * P.nb;
    drow[r] = (F::KQ == 6) ? P.dsup + size_t(nn) * (P.nb / 8) : nullptr;
  }
  const uint32_t nb = sg.w0.nb;
  const uint32_t nu = a.nu;

  float acc[RT][M];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  DecodeK dk{};
  if constexpr (FMT == SKG_Q4_0_F32 || FMT == SKG_Q4_K_F32 || FMT == SKG_Q8_0_F32 || FMT == SKG_Q6_K_F32)
    dk = decode_consts();
  const int nchunks = int((nu + UC - 1) / UC);
  for (int c = kw; c < nchunks; c += KW) {
    const uint32_t ub = uint32_t(c) * UC;
    // Issue order matters: the vector-memory counter retires loads in order,
    // so the activation (small, mostly L2 hits) is requested first and the
    // weight stream second; the first wait then covers only the activation
    // and every weight load stays in flight until it is consumed.
    XRaw<FMT> xr[XLDS ? 1 : J][XLDS ? 1 : M];
    // staging threads: the waves of this K class
    constexpr int ST = (WAVES / XCLS) * 64;
    const int tl = (wave / XCLS) * 64 + lane;
    u32x4 stage[XLDS && !F::XQ8 ? (M * UC * PP + ST - 1) / ST : 1];
    // Q8_1 activation staged whole blocks per thread (nine dwords each)
    constexpr int NQ = (XLDS && F::XQ8) ? (M * UC + ST - 1) / ST : 1;
    uint32_t qstage[NQ][9];
    u32x4* xreg = xlds + size_t(XCLS > 1 ? kw : 0) * (M * PP * XPS);
    uint32_t* qreg = reinterpret_cast<uint32_t*>(xlds) + size_t(XCLS > 1 ? kw : 0) * (M * 9 * UC);
    if constexpr (XLDS && F::XQ8) {
      // Cooperative staging of this chunk's Q8_1 activation, all M rows: thread
      // t copies block t (36 contiguous bytes; a wave reads 2304 contiguous
      // bytes) into nine LDS planes [m][dword][unit], so both the writes here
      // and the lane-per-unit reads later hit consecutive banks.
      if (c != kw) __syncthreads();
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int i = tl + t * ST;
        const int m = i / UC, uu = i % UC;
        const uint32_t gu = ub + uint32_t(uu);
        const bool ok = (m < M) && (gu < nu);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.x + (size_t(ok ? m : 0) * nb + (ok ? gu : 0u)) * 36);
#pragma unroll
        for (int k = 0; k < 9; ++k) qstage[t][k] = ok ? src[k] : 0u;
      }
    } else if constexpr (!XLDS) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t u = ub + uint32_t(j * 64 + lane);
#pragma unroll
        for (int m = 0; m < M; ++m) load_x_raw<FMT>(xr[j][m], a.x, a.K, nb, m, (u < nu) ? u : 0u);
      }
    } else {
      // Cooperative staging of this chunk's activation, all M rows, into a
      // piece-planar LDS layout [m][piece][unit]: lanes reading consecutive
      // units then hit consecutive 16-byte LDS words (no bank conflicts).
      if (c != kw) __syncthreads();
      constexpr int ESZ = F::XB / F::E;
      constexpr int NS = sizeof(stage) / sizeof(stage[0]);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const int i = tl + t * ST;
        const int p = i % PP;
        const int uu = (i / PP) % UC;
        const int m = i / (PP * UC);
        const uint32_t gu = ub + uint32_t(uu);
        const bool ok = (m < M) && (gu < nu);
        const u32x4 v = ld_u32x4(a.x + (size_t(ok ? m : 0) * size_t(a.K) + size_t(ok ? gu : 0u) * F::E) * ESZ +
                                 size_t(p) * 16);
        stage[t] = ok ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // Keep the scheduler from sinking the activation loads below the weight
    // loads (a later wait for them would then drain the weight stream too).
    __builtin_amdgcn_sched_barrier(0);
    // Weight loads are unconditional: a unit past the end of the row reads
    // unit 0 of the row (its activation is zeroed, so it adds exactly 0), and
    // a row past N reads row 0 (its output is never stored).
    WUnit<FMT> w[RT][J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t u = ub + uint32_t(j * 64 + lane);
      const uint32_t uc = (u < nu) ? u : 0u;
#pragma unroll
      for (int r = 0; r < RT; ++r) load_w<FMT>(w[r][j], rowp[r], srow[r], nb, uc, drow[r]);
    }
    // Every load of the chunk is issued before any result is used.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XLDS && F::XQ8) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int i = tl + t * ST;
        if (i < M * UC) {
          const int m = i / UC, uu = i % UC;
#pragma unroll
          for (int k = 0; k < 9; ++k) qreg[(m * 9 + k) * UC + uu] = qstage[t][k];
        }
      }
      __syncthreads();
    } else if constexpr (XLDS) {
      constexpr int NS = sizeof(stage) / sizeof(stage[0]);
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const int i = tl + t * ST;
        if (i < M * UC * PP) {
          const int p = i % PP;
          const int uu = (i / PP) % UC;
          const int m = i / (PP * UC);
          xreg[(m * PP + p) * XPS + uu] = stage[t];
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t u = ub + uint32_t(j * 64 + lane);
      const bool uok = u < nu;
#pragma unroll
      for (int r = 0; r < RT; ++r) prep_w<FMT>(w[r][j]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        XUnit<FMT> xu;
        if constexpr (XLDS && F::XQ8) {
          XRaw<FMT> r;
#pragma unroll
          for (int k = 0; k < 9; ++k) r.w[k] = qreg[(m * 9 + k) * UC + j * 64 + lane];
          x_from_raw<FMT>(xu, r, uok);
        } else if constexpr (XLDS) {
          u32x4 pc[PP];
#pragma unroll
          for (int p = 0; p < PP; ++p) pc[p] = xreg[(m * PP + p) * XPS + j * 64 + lane];
          x_from_pieces<FMT>(xu, pc);
        } else {
          x_from_raw<FMT>(xu, xr[j][m], uok);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) acc[r][m] = unit_acc<FMT>(w[r][j], xu, acc[r][m], dk);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = wave_sum(acc[r][m]);

  if constexpr (KW > 1) {
    // Partial sums of the KW waves of a row group meet in LDS; the group's
    // first wave adds them (in a fixed order) and writes the outputs.
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) red[wave][r * M + m] = acc[r][m];
    }
    __syncthreads();
    // (with the Q8_1 epilogue every wave stays for the block barrier below)
    if (EPI != SKG_EPI_SWIGLU_Q8_1 && kw != 0) return;
    if (kw == 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float t = red[wave][r * M + m];
#pragma unroll
          for (int k = 1; k < KW; ++k) t += red[wave + k][r * M + m];
          acc[r][m] = t;
        }
    }
  }

  float out = 0.f;
#pragma unroll
  for (int ro = 0; ro < RO; ++ro)
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (lane == ro * M + m) {
        if constexpr (EPI != SKG_EPI_NONE)
          out = silu_f32(acc[ro][m]) * acc[RO + ro][m];
        else
          out = acc[ro][m];
      }
  if (kw == 0 && lane < RO * M) {
    const int ro = lane / M;
    const int m = lane % M;
    const int64_t n = n0 + ro;
    if (n < sg.N) sg.y[size_t(m) * size_t(sg.N) + size_t(n)] = out;
    if constexpr (EPI == SKG_EPI_SWIGLU_Q8_1) hq[m * RWG + (wave / KW) * RO + ro] = out;
  }
  if constexpr (EPI == SKG_EPI_SWIGLU_Q8_1) {
    // Every wave reaches this barrier (none returned above).  Then each
    // 32-lane half-wave quantises one block of 32 consecutive outputs of one
    // activation row; blocks past N (N is a multiple of 32) are skipped.
    __syncthreads();
    constexpr int NBLK = M * (RWG / QK);
    const int64_t row0 = int64_t(blk - sg.blk_begin) * RWG;
    const int64_t nbh = sg.N / QK;
    for (int bi = int(threadIdx.x >> 5); bi < NBLK; bi += WAVES * 2) {
      const int m = bi / (RWG / QK), b = bi % (RWG / QK);
      const int64_t hb = row0 / QK + b;  // block index along N
      const float v = hq[m * RWG + b * QK + int(threadIdx.x & 31)];
      quantise_half_q8_1(v, sg.yq + (size_t(m) * size_t(nbh) + size_t(hb < nbh ? hb : 0)) * 36, hb < nbh);
    }
  }
}

// Registry entry of one compiled kernel instance.  xlds: 0 = activation in
// registers, 1 = staged in LDS, 2 = matrix-core kernel (activation held as
// fp16 MFMA operands; j is then the number of fp16 terms per element).
// lds: fixed LDS bytes (matrix-core kernel); max_nb: largest number of
// quantisation blocks per row it handles (0 = any).
struct GemvEntry {
  const void* fn;
  int fmt, M, epi, ro, j, xlds, waves, kw;
  int lds = 0;
  int max_nb = 0;
  // tiles (or K chunks) of weight loads in flight per wave or workgroup:
  // 1 for the vector kernels, the prefetch depth of the register-fed
  // matrix-core kernel, the ring slots of the LDS-ring kernel
  int depth = 1;
};

template <int FMT, int M, int RO, int J, bool XLDS, int WAVES, int EPI, int KW>
inline GemvEntry gemv_entry() {
  return GemvEntry{reinterpret_cast<const void*>(&gemv_kernel<FMT, M, RO, J, XLDS, WAVES, EPI, KW>),
                   FMT, M, EPI, RO, J, XLDS ? 1 : 0, WAVES, KW};
}

// LDS bytes an instance needs (0 when the activation lives in registers).
inline size_t gemv_lds_bytes(int fmt, int M, int J, int xlds, int kw = 1) {
  if (!xlds) return 0;
  const bool q8 = fmt == SKG_Q4_0_Q8_1 || fmt == SKG_Q8_0_Q8_1 || fmt == SKG_Q4_K_Q8_1 || fmt == SKG_Q6_K_Q8_1;
  if (q8) return size_t(M) * size_t(64 * J) * 36 * size_t(kw);
  const int pp = (fmt == SKG_BF16_BF16) ? 1 : 8;  // 16-byte pieces per unit
  return size_t(M) * size_t(pp) * size_t(gemv_x_plane_stride(pp, 64 * J)) * 16 * size_t(kw);
}

}  // namespace skg
