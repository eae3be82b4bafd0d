// Internal definitions shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "skg.h"

namespace skg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QK = 32;  // elements per quantisation block along K

enum WKind { WK_BF16 = 0, WK_Q8_0 = 1, WK_Q4_0 = 2, WK_Q4_K = 3, WK_Q6_K = 4, WK_INVALID = -1 };

constexpr int QK_K = 256;  // elements per K-quant super-block

__host__ __device__ inline int wkind_of(int fmt) {
  switch (fmt) {
    case SKG_BF16_BF16: return WK_BF16;
    case SKG_Q8_0_F32:
    case SKG_Q8_0_Q8_1:
    case SKG_Q8_0_BF16: return WK_Q8_0;
    case SKG_Q4_0_F32:
    case SKG_Q4_0_Q8_1:
    case SKG_Q4_0_BF16: return WK_Q4_0;
    case SKG_Q4_K_F32:
    case SKG_Q4_K_Q8_1:
    case SKG_Q4_K_BF16: return WK_Q4_K;
    case SKG_Q6_K_F32:
    case SKG_Q6_K_Q8_1:
    case SKG_Q6_K_BF16: return WK_Q6_K;
    default: return WK_INVALID;
  }
}

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Packed weight layout (opaque to callers, version 1):
//   payload: row-major, row n at n * row_bytes.  Within a row, 16-byte units
//     in K order: bf16 -> 8 elements per unit (the canonical row unchanged);
//     q4_0 -> one unit per block (its 16 code bytes);
//     q8_0 -> two planes of nb units: plane 0 holds codes 0..15 of every
//             block, plane 1 codes 16..31, so each plane streams contiguously.
//   scales (q8_0, q4_0): fp16 [N][nb] at scale_off (256-byte aligned).
//   q4_K: payload one 16-byte unit per 32-element sub-block, its codes in the
//     q4_0 order (byte i: element i in the low nibble, element 16 + i in the
//     high nibble); at scale_off the 16-byte header {d, dmin, 12 scale bytes}
//     of every super-block [N][K/256], i.e. 2 bytes per 32 elements as q4_0.
//   q6_K: per row nb low units (16 bytes, the low four bits of each code in
//     the q4_0 order) then nb high units (8 bytes: dword t holds, for code
//     dwords k = 2t + s of the low unit, the top two bits of element 4k + b
//     at bits 8b + 4 - 4s and of element 16 + 4k + b at bits 8b + 6 - 4s);
//     int8 sub-block scales [N][K/16] at scale_off; fp16 d [N][K/256] at
//     d_off.
struct Layout {
  int64_t N = 0, K = 0, nb = 0;
  int wk = WK_INVALID;
  size_t row_bytes = 0, payload_bytes = 0, scale_off = 0, d_off = 0, total = 0;
};

__host__ __device__ inline Layout layout_of(int wk, int64_t N, int64_t K) {
  Layout L;
  L.N = N;
  L.K = K;
  L.wk = wk;
  L.nb = K / QK;
  if (wk == WK_BF16) {
    L.row_bytes = size_t(K) * 2;
    L.payload_bytes = size_t(N) * L.row_bytes;
    L.scale_off = align256(L.payload_bytes);
    L.total = L.scale_off;
  } else {
    L.row_bytes = size_t(L.nb) * (wk == WK_Q8_0 ? 32 : wk == WK_Q6_K ? 24 : 16);
    L.payload_bytes = size_t(N) * L.row_bytes;
    L.scale_off = align256(L.payload_bytes);
    L.total = align256(L.scale_off + size_t(N) * size_t(L.nb) * 2);
    if (wk == WK_Q6_K) {
      L.d_off = L.total;
      L.total = align256(L.d_off + size_t(N) * size_t(K / QK_K) * 2);
    }
  }
  return L;
}

// A packed matrix as the kernels see it.
struct PackedW {
  const uint8_t* payload;
  const uint16_t* scales;  // 2 bytes per 32-element block per row (q6_K: two int8 scales)
  const uint16_t* dsup;    // q6_K: fp16 d per super-block [N][K/256]; else null
  uint32_t row_bytes;
  uint32_t nb;
};

inline PackedW packed_view(const void* base, const Layout& L) {
  PackedW p;
  p.payload = static_cast<const uint8_t*>(base);
  p.scales = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(base) + L.scale_off);
  p.dsup = L.d_off ? reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(base) + L.d_off) : nullptr;
  p.row_bytes = uint32_t(L.row_bytes);
  p.nb = uint32_t(L.nb);
  return p;
}

__device__ inline u32x4 ld_u32x4(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Full 6-bit codes of a packed q6_K unit as bytes, from its low unit w and
// high unit h: code dword k of elements 4k..4k+3 (a) and of elements
// 16+4k..16+4k+3 (b).
__device__ inline void q6_K_codes(const uint32_t (&w)[4], const uint32_t (&h)[2], int k, uint32_t& a,
                                  uint32_t& b) {
  const uint32_t H = h[k >> 1];
  const uint32_t hA = (k & 1) ? (H << 4) : H;
  const uint32_t hB = (k & 1) ? (H << 2) : (H >> 2);
  a = (w[k] & 0x0F0F0F0Fu) | (hA & 0x30303030u);
  b = ((w[k] >> 4) & 0x0F0F0F0Fu) | (hB & 0x30303030u);
}

// Scale and min of sub-block j of a q4_K super-block from its 12 packed
// scale bytes s[0..11] (s0 = s[0..3], s1 = s[4..7], s2 = s[8..11]): for
// j < 4, sc = s[j] & 63 and m = s[j + 4] & 63; for j >= 4, the low four bits
// come from s[j + 4] (sc: low nibble, m: high nibble) and the top two from
// bits 6..7 of s[j - 4] (sc) and s[j] (m).
__device__ inline void q4_K_sc_m(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t j, uint32_t& sc, uint32_t& m) {
  const uint32_t sh = 8u * (j & 3u);
  const uint32_t b0 = (s0 >> sh) & 0xFFu, b1 = (s1 >> sh) & 0xFFu, b2 = (s2 >> sh) & 0xFFu;
  const bool lo = j < 4u;
  sc = lo ? (b0 & 63u) : ((b2 & 15u) | ((b0 >> 6) << 4));
  m = lo ? (b1 & 63u) : ((b2 >> 4) | ((b1 >> 6) << 4));
}

// Byte i of v as a float, one v_cvt_f32_ubyte<i> instruction.  Written as
// asm because the compiler otherwise narrows the byte mask it can prove and
// emits a bit-field extract plus a conversion (two VALU ops per element).
template <int I>
__device__ inline float cvt_ubyte(uint32_t v) {
  float r;
  if constexpr (I == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
  if constexpr (I == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
  if constexpr (I == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
  if constexpr (I == 3) asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

__device__ inline float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16)));
}

// Q8_1 quantisation of one 32-element block {fp16 d, fp16 s, int8 q[32]}, as
// the RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach &
// Methodology) feeds the Q4_0 integer-dot matvec.  Every step is one IEEE
// binary32 operation (the library is built without fast-math, so '/' is
// correctly rounded, and contraction is off in these helpers):
//   amax = max|x_i|, d = amax / 127, id = d != 0 ? 1 / d : 0,
//   q_i = round-half-away(x_i * id), stored d = fp16_rne(d),
//   stored s = fp16_rne(binary32(d * sum_i q_i)).
// The steps are shared by the standalone quantiser (one thread per block) and
// the SwiGLU epilogue that quantises its output (one lane per element); max
// and the integer sum do not depend on the order of reduction, so both
// produce the same bits.
__device__ inline float q8_1_d(float amax) {
#pragma clang fp contract(off)
  return amax / 127.0f;
}
__device__ inline float q8_1_id(float d) {
#pragma clang fp contract(off)
  return (d != 0.0f) ? 1.0f / d : 0.0f;
}
__device__ inline int q8_1_code(float v, float id) {
#pragma clang fp contract(off)
  const int q = int(roundf(v * id));
  return q > 127 ? 127 : (q < -127 ? -127 : q);
}
// fp16 bits of d and of the block sum s = d * sum.
__device__ inline uint32_t q8_1_d16(float d) { return __half_as_ushort(__float2half_rn(d)); }
__device__ inline uint32_t q8_1_s16(float d, int sum) {
#pragma clang fp contract(off)
  // The empty asm pins the binary32 product in a register: without it the
  // backend folds multiply and conversion into one v_fma_mix (one rounding,
  // which differs on rare double-rounding ties).
  float sp = d * float(sum);
  asm volatile("" : "+v"(sp));
  return __half_as_ushort(__float2half_rn(sp));
}

struct Q8_1Block {
  uint32_t q[8];  // codes 4k .. 4k+3 in word k, low byte first
  uint32_t d16, s16;
};

__device__ inline Q8_1Block quantize_block_q8_1(const float (&v)[QK]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QK; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float d = q8_1_d(amax);
  const float id = q8_1_id(d);
  int sum = 0;
  Q8_1Block b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = q8_1_code(v[4 * k + i], id);
      sum += q;
      word |= (uint32_t(q) & 0xFFu) << (8 * i);
    }
    b.q[k] = word;
  }
  b.d16 = q8_1_d16(d);
  b.s16 = q8_1_s16(d, sum);
  return b;
}

// Direct global -> LDS copies (global_load_lds_dwordx4) and their waits.
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((const lds_u8*)p));
}

// Lane i copies 16 bytes from src (its own address) to LDS byte address
// dst + 16 i (dst uniform across the wave).  Written as asm on purpose: the
// compiler tracks these transfers only coarsely and would drain every
// transfer in flight at each LDS read behind a branch, so the kernel keeps
// the vmcnt bookkeeping itself (wait_vmcnt before each barrier) and issues
// no register loads while transfers are in flight.  The asm writes no VGPR.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else in these kernels uses it
__device__ inline void dma16(const void* src, uint32_t dst) {
  // dst is wave-uniform; readfirstlane keeps it in a scalar register whatever
  // the surrounding code lets the compiler prove
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(dst)),
               "v"(src)
               : "memory", "m0");
}
// Forces a lambda's call operator inline (kernels built from many lambdas
// otherwise get some outlined as calls with stack traffic).
#define SKG_INL __attribute__((always_inline))

// The same copy addressed as a wave-uniform base (scalar register pair) plus
// a 32-bit per-lane byte offset: no per-lane 64-bit address arithmetic.
__device__ inline void dma16_sv(const void* base, uint32_t off, uint32_t dst) {
  // readfirstlane returns a signed int: widen through uint32_t, or a low
  // word >= 2^31 would sign-extend into the high word
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t sb = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b)))) |
                      (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(b >> 32)))) << 32);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(dst)),
               "v"(off), "s"(sb)
               : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read exactly once per
// launch (weights): it streams past the caches that hold what is re-read
// (measured on the LDS-ring decode kernels: 12.85 -> 12.48 us for q4_0 at
// M = 8, 17.08 -> 16.36 us for q8_0).
__device__ inline void dma16_stream(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(
                   __builtin_amdgcn_readfirstlane(dst)),
               "v"(src)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) (N <= 63), other counters untouched.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// DPP row operations (gfx9 encodings).
#define SKG_DPP_QUAD_XOR1 0xB1   // quad_perm [1,0,3,2]
#define SKG_DPP_QUAD_XOR2 0x4E   // quad_perm [2,3,0,1]
#define SKG_DPP_ROW_HALF_MIRROR 0x141
#define SKG_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave; every lane receives the same total.
// Quads first (two quad_perm swaps), then 8 and 16 lanes by mirroring, then
// the 16-lane rows by swapping across the two 32-lane halves and across rows.
__device__ inline float wave_sum(float v) {
  v += dpp_f<SKG_DPP_QUAD_XOR1>(v);
  v += dpp_f<SKG_DPP_QUAD_XOR2>(v);
  v += dpp_f<SKG_DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f<SKG_DPP_ROW_MIRROR>(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

}  // namespace skg
