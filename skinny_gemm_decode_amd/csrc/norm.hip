// RMSNorm with a per-channel gain and, in the same pass, the Q8_1 encoding of
// its output.
//
// The RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach &
// Methodology) lets the RMSNorm-plus-scale dispatch in front of a Q4_0 matvec
// write that matvec's Q8_1 activation itself, which removes the standalone
// quantisation dispatch; "Six hypotheses, four refutations" (Hypothesis
// ledger: fewer, longer kernels) books the same fusion as one launch saved per
// layer.  Per row of K values:
//   ss = sum_k x_k^2,  r = 1 / sqrt(ss / K + eps),  xn_k = (x_k * r) * g_k
// in binary32, then the Q8_1 quantiser of the standalone dispatch applied to
// xn (same per-block steps, so xq is exactly quantize_act_q8_1(xn)).
//
// Layout: a row is split into slices of 1024 elements (32 Q8_1 blocks), one
// workgroup of 256 threads per slice, each thread holding 4 consecutive
// elements per 1024-element chunk (16-byte loads).  Every workgroup of a row
// reads the whole row and forms the sum of squares with the same code in the
// same order (per thread, across the wave, then the 4 wave totals in index
// order), so all of them hold the same r, bit for bit, and every call gives
// the same bits; each then scales, quantises and stores only its own slice.
// The redundant reads of x are cheap (the row is 16-44 KB and the copies meet
// in L2), while spreading one row over several CUs puts more of its loads in
// flight at once: at M = 1, K = 4096 one 1024-thread workgroup per row took
// 4.3 us per graph-replayed launch, four 256-thread workgroups 2.3 us.
//
// Q8_1 blocks are quantised by 8-lane groups: lane j of an aligned group of 8
// holds elements 4j .. 4j+3 of one block, and the group's max and integer sum
// (exact, order-free) feed the shared per-block steps.
#include "gemv_impl.h"
#include "kernels.h"

#include <array>
#include <utility>

namespace skg {

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / 64;
constexpr int kNormSlice = 4 * kNormThreads;  // elements per workgroup

__device__ inline float oct_max(float v) {
  v = fmaxf(v, dpp_f<SKG_DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<SKG_DPP_QUAD_XOR2>(v));
  return fmaxf(v, dpp_f<SKG_DPP_ROW_HALF_MIRROR>(v));
}
__device__ inline int oct_sum(int v) {
  v += dpp_i<SKG_DPP_QUAD_XOR1>(v);
  v += dpp_i<SKG_DPP_QUAD_XOR2>(v);
  return v + dpp_i<SKG_DPP_ROW_HALF_MIRROR>(v);
}

// One Q8_1 block from the 8 lanes of an aligned group (lane j holds y = the
// block's elements 4j .. 4j+3), written to dst (36 bytes, 4-byte aligned)
// when `store`.  Every lane of the group must execute it.
__device__ inline void quantise_oct_q8_1(const float (&y)[4], uint8_t* dst, bool store) {
  const uint32_t j = threadIdx.x & 7;
  const float am = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
  const float d = q8_1_d(oct_max(am));
  const float id = q8_1_id(d);
  int s = 0;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = q8_1_code(y[i], id);
    s += q;
    word |= (uint32_t(q) & 0xFFu) << (8 * i);
  }
  const int sum = oct_sum(s);
  if (store) {
    uint32_t* w = reinterpret_cast<uint32_t*>(dst);
    w[1 + j] = word;
    if (j == 0) w[0] = q8_1_d16(d) | (q8_1_s16(d, sum) << 16);
  }
}

// NCH = slices per row (= workgroups per row).
template <int NCH>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_q8_1_kernel(const float* __restrict__ x,
                                                                    const float* __restrict__ g, float eps,
                                                                    int K, float* __restrict__ xn,
                                                                    uint8_t* __restrict__ xq) {
  __shared__ float part[kNormWaves];
  const int t = threadIdx.x;
  const size_t row = blockIdx.x / NCH;
  const int own = blockIdx.x % NCH;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * size_t(K));
  const int K4 = K / 4;
  const int io = own * kNormThreads + t;  // this thread's 4-element unit of the own slice
  // K % 32 == 0, so `ok` is uniform over each 8-lane block group.
  const bool ok = io < K4;

  // All loads first, so their latencies overlap.
  f32x4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = c * kNormThreads + t;
    v[c] = i < K4 ? xr[i] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f32x4 gv = (ok && g) ? reinterpret_cast<const f32x4*>(g)[io] : f32x4{1.f, 1.f, 1.f, 1.f};

  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    ss = fmaf(v[c].x, v[c].x, ss);
    ss = fmaf(v[c].y, v[c].y, ss);
    ss = fmaf(v[c].z, v[c].z, ss);
    ss = fmaf(v[c].w, v[c].w, ss);
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormWaves; ++w) tot += part[w];

  float r;
  {
#pragma clang fp contract(off)
    r = 1.0f / sqrtf(tot / float(K) + eps);
  }

  f32x4 xo = v[0];
#pragma unroll
  for (int c = 1; c < NCH; ++c)
    if (c == own) xo = v[c];
  float y[4];
  {
#pragma clang fp contract(off)
    y[0] = (xo.x * r) * gv.x;
    y[1] = (xo.y * r) * gv.y;
    y[2] = (xo.z * r) * gv.z;
    y[3] = (xo.w * r) * gv.w;
  }
  if (xn && ok) reinterpret_cast<f32x4*>(xn + row * size_t(K))[io] = f32x4{y[0], y[1], y[2], y[3]};
  if (xq) quantise_oct_q8_1(y, xq + (row * size_t(K / QK) + size_t(ok ? (4 * io) / QK : 0)) * 36, ok);
}

namespace {

using NormFn = void (*)(const float*, const float*, float, int, float*, uint8_t*);

template <int... I>
constexpr auto norm_table(std::integer_sequence<int, I...>) {
  return std::array<NormFn, sizeof...(I)>{&rmsnorm_q8_1_kernel<I + 1>...};
}

constexpr auto kNormKernels = norm_table(std::make_integer_sequence<int, kNormMaxK / kNormSlice>{});

}  // namespace

hipError_t launch_rmsnorm_q8_1(int64_t M, int64_t K, const float* x, const float* g, float eps, float* xn,
                               void* xq, hipStream_t stream) {
  const int64_t nch = (K + kNormSlice - 1) / kNormSlice;
  if (nch < 1 || nch > int64_t(kNormKernels.size()) || M < 1 || M * nch > int64_t(0x7FFFFFFF))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(kNormKernels[size_t(nch - 1)], dim3(unsigned(M * nch)), dim3(kNormThreads), 0, stream, x, g,
                     eps, int(K), xn, static_cast<uint8_t*>(xq));
  return hipGetLastError();
}

}  // namespace skg
