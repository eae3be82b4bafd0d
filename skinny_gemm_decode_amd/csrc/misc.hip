// Test and measurement kernels: integer block dots through the GEMV's own
// device functions, the streaming-read bandwidth ceiling and the empty kernel
// that measures the launch floor.
#include "gemv_impl.h"
#include "kernels.h"

namespace skg {

// out[r][b] = integer block dot of row n0 + r, block b, against xq (one row).
template <int FMT>
__global__ void block_dots_kernel(PackedW P, int64_t n0, int64_t nr, const uint8_t* __restrict__ xq,
                                  int32_t* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nb = P.nb;
  if (i >= nr * nb) return;
  const int64_t r = i / nb;
  const uint32_t b = uint32_t(i % nb);
  const int64_t n = n0 + r;
  WUnit<FMT> w;
  load_w<FMT>(w, P.payload + size_t(n) * P.row_bytes, P.scales + size_t(n) * nb, P.nb, b);
  XUnit<FMT> x;
  fetch_x_global<FMT>(x, xq, 0, P.nb, 0, b);
  out[i] = unit_idot<FMT>(w, x);
}

hipError_t launch_block_dots(int fmt, const void* W, const Layout& L, int64_t n0, int64_t nr, const void* xq,
                             int32_t* out, hipStream_t stream) {
  const PackedW P = packed_view(W, L);
  const int64_t total = nr * L.nb;
  const int threads = 256;
  const unsigned grid = unsigned((total + threads - 1) / threads);
  if (fmt == SKG_Q4_0_Q8_1)
    hipLaunchKernelGGL(block_dots_kernel<SKG_Q4_0_Q8_1>, dim3(grid), dim3(threads), 0, stream, P, n0, nr,
                       static_cast<const uint8_t*>(xq), out);
  else
    hipLaunchKernelGGL(block_dots_kernel<SKG_Q8_0_Q8_1>, dim3(grid), dim3(threads), 0, stream, P, n0, nr,
                       static_cast<const uint8_t*>(xq), out);
  return hipGetLastError();
}

// Streaming read: one non-temporal 16-byte load per thread, 4 KB per
// workgroup, as many workgroups as the buffer needs.  Of the read shapes
// measured on MI355X (grid-stride loops with 1-8 loads in flight per thread,
// per-workgroup chunks of 4-16 KB) this is the fastest at 33 MB to 1 GB.  The
// words are folded into a hash that is stored only if it equals a sentinel the
// host passes, so the loads stay live and almost nothing is written.  "Six
// hypotheses, four refutations" (What the failure left behind) uses such a
// trivially parallel kernel as the achievable-bandwidth reference.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t nwords,
                                                          uint32_t sentinel, uint32_t* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const u32x4 a = __builtin_nontemporal_load(buf + i);
  const uint32_t h = (a.x + a.y) ^ (a.z + a.w);
  if (h == sentinel) out[0] = h;  // practically never; the compiler cannot prove it
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, hipStream_t stream) {
  (void)grid;
  const int64_t nwords = int64_t(bytes / 16);
  const int64_t blocks = (nwords + 255) / 256;
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), nwords, 0x9E3779B9u, out);
  return hipGetLastError();
}

// Does nothing: back-to-back launches of it time the fixed cost of a launch.
__global__ void empty_kernel() {}

hipError_t launch_empty(int64_t grid, int block, hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(unsigned(grid)), dim3(unsigned(block)), 0, stream);
  return hipGetLastError();
}

}  // namespace skg
