// C ABI of the skinny decode GEMM / GEMV library: host-side validation,
// device check, kernel selection and launch.  Every argument is validated on
// the host before any HIP call, so every error path can be exercised without
// a GPU; nothing falls back to another code path when validation fails.
#include <atomic>
#include <climits>
#include <cerrno>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <tuple>
#include <vector>

#include "gemv_registry.h"
#include "gemv_mfma.h"
#include "gemv_mfma_pw.h"
#include "kernels.h"

using namespace skg;

namespace {

thread_local char g_err[512] = "";

skg_status fail(skg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

skg_status ok() {
  g_err[0] = '\0';
  return SKG_OK;
}

constexpr int MAX_DEV = 64;
std::atomic<int> g_dev_state[MAX_DEV];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[MAX_DEV];

skg_status check_device(int* cus = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SKG_E_DEVICE, "no HIP device (%s)", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEV) return fail(SKG_E_DEVICE, "device index %d out of range", dev);
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(SKG_E_DEVICE, "hipGetDeviceProperties failed (%s)", hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return fail(SKG_E_DEVICE, "device %d is not gfx950; this library is built for gfx950 only", dev);
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return SKG_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_gemv_fmt(int fmt) {
  return (fmt >= SKG_BF16_BF16 && fmt <= SKG_Q8_0_Q8_1) || (fmt >= SKG_Q4_K_F32 && fmt <= SKG_Q6_K_Q8_1);
}
bool is_any_fmt(int fmt) { return fmt >= SKG_BF16_BF16 && fmt <= SKG_Q6_K_BF16; }
constexpr int kNumFmts = SKG_Q6_K_BF16 + 1;

// K and N rules shared by packing and products.
skg_status check_nk(int fmt, int64_t N, int64_t K) {
  const int wk = wkind_of(fmt);
  if (wk == WK_INVALID) return fail(SKG_E_INVALID_ARG, "unknown fmt %d", fmt);
  if (N < 1) return fail(SKG_E_SHAPE, "N must be >= 1 (got %lld)", (long long)N);
  if (wk == WK_BF16) {
    if (K < 8 || K % 8) return fail(SKG_E_SHAPE, "bf16 needs K >= 8 and K %% 8 == 0 (got %lld)", (long long)K);
  } else if (wk == WK_Q4_K || wk == WK_Q6_K) {
    if (K < QK_K || K % QK_K)
      return fail(SKG_E_SHAPE, "q4_K/q6_K need K >= 256 and K %% 256 == 0 (got %lld)", (long long)K);
  } else {
    if (K < 32 || K % 32) return fail(SKG_E_SHAPE, "q8_0/q4_0 need K >= 32 and K %% 32 == 0 (got %lld)", (long long)K);
  }
  if (K > (int64_t(1) << 30) || N > INT32_MAX)
    return fail(SKG_E_SHAPE, "N=%lld K=%lld exceed the supported range", (long long)N, (long long)K);
  return SKG_OK;
}

// Packing and the block-dot hook launch one thread per block in a 1-D grid of
// 256-thread workgroups: at most 2^31 - 1 workgroups.
skg_status check_block_grid(int64_t rows, int64_t K, const char* what) {
  if (rows * (K / 32) / 256 >= INT32_MAX)
    return fail(SKG_E_SHAPE, "%s: %lld rows x K=%lld exceed one launch", what, (long long)rows, (long long)K);
  return SKG_OK;
}

// ---- GEMV variant registry ------------------------------------------------

std::once_flag g_reg_once;
std::vector<GemvEntry>* g_reg = nullptr;
std::mutex g_sel_mu;
// selected registry index per (fmt, M, epi); -1 = default (first registered)
int g_sel[kNumFmts][9][3];
std::atomic<int64_t> g_lds_pad{0};
// Set when SKG_LDS_PAD_BYTES holds something other than an integer in
// 0..kMaxLdsPad: every GEMV call is then refused until skg_set_lds_pad
// replaces the value.
constexpr int64_t kMaxLdsPad = 64 * 1024;
std::atomic<bool> g_lds_pad_env_bad{false};
char g_lds_pad_env[64] = "";

// Whole-string base-10 integer in [0, kMaxLdsPad] (leading/trailing blanks allowed).
bool parse_lds_pad(const char* s, int64_t* out) {
  if (!s) return false;
  errno = 0;
  char* end = nullptr;
  const long long v = std::strtoll(s, &end, 10);
  if (end == s || errno == ERANGE) return false;
  while (*end == ' ' || *end == '\t') ++end;
  if (*end != '\0' || v < 0 || v > kMaxLdsPad) return false;
  *out = int64_t(v);
  return true;
}

void init_registry() {
  std::call_once(g_reg_once, [] {
    auto* v = new std::vector<GemvEntry>();
    // Matrix-core defaults first (fp32 activations: M >= 2 for q4_0, M >= 4
    // for q8_0; Q8_1 activations: M = 7, 8), where they measure faster; their
    // measurement variants last.
    register_gemv_mfma_q4_0(*v);
    register_gemv_mfma_q8_0(*v);
    register_gemv_bf16(*v);
    register_gemv_q8_0_f32(*v);
    register_gemv_q8_0_f32_m38(*v);
    register_gemv_q4_0_f32(*v);
    register_gemv_q4_0_f32_m35(*v);
    register_gemv_q4_0_f32_m68(*v);
    register_gemv_mfma_q8_1(*v);
    register_gemv_q8_1(*v);
    register_gemv_mfma_q8_1_alt(*v);
    register_gemv_mfma_q4_0_alt(*v);
    register_gemv_mfma_q8_0_alt(*v);
    register_gemv_q4_K(*v);
    register_gemv_q6_K(*v);
    for (auto& a : g_sel)
      for (auto& b : a)
        for (int& c : b) c = -1;
    if (const char* e = std::getenv("SKG_LDS_PAD_BYTES")) {
      int64_t pad = 0;
      if (parse_lds_pad(e, &pad)) {
        g_lds_pad.store(pad);
      } else {
        std::snprintf(g_lds_pad_env, sizeof g_lds_pad_env, "%s", e);
        g_lds_pad_env_bad.store(true);
      }
    }
    g_reg = v;
  });
}

// The matrix-core kernels run nb / kw waves of kw blocks each; the LDS-ring
// variants (x_lds = 3, 5) are compiled for one K.
bool variant_supports(const GemvEntry& e, int64_t K) {
  const int64_t nb = K / 32;
  if (e.xlds == 3 || e.xlds == 5) return nb == e.max_nb;
  if (e.xlds == 4) return nb % PW_BPW == 0 && nb <= e.max_nb;
  if (e.xlds == 1 && e.kw > 1) {
    // every K class of the LDS-staged split walks the same number of chunks
    const int64_t nu = (e.fmt == SKG_BF16_BF16) ? K / 8 : nb;
    const int64_t chunks = (nu + 64 * e.j - 1) / (64 * e.j);
    return chunks % e.kw == 0;
  }
  if (e.xlds != 2) return true;
  return nb % e.kw == 0 && nb >= e.kw && nb <= e.max_nb;
}

// The selected variant, else the first registered one that supports K.
const GemvEntry* find_variant(int fmt, int M, int epi, int64_t K) {
  init_registry();
  int sel;
  {
    std::lock_guard<std::mutex> lk(g_sel_mu);
    sel = g_sel[fmt][M][epi];
  }
  if (sel >= 0) {
    const GemvEntry& e = (*g_reg)[size_t(sel)];
    return variant_supports(e, K) ? &e : nullptr;
  }
  for (const GemvEntry& e : *g_reg)
    if (e.fmt == fmt && e.M == M && e.epi == epi && variant_supports(e, K)) return &e;
  return nullptr;
}

// Workgroups of a persistent launch that fit on one CU at once.
int blocks_per_cu(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static std::vector<std::tuple<const void*, int, size_t, int>> cache;
  std::lock_guard<std::mutex> lk(mu);
  for (auto& c : cache)
    if (std::get<0>(c) == fn && std::get<1>(c) == threads && std::get<2>(c) == lds) return std::get<3>(c);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess || n < 1) n = 1;
  cache.emplace_back(fn, threads, lds, n);
  return n;
}

// Raises a kernel's dynamic LDS limit once per (device, kernel) instead of on
// every launch.
hipError_t ensure_dynamic_lds(const void* fn, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<std::tuple<int, const void*, size_t>> done;
  std::lock_guard<std::mutex> lk(mu);
  for (auto& d : done)
    if (std::get<0>(d) == dev && std::get<1>(d) == fn && std::get<2>(d) >= lds) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e == hipSuccess) done.emplace_back(dev, fn, lds);
  return e;
}

skg_status launch_gemv_mfma(const GemvEntry& v, int64_t K, int nseg, const int64_t* Ns, const void* W,
                            const void* x, float* const* ys, int epi, hipStream_t stream) {
  const int wk = wkind_of(v.fmt);
  MfArgs a;
  std::memset(&a, 0, sizeof a);
  a.K = K;
  a.nb = uint32_t(K / 32);
  a.x = static_cast<const float*>(x);
  const uint8_t* base = static_cast<const uint8_t*>(W);
  int64_t tiles = 0;
  if (epi == SKG_EPI_SWIGLU) {
    const Layout L = layout_of(wk, Ns[0], K);
    a.nseg = 1;
    a.seg[0].w0 = packed_view(base, L);
    a.seg[0].w1 = packed_view(base + L.total, L);
    a.seg[0].y = ys[0];
    a.seg[0].N = Ns[0];
    tiles = (Ns[0] + MF_ROWS - 1) / MF_ROWS;
  } else {
    a.nseg = nseg;
    size_t off = 0;
    for (int i = 0; i < nseg; ++i) {
      const Layout L = layout_of(wk, Ns[i], K);
      a.seg[i].w0 = packed_view(base + off, L);
      a.seg[i].w1 = a.seg[i].w0;
      a.seg[i].y = ys[i];
      a.seg[i].N = Ns[i];
      a.seg[i].tile_begin = int(tiles);
      tiles += (Ns[i] + MF_ROWS - 1) / MF_ROWS;
      off += L.total;
    }
  }
  if (tiles > 0x7FFFFFFF) return fail(SKG_E_SHAPE, "too many rows");
  a.ntiles = int(tiles);
  int cus = 0;
  skg_status st = check_device(&cus);
  if (st != SKG_OK) return st;
  const int threads = int(a.nb / uint32_t(v.kw)) * 64;
  const size_t lds = size_t(v.lds);  // dynamic LDS (the LDS-ring variant's is static)
  if (hipError_t e = ensure_dynamic_lds(v.fn, lds); e != hipSuccess)
    return fail(SKG_E_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  const int64_t resident = int64_t(cus) * blocks_per_cu(v.fn, threads, lds);
  // As many passes over the resident workgroups as the tiles need, with the
  // tiles spread evenly over them (896 tiles on 512 resident workgroups:
  // 448 workgroups of two tiles, rather than 384 of two and 128 of one).
  const int64_t passes = (tiles + resident - 1) / resident;
  int64_t grid = (tiles + passes - 1) / passes;
  if (v.xlds == 3 || v.xlds == 5) {
    // the LDS-ring kernel processes at most MF_DMA_TILES tiles per workgroup
    const int64_t need = (tiles + MF_DMA_TILES - 1) / MF_DMA_TILES;
    if (grid < need) grid = need;
  }
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(v.fn, dim3(unsigned(grid)), dim3(unsigned(threads)), args, lds, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "gemv launch: %s", hipGetErrorString(e));
  return ok();
}

// Per-wave-ring matrix-core kernel: every workgroup owns a contiguous range
// of the concatenated rows, spread over all CUs (16 .. 64 rows each).
skg_status launch_gemv_mfma_pw(const GemvEntry& v, int64_t K, int nseg, const int64_t* Ns, const void* W,
                               const void* x, float* const* ys, hipStream_t stream) {
  const int wk = wkind_of(v.fmt);
  PwArgs a;
  std::memset(&a, 0, sizeof a);
  a.K = K;
  a.nb = uint32_t(K / 32);
  a.x = static_cast<const float*>(x);
  a.nseg = nseg;
  const uint8_t* base = static_cast<const uint8_t*>(W);
  size_t off = 0;
  int64_t rows = 0;
  for (int i = 0; i < nseg; ++i) {
    const Layout L = layout_of(wk, Ns[i], K);
    a.seg[i].w = packed_view(base + off, L);
    a.seg[i].y = ys[i];
    a.seg[i].N = Ns[i];
    a.seg[i].row_begin = rows;
    rows += Ns[i];
    off += L.total;
  }
  a.ntot = rows;
  int cus = 0;
  skg_status st = check_device(&cus);
  if (st != SKG_OK) return st;
  int64_t per = (rows + cus - 1) / cus;
  per = per < 16 ? 16 : (per > 16 * PW_MAXT ? 16 * PW_MAXT : per);
  a.rows_per_wg = per;
  const int64_t grid = (rows + per - 1) / per;
  if (grid > 0x7FFFFFFF) return fail(SKG_E_SHAPE, "too many rows");
  const int waves = int(a.nb / PW_BPW);
  const size_t lds = pw_lds_bytes_of(v, waves);
  if (hipError_t e = ensure_dynamic_lds(v.fn, lds); e != hipSuccess)
    return fail(SKG_E_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(v.fn, dim3(unsigned(grid)), dim3(unsigned(waves * 64)), args, lds, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "gemv launch: %s", hipGetErrorString(e));
  return ok();
}

size_t packed_size_multi(int fmt, int n, const int64_t* Ns, int64_t K) {
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += layout_of(wkind_of(fmt), Ns[i], K).total;
  return total;
}

skg_status launch_gemv_segments(int fmt, int64_t M, int64_t K, int nseg, const int64_t* Ns, const void* W,
                                const void* x, float* const* ys, int epi, hipStream_t stream) {
  const GemvEntry* v = find_variant(fmt, int(M), epi, K);
  if (!v)
    return fail(SKG_E_UNSUPPORTED, "no compiled kernel (or the selected variant does not take K=%lld) for fmt=%d "
                "M=%lld epi=%d", (long long)K, fmt, (long long)M, epi);
  if (v->xlds == 2 || v->xlds == 3 || v->xlds == 5) return launch_gemv_mfma(*v, K, nseg, Ns, W, x, ys, epi, stream);
  if (v->xlds == 4) return launch_gemv_mfma_pw(*v, K, nseg, Ns, W, x, ys, stream);
  const int wk = wkind_of(fmt);
  GemvArgs a;
  std::memset(&a, 0, sizeof a);
  a.K = K;
  a.nu = uint32_t(wk == WK_BF16 ? K / 8 : K / 32);
  a.x = static_cast<const uint8_t*>(x);
  const int rows_per_block = (v->waves / v->kw) * v->ro;
  if (rows_per_block <= 0) return fail(SKG_E_UNSUPPORTED, "variant with x_lds=%d has no VALU row layout", v->xlds);
  int64_t blocks = 0;
  const uint8_t* base = static_cast<const uint8_t*>(W);
  if (epi == SKG_EPI_SWIGLU_Q8_1 && rows_per_block % 32 != 0)
    return fail(SKG_E_UNSUPPORTED, "selected variant covers %d rows per workgroup; the Q8_1 epilogue needs whole "
                "32-row blocks", rows_per_block);
  if (epi != SKG_EPI_NONE) {
    const Layout L = layout_of(wk, Ns[0], K);
    a.nseg = 1;
    a.seg[0].w0 = packed_view(base, L);
    a.seg[0].w1 = packed_view(base + L.total, L);
    a.seg[0].y = ys[0];
    a.seg[0].yq = (epi == SKG_EPI_SWIGLU_Q8_1) ? reinterpret_cast<uint8_t*>(ys[1]) : nullptr;
    a.seg[0].N = Ns[0];
    a.seg[0].blk_begin = 0;
    blocks = (Ns[0] + rows_per_block - 1) / rows_per_block;
  } else {
    a.nseg = nseg;
    size_t off = 0;
    for (int i = 0; i < nseg; ++i) {
      const Layout L = layout_of(wk, Ns[i], K);
      a.seg[i].w0 = packed_view(base + off, L);
      a.seg[i].w1 = a.seg[i].w0;
      a.seg[i].y = ys[i];
      a.seg[i].N = Ns[i];
      a.seg[i].blk_begin = int(blocks);
      blocks += (Ns[i] + rows_per_block - 1) / rows_per_block;
      off += L.total;
    }
  }
  if (blocks > 0x7FFFFFFF) return fail(SKG_E_SHAPE, "too many rows");
  size_t lds = gemv_lds_bytes(fmt, int(M), v->j, v->xlds, v->xlds ? v->kw : 1) + size_t(g_lds_pad.load());
  if (lds > 160 * 1024) return fail(SKG_E_UNSUPPORTED, "variant needs %zu bytes of LDS", lds);
  if (hipError_t e = ensure_dynamic_lds(v->fn, lds); e != hipSuccess)
    return fail(SKG_E_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(v->fn, dim3(unsigned(blocks)), dim3(unsigned(v->waves * 64)), args, lds, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "gemv launch: %s", hipGetErrorString(e));
  return ok();
}

skg_status check_gemv_common(int fmt, int64_t M, int64_t K, const void* W, const void* x) {
  if (!is_gemv_fmt(fmt)) {
    if (is_any_fmt(fmt)) return fail(SKG_E_UNSUPPORTED, "fmt %d is not a gemv format (use skg_gemm_tiled)", fmt);
    return fail(SKG_E_INVALID_ARG, "unknown fmt %d", fmt);
  }
  if (M < 1 || M > 8) return fail(SKG_E_SHAPE, "gemv needs 1 <= M <= 8 (got %lld)", (long long)M);
  init_registry();
  if (g_lds_pad_env_bad.load())
    return fail(SKG_E_INVALID_ARG, "SKG_LDS_PAD_BYTES='%s' is not an integer in 0..%lld", g_lds_pad_env,
                (long long)kMaxLdsPad);
  if (!W || !x) return fail(SKG_E_INVALID_ARG, "null W or x");
  if (!aligned(W, 16)) return fail(SKG_E_ALIGN, "W must be 16-byte aligned");
  const bool q8 = (fmt == SKG_Q4_0_Q8_1 || fmt == SKG_Q8_0_Q8_1 || fmt == SKG_Q4_K_Q8_1 || fmt == SKG_Q6_K_Q8_1);
  if (!aligned(x, q8 ? 4 : 16)) return fail(SKG_E_ALIGN, "x must be %d-byte aligned", q8 ? 4 : 16);
  (void)K;
  return SKG_OK;
}

}  // namespace

extern "C" {

int skg_abi_version(void) { return SKG_ABI_VERSION; }

const char* skg_status_str(int status) {
  switch (status) {
    case SKG_OK: return "SKG_OK";
    case SKG_E_INVALID_ARG: return "SKG_E_INVALID_ARG";
    case SKG_E_SHAPE: return "SKG_E_SHAPE";
    case SKG_E_ALIGN: return "SKG_E_ALIGN";
    case SKG_E_UNSUPPORTED: return "SKG_E_UNSUPPORTED";
    case SKG_E_DEVICE: return "SKG_E_DEVICE";
    case SKG_E_HIP: return "SKG_E_HIP";
    default: return "SKG_E_UNKNOWN";
  }
}

const char* skg_last_error(void) { return g_err; }

size_t skg_packed_size(skg_fmt fmt, int64_t N, int64_t K) {
  if (check_nk(fmt, N, K) != SKG_OK) return 0;
  return layout_of(wkind_of(fmt), N, K).total;
}

size_t skg_packed_size_multi(skg_fmt fmt, int n, const int64_t* Ns, int64_t K) {
  if (n < 1 || n > MAX_SEGS || !Ns) return 0;
  for (int i = 0; i < n; ++i)
    if (check_nk(fmt, Ns[i], K) != SKG_OK) return 0;
  return packed_size_multi(fmt, n, Ns, K);
}

skg_status skg_pack_weights(skg_fmt fmt, int64_t N, int64_t K, const void* src, void* dst, hipStream_t stream) {
  skg_status st = check_nk(fmt, N, K);
  if (st != SKG_OK) return st;
  if ((st = check_block_grid(N, K, "pack")) != SKG_OK) return st;
  if (!src || !dst) return fail(SKG_E_INVALID_ARG, "null src or dst");
  if (!aligned(src, 2)) return fail(SKG_E_ALIGN, "src must be 2-byte aligned");
  if (!aligned(dst, 16)) return fail(SKG_E_ALIGN, "dst must be 16-byte aligned");
  if ((st = check_device()) != SKG_OK) return st;
  hipError_t e = launch_pack(wkind_of(fmt), N, K, src, dst, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "pack: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_pack_weights_multi(skg_fmt fmt, int n, const int64_t* Ns, int64_t K, const void* const* srcs,
                                  void* dst, hipStream_t stream) {
  if (n < 1 || n > MAX_SEGS) return fail(SKG_E_INVALID_ARG, "n must be 1..%d (got %d)", MAX_SEGS, n);
  if (!Ns || !srcs || !dst) return fail(SKG_E_INVALID_ARG, "null Ns, srcs or dst");
  for (int i = 0; i < n; ++i) {
    skg_status st = check_nk(fmt, Ns[i], K);
    if (st != SKG_OK) return st;
    if ((st = check_block_grid(Ns[i], K, "pack")) != SKG_OK) return st;
    if (!srcs[i]) return fail(SKG_E_INVALID_ARG, "null srcs[%d]", i);
    if (!aligned(srcs[i], 2)) return fail(SKG_E_ALIGN, "srcs[%d] must be 2-byte aligned", i);
  }
  if (!aligned(dst, 16)) return fail(SKG_E_ALIGN, "dst must be 16-byte aligned");
  skg_status st = check_device();
  if (st != SKG_OK) return st;
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    hipError_t e = launch_pack(wkind_of(fmt), Ns[i], K, srcs[i], static_cast<uint8_t*>(dst) + off, stream);
    if (e != hipSuccess) return fail(SKG_E_HIP, "pack: %s", hipGetErrorString(e));
    off += layout_of(wkind_of(fmt), Ns[i], K).total;
  }
  return ok();
}

skg_status skg_quantize_act_q8_1(int64_t M, int64_t K, const float* x, void* xq, hipStream_t stream) {
  if (M < 1) return fail(SKG_E_SHAPE, "M must be >= 1 (got %lld)", (long long)M);
  if (K < 32 || K % 32) return fail(SKG_E_SHAPE, "K must be >= 32 and a multiple of 32 (got %lld)", (long long)K);
  if (M * (K / 32) > (int64_t(1) << 36)) return fail(SKG_E_SHAPE, "too many blocks");
  if (!x || !xq) return fail(SKG_E_INVALID_ARG, "null x or xq");
  if (!aligned(x, 16)) return fail(SKG_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(xq, 4)) return fail(SKG_E_ALIGN, "xq must be 4-byte aligned");
  skg_status st = check_device();
  if (st != SKG_OK) return st;
  hipError_t e = launch_quantize_q8_1(M, K, x, xq, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "quantize: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_rmsnorm_q8_1(int64_t M, int64_t K, const float* x, const float* g, float eps, float* xn, void* xq,
                            hipStream_t stream) {
  if (M < 1 || M > kNormMaxM) return fail(SKG_E_SHAPE, "M must be in [1, %lld] (got %lld)", (long long)kNormMaxM, (long long)M);
  if (K < 32 || K % 32 || K > kNormMaxK)
    return fail(SKG_E_SHAPE, "K must be a multiple of 32 in [32, %lld] (got %lld)", (long long)kNormMaxK, (long long)K);
  if (!x) return fail(SKG_E_INVALID_ARG, "null x");
  if (!xn && !xq) return fail(SKG_E_INVALID_ARG, "at least one of xn and xq must be given");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(SKG_E_INVALID_ARG, "eps must be finite and >= 0");
  if (!aligned(x, 16) || (g && !aligned(g, 16)) || (xn && !aligned(xn, 16)))
    return fail(SKG_E_ALIGN, "x, g and xn must be 16-byte aligned");
  if (xq && !aligned(xq, 4)) return fail(SKG_E_ALIGN, "xq must be 4-byte aligned");
  skg_status st = check_device();
  if (st != SKG_OK) return st;
  hipError_t e = launch_rmsnorm_q8_1(M, K, x, g, eps, xn, xq, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "rmsnorm: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_gemv(skg_fmt fmt, int64_t M, int64_t K, int64_t N, const void* W, const void* x, float* y,
                    hipStream_t stream) {
  skg_status st = check_gemv_common(fmt, M, K, W, x);
  if (st != SKG_OK) return st;
  if ((st = check_nk(fmt, N, K)) != SKG_OK) return st;
  if (!y) return fail(SKG_E_INVALID_ARG, "null y");
  if (!aligned(y, 4)) return fail(SKG_E_ALIGN, "y must be 4-byte aligned");
  if ((st = check_device()) != SKG_OK) return st;
  return launch_gemv_segments(fmt, M, K, 1, &N, W, x, &y, SKG_EPI_NONE, stream);
}

skg_status skg_gemv_multi(skg_fmt fmt, int64_t M, int64_t K, int n, const int64_t* Ns, const void* W,
                          const void* x, float* const* ys, skg_epi epi, hipStream_t stream) {
  skg_status st = check_gemv_common(fmt, M, K, W, x);
  if (st != SKG_OK) return st;
  if (!Ns || !ys) return fail(SKG_E_INVALID_ARG, "null Ns or ys");
  if (epi == SKG_EPI_NONE) {
    if (n < 1 || n > MAX_SEGS) return fail(SKG_E_INVALID_ARG, "n must be 1..%d (got %d)", MAX_SEGS, n);
  } else if (epi == SKG_EPI_SWIGLU || epi == SKG_EPI_SWIGLU_Q8_1) {
    if (n != 2) return fail(SKG_E_INVALID_ARG, "SwiGLU needs n == 2 (gate, up), got %d", n);
    if (Ns[0] != Ns[1]) return fail(SKG_E_SHAPE, "SwiGLU needs Ns[0] == Ns[1]");
    if (epi == SKG_EPI_SWIGLU_Q8_1) {
      if (fmt != SKG_Q4_0_Q8_1 && fmt != SKG_Q8_0_Q8_1)
        return fail(SKG_E_UNSUPPORTED, "the Q8_1 SwiGLU epilogue exists for SKG_Q4_0_Q8_1 and SKG_Q8_0_Q8_1");
      if (Ns[0] % 32) return fail(SKG_E_SHAPE, "the Q8_1 SwiGLU epilogue needs Ns[0] %% 32 == 0");
    }
  } else {
    return fail(SKG_E_INVALID_ARG, "unknown epilogue %d", int(epi));
  }
  for (int i = 0; i < n; ++i)
    if ((st = check_nk(fmt, Ns[i], K)) != SKG_OK) return st;
  const int nout = (epi == SKG_EPI_SWIGLU) ? 1 : (epi == SKG_EPI_SWIGLU_Q8_1) ? 2 : n;
  for (int i = 0; i < nout; ++i) {
    if (!ys[i]) return fail(SKG_E_INVALID_ARG, "null ys[%d]", i);
    if (!aligned(ys[i], 4)) return fail(SKG_E_ALIGN, "ys[%d] must be 4-byte aligned", i);
  }
  if ((st = check_device()) != SKG_OK) return st;
  return launch_gemv_segments(fmt, M, K, n, Ns, W, x, ys, epi, stream);
}

skg_status skg_gemm_tiled(skg_fmt fmt, int64_t M, int64_t K, int64_t N, const void* W, const void* x, float* y,
                          hipStream_t stream) {
  if (!is_any_fmt(fmt)) return fail(SKG_E_INVALID_ARG, "unknown fmt %d", int(fmt));
  if (fmt == SKG_Q4_0_Q8_1 || fmt == SKG_Q8_0_Q8_1) {
    // integer matrix-core tile: Q8_1 activation blocks
    skg_status st = check_nk(fmt, N, K);
    if (st != SKG_OK) return st;
    if (K % 64) return fail(SKG_E_SHAPE, "the Q8_1 tile needs K %% 64 == 0 (got %lld)", (long long)K);
    if (M < 1 || M > INT32_MAX) return fail(SKG_E_SHAPE, "M must be in [1, 2^31 - 1] (got %lld)", (long long)M);
    if (((M + 255) / 256) * ((N + 63) / 64) > INT32_MAX)
      return fail(SKG_E_SHAPE, "M=%lld x N=%lld needs more output tiles than one launch takes", (long long)M,
                  (long long)N);
    if (!W || !x || !y) return fail(SKG_E_INVALID_ARG, "null W, x or y");
    if (!aligned(W, 16)) return fail(SKG_E_ALIGN, "W must be 16-byte aligned");
    if (!aligned(x, 4) || !aligned(y, 4)) return fail(SKG_E_ALIGN, "x and y must be 4-byte aligned");
    if ((st = check_device()) != SKG_OK) return st;
    hipError_t e = launch_gemm_i8(M, K, N, W, layout_of(wkind_of(fmt), N, K), x, y, stream);
    if (e != hipSuccess) return fail(SKG_E_HIP, "gemm_tiled: %s", hipGetErrorString(e));
    return ok();
  }
  if (fmt != SKG_Q4_0_BF16 && fmt != SKG_Q8_0_BF16 && fmt != SKG_Q4_K_BF16 && fmt != SKG_Q6_K_BF16)
    return fail(SKG_E_UNSUPPORTED, "gemm_tiled supports SKG_Q4_0_BF16, SKG_Q8_0_BF16, SKG_Q4_K_BF16, SKG_Q6_K_BF16, "
                "SKG_Q4_0_Q8_1 and SKG_Q8_0_Q8_1");
  const int variant = g_gemm_variant.load(std::memory_order_relaxed);
  if (fmt != SKG_Q4_0_BF16 && variant != 3 && variant != 4)
    return fail(SKG_E_UNSUPPORTED, "q8_0, q4_K and q6_K tiles run on prefill organisations 3 and 4 (selected: %d)",
                variant);
  skg_status st = check_nk(fmt, N, K);
  if (st != SKG_OK) return st;
  if (M < 1 || M > INT32_MAX) return fail(SKG_E_SHAPE, "M must be in [1, 2^31 - 1] (got %lld)", (long long)M);
  // one workgroup per 256 x 112 (or 256 x 128) output tile, in a 1-D grid
  if (((M + 255) / 256) * ((N + 111) / 112) > INT32_MAX)
    return fail(SKG_E_SHAPE, "M=%lld x N=%lld needs more output tiles than one launch takes", (long long)M,
                (long long)N);
  if (!W || !x || !y) return fail(SKG_E_INVALID_ARG, "null W, x or y");
  if (!aligned(W, 16) || !aligned(x, 16)) return fail(SKG_E_ALIGN, "W and x must be 16-byte aligned");
  if (!aligned(y, 4)) return fail(SKG_E_ALIGN, "y must be 4-byte aligned");
  if ((st = check_device()) != SKG_OK) return st;
  const Layout L = layout_of(wkind_of(fmt), N, K);
  hipError_t e = launch_gemm_tiled(M, K, N, W, L, x, y, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "gemm_tiled: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_debug_block_dots(skg_fmt fmt, int64_t N, int64_t K, int64_t n0, int64_t nr, const void* W,
                                const void* xq, int32_t* out, hipStream_t stream) {
  if (fmt != SKG_Q4_0_Q8_1 && fmt != SKG_Q8_0_Q8_1) {
    if (is_any_fmt(fmt)) return fail(SKG_E_UNSUPPORTED, "block dots exist for the Q8_1 formats only");
    return fail(SKG_E_INVALID_ARG, "unknown fmt %d", int(fmt));
  }
  skg_status st = check_nk(fmt, N, K);
  if (st != SKG_OK) return st;
  if (n0 < 0 || nr < 1 || n0 + nr > N) return fail(SKG_E_SHAPE, "rows [n0, n0+nr) must lie in [0, N)");
  if ((st = check_block_grid(nr, K, "block dots")) != SKG_OK) return st;
  if (!W || !xq || !out) return fail(SKG_E_INVALID_ARG, "null W, xq or out");
  if (!aligned(W, 16) || !aligned(xq, 4) || !aligned(out, 4)) return fail(SKG_E_ALIGN, "misaligned pointer");
  if ((st = check_device()) != SKG_OK) return st;
  hipError_t e = launch_block_dots(fmt, W, layout_of(wkind_of(fmt), N, K), n0, nr, xq, out, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "block dots: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream) {
  if (!buf || !out) return fail(SKG_E_INVALID_ARG, "null buf or out");
  if (bytes == 0 || bytes % 16) return fail(SKG_E_SHAPE, "bytes must be a positive multiple of 16");
  if (bytes / 4096 >= INT32_MAX) return fail(SKG_E_SHAPE, "bytes exceed one launch (4 KB per workgroup)");
  if (!aligned(buf, 16) || !aligned(out, 4)) return fail(SKG_E_ALIGN, "buf must be 16-byte aligned");
  int cus = 0;
  skg_status st = check_device(&cus);
  if (st != SKG_OK) return st;
  hipError_t e = launch_stream_read(buf, bytes, out, cus * 8, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "stream read: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_empty_launch(int64_t grid, int block, hipStream_t stream) {
  if (grid < 1 || grid > INT32_MAX) return fail(SKG_E_SHAPE, "grid must be 1..2^31-1 (got %lld)", (long long)grid);
  if (block < 64 || block > 1024 || block % 64)
    return fail(SKG_E_SHAPE, "block must be a multiple of 64 in 64..1024 (got %d)", block);
  skg_status st = check_device();
  if (st != SKG_OK) return st;
  hipError_t e = launch_empty(grid, block, stream);
  if (e != hipSuccess) return fail(SKG_E_HIP, "empty launch: %s", hipGetErrorString(e));
  return ok();
}

skg_status skg_gemv_default_variant(skg_fmt fmt, int M, skg_epi epi, int64_t K, int* out) {
  if (!is_gemv_fmt(fmt)) return fail(SKG_E_INVALID_ARG, "unknown gemv fmt %d", int(fmt));
  if (M < 1 || M > 8) return fail(SKG_E_SHAPE, "M must be 1..8");
  if (epi != SKG_EPI_NONE && epi != SKG_EPI_SWIGLU && epi != SKG_EPI_SWIGLU_Q8_1)
    return fail(SKG_E_INVALID_ARG, "unknown epilogue");
  if (!out) return fail(SKG_E_INVALID_ARG, "null out");
  const GemvEntry* e = find_variant(fmt, M, epi, K);
  if (!e) return fail(SKG_E_UNSUPPORTED, "no compiled variant takes K=%lld", (long long)K);
  const int rec[SKG_VARIANT_FIELDS] = {e->fmt, e->M, e->epi, e->ro, e->j, e->xlds, e->waves, e->kw, e->depth};
  for (int i = 0; i < SKG_VARIANT_FIELDS; ++i) out[i] = rec[i];
  return ok();
}

skg_status skg_gemv_set_variant(skg_fmt fmt, int M, skg_epi epi, int ro, int j, int x_lds, int waves, int kw,
                                int depth) {
  if (!is_gemv_fmt(fmt)) return fail(SKG_E_INVALID_ARG, "unknown gemv fmt %d", int(fmt));
  if (M < 1 || M > 8) return fail(SKG_E_SHAPE, "M must be 1..8");
  if (epi != SKG_EPI_NONE && epi != SKG_EPI_SWIGLU && epi != SKG_EPI_SWIGLU_Q8_1)
    return fail(SKG_E_INVALID_ARG, "unknown epilogue");
  init_registry();
  int idx = -1;
  if (ro != 0) {
    for (size_t i = 0; i < g_reg->size(); ++i) {
      const GemvEntry& e = (*g_reg)[i];
      if (e.fmt == fmt && e.M == M && e.epi == epi && e.ro == ro && e.j == j && e.xlds == x_lds && e.waves == waves &&
          e.kw == kw && (depth == 0 || e.depth == depth)) {
        idx = int(i);
        break;
      }
    }
    if (idx < 0)
      return fail(SKG_E_UNSUPPORTED, "no compiled variant ro=%d j=%d x_lds=%d waves=%d kw=%d depth=%d", ro, j, x_lds,
                  waves, kw, depth);
  }
  std::lock_guard<std::mutex> lk(g_sel_mu);
  g_sel[fmt][M][epi] = idx;
  return ok();
}

int skg_gemv_variants(int* out, int max_entries) {
  init_registry();
  const int n = int(g_reg->size());
  if (out) {
    for (int i = 0; i < n && i < max_entries; ++i) {
      const GemvEntry& e = (*g_reg)[size_t(i)];
      int* o = out + SKG_VARIANT_FIELDS * i;
      o[0] = e.fmt;
      o[1] = e.M;
      o[2] = e.epi;
      o[3] = e.ro;
      o[4] = e.j;
      o[5] = e.xlds;
      o[6] = e.waves;
      o[7] = e.kw;
      o[8] = e.depth;
    }
  }
  return n;
}

skg_status skg_gemm_tiled_set_variant(int variant) {
  if (variant < -1 || variant > 4) return fail(SKG_E_INVALID_ARG, "prefill variant must be -1..4");
  g_gemm_variant.store(variant < 0 ? kGemmDefaultVariant : variant, std::memory_order_relaxed);
  return ok();
}

skg_status skg_set_lds_pad(int64_t bytes) {
  if (bytes < 0 || bytes > kMaxLdsPad) return fail(SKG_E_INVALID_ARG, "LDS pad must be 0..65536 bytes");
  init_registry();
  g_lds_pad.store(bytes);
  g_lds_pad_env_bad.store(false);
  return ok();
}

}  // extern "C"
