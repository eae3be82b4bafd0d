/*
 * skg.h - C ABI of the MI355X (gfx950) skinny decode GEMM / GEMV library.
 *
 * The library computes the weight x activation products of LLM token decode:
 * y[m][n] = sum_k W[n][k] * x[m][k] for M = 1..8 activation rows against an
 * N x K weight matrix, plus the M = 512 tiled prefill product.
 *
 *   "The Shape That Actually Matters" (amarbaro.com), The shape a decode step
 *   actually runs: one activation row times every weight matrix, the skinny
 *   M=1, K=4096, N=12288 shape, bound by streaming the weights from HBM.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Orientation: W is N x K, row-major, K contiguous; y = W x.  x is M x K
 * row-major; y is M x N row-major float32 and is overwritten (no accumulate).
 *
 * Canonical formats (32-element blocks along K, little-endian):
 *   bf16  : uint16 bit patterns (upper half of a binary32).
 *   q8_0  : 34-byte block {fp16 d; int8 q[32]},              w_i = d * q_i.
 *   q4_0  : 18-byte block {fp16 d; uint8 qs[16]},            w_i = d * (c_i - 8),
 *           c_i = low nibble of qs[i] for i < 16, high nibble of qs[i-16] else.
 *   Q8_1  : 36-byte block {fp16 d; fp16 s; int8 q[32]},      a_i = d * q_i,
 *           s = fp16(d_f32 * sum_i q_i).
 * K-quant super-blocks (256 elements along K): "Chapter 2.2 - speed - 64-lane
 * Metal" (In twenty seconds - The fix) runs q4_K and q6_K weights without
 * defining them; these are the GGUF super-block layouts such files carry.
 *   q4_K  : 144 bytes {fp16 d; fp16 dmin; uint8 s[12]; uint8 qs[128]}: eight
 *           6-bit scales sc_j and mins m_j (j < 4: sc_j = s[j] & 63,
 *           m_j = s[j+4] & 63; j >= 4: sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
 *           m_j = (s[j+4] >> 4) | (s[j] >> 6) << 4); element 64c + i (i < 32)
 *           is the low nibble of qs[32c + i], element 64c + 32 + i its high
 *           nibble; w = d * sc_j * q - dmin * m_j for element e in j = e / 32.
 *   q6_K  : 210 bytes {uint8 ql[128]; uint8 qh[64]; int8 sc[16]; fp16 d}:
 *           element e, h = e / 128, r = e % 128, g = r / 32, l = r % 32, takes
 *           nibble (g >> 1) of ql[64h + 32(g & 1) + l] and bits 2g, 2g+1 of
 *           qh[32h + l] as its high two bits: q in 0..63,
 *           w = d * sc[e / 16] * (q - 32).
 *
 * Memory: every pointer argument named W/x/y/xq/src/dst/buf/out is a DEVICE
 * pointer on the current HIP device; pointer arrays (Ns, srcs, ys) are HOST
 * arrays.  The caller owns every buffer.  The library never allocates or frees
 * memory and keeps no pointer after a call returns.
 *
 * Asynchrony: every call validates its arguments synchronously on the host
 * (before any HIP call), then only enqueues kernels on `stream` (NULL = the
 * device's null stream) and returns.  It never synchronizes.  Results are
 * visible after the stream is synchronized.
 *
 * Errors: a nonzero skg_status means nothing was enqueued (except SKG_E_HIP,
 * a launch failure).  skg_last_error() returns a thread-local message for the
 * last failing call on the calling thread.  Nothing is silently demoted to
 * another code path: invalid arguments and unsupported devices are rejected,
 * as the RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach &
 * Methodology) requires of its shape-specific routes.
 *
 * Devices: the kernels are built for gfx950 only; on any other device every
 * compute entry point returns SKG_E_DEVICE.
 *
 * Thread safety: all entry points are reentrant.  Calls that write the same
 * output buffer on different streams race, as with any kernel.
 */
#ifndef SKG_H
#define SKG_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKG_ABI_VERSION 2

typedef enum skg_status {
  SKG_OK = 0,
  SKG_E_INVALID_ARG = 1, /* null pointer, unknown enum value, bad count     */
  SKG_E_SHAPE = 2,       /* K/M/N outside what the entry point accepts      */
  SKG_E_ALIGN = 3,       /* pointer not aligned as documented               */
  SKG_E_UNSUPPORTED = 4, /* valid enum values that this entry point rejects */
  SKG_E_DEVICE = 5,      /* no device, or the current device is not gfx950  */
  SKG_E_HIP = 6          /* a HIP launch failed; see skg_last_error()       */
} skg_status;

/* (weight format, activation format) pair of a product. */
typedef enum skg_fmt {
  SKG_BF16_BF16 = 0, /* bf16 W  x bf16 x          (gemv)                    */
  SKG_Q8_0_F32 = 1,  /* q8_0 W  x float32 x       (gemv)                    */
  SKG_Q4_0_F32 = 2,  /* q4_0 W  x float32 x       (gemv)                    */
  SKG_Q4_0_Q8_1 = 3, /* q4_0 W  x Q8_1 x, integer dot (gemv)                */
  SKG_Q8_0_Q8_1 = 4, /* q8_0 W  x Q8_1 x, integer dot (gemv)                */
  SKG_Q4_0_BF16 = 5, /* q4_0 W  x bf16 x, MFMA tile (gemm_tiled)            */
  SKG_Q8_0_BF16 = 6, /* q8_0 W  x bf16 x, MFMA tile (gemm_tiled)            */
  SKG_Q4_K_F32 = 7,  /* q4_K W  x float32 x       (gemv)                    */
  SKG_Q6_K_F32 = 8,  /* q6_K W  x float32 x       (gemv)                    */
  SKG_Q4_K_Q8_1 = 9, /* q4_K W  x Q8_1 x, integer dot (gemv)                */
  SKG_Q6_K_Q8_1 = 10, /* q6_K W  x Q8_1 x, integer dot (gemv)               */
  SKG_Q4_K_BF16 = 11, /* q4_K W  x bf16 x, MFMA tile (gemm_tiled)           */
  SKG_Q6_K_BF16 = 12  /* q6_K W  x bf16 x, MFMA tile (gemm_tiled)           */
} skg_fmt;

typedef enum skg_epi {
  SKG_EPI_NONE = 0,       /* each matrix writes its own output              */
  SKG_EPI_SWIGLU = 1,     /* two matrices (gate, up) -> h = silu(g) * u     */
  SKG_EPI_SWIGLU_Q8_1 = 2 /* as SWIGLU, and h also as Q8_1 blocks           */
} skg_epi;

/* ABI version of the loaded library (SKG_ABI_VERSION it was built with). */
int skg_abi_version(void);

/* Static text of a status code ("SKG_OK", ...); never NULL. */
const char* skg_status_str(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* skg_last_error(void);

/*
 * Weight packing (load time, not on the timed path).
 *
 * "The Shape That Actually Matters" (Round 1 and Round 2) re-lays the weights
 * out once at load time so that loads coalesce; "Six hypotheses, four
 * refutations" (What the failure left behind) gives every lane a full q4_0
 * block through wide loads.  pack_weights is that one-time byte permutation:
 * the 18/34-byte blocks are split into 16-byte-aligned code payloads and a
 * separate fp16 scale stream, so every lane streams whole blocks with 16-byte
 * loads.  The packed layout is opaque and versioned by skg_packed_size.
 *
 * skg_packed_size: bytes of the packed buffer for an N x K matrix of the
 *   weight format of `fmt`, or 0 if (fmt, N, K) is invalid.  1 <= N <=
 *   2^31 - 1; K <= 2^30 and K >= 32, K % 32 == 0 for q8_0/q4_0, K >= 8 and
 *   K % 8 == 0 for bf16, K >= 256 and K % 256 == 0 for q4_K/q6_K.
 * skg_pack_weights: src = canonical N x K weights (device, 2-byte aligned),
 *   N * K / 32 / 256 < 2^31 - 1 for q8_0/q4_0 (one launch; else SKG_E_SHAPE),
 *   dst = packed buffer of skg_packed_size bytes (device, 256-byte aligned).
 *   src and dst must not overlap.
 * skg_packed_size_multi / skg_pack_weights_multi: n (1..4) matrices of
 *   Ns[i] x K sharing one activation (fused Q/K/V, or gate and up) packed into
 *   one buffer, in order.  srcs is a host array of n device pointers.
 */
size_t skg_packed_size(skg_fmt fmt, int64_t N, int64_t K);
skg_status skg_pack_weights(skg_fmt fmt, int64_t N, int64_t K, const void* src, void* dst,
                            hipStream_t stream);
size_t skg_packed_size_multi(skg_fmt fmt, int n, const int64_t* Ns, int64_t K);
skg_status skg_pack_weights_multi(skg_fmt fmt, int n, const int64_t* Ns, int64_t K,
                                  const void* const* srcs, void* dst, hipStream_t stream);

/*
 * Activation quantisation to Q8_1.
 *
 * The RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach &
 * Methodology) feeds Q8_1 activations to its Q4_0 x Q8_1 integer-dot matvec.
 * Per 32-element block, in IEEE binary32: amax = max|x_i|; d = amax / 127;
 * id = (d != 0) ? 1/d : 0; q_i = round-half-away(x_i * id); stored
 * d = fp16_rne(d); stored s = fp16_rne(d * (float)sum_i q_i).
 *
 * x : float32 [M][K] device, 16-byte aligned.  xq : [M][K/32] 36-byte Q8_1
 * blocks, device, 4-byte aligned.  M >= 1 (any), K >= 32, K % 32 == 0.
 * The result is bit-exact (unique given the operation sequence above).
 */
skg_status skg_quantize_act_q8_1(int64_t M, int64_t K, const float* x, void* xq, hipStream_t stream);

/*
 * RMSNorm with a per-channel gain, optionally writing its Q8_1 encoding in
 * the same launch.
 *
 * The RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach &
 * Methodology) has the RMSNorm-plus-scale dispatch before a Q4_0 matvec write
 * the Q8_1 activation that matvec reads, so no standalone quantisation
 * dispatch runs; "Six hypotheses, four refutations" (Hypothesis ledger:
 * fewer, longer kernels) counts the same fusion among its launch savings.
 * Per row m, in IEEE binary32: ss = sum_k x[m][k]^2 (a fixed reduction order,
 * so repeated calls give identical bits); r = 1 / sqrt(ss / K + eps);
 * xn[m][k] = (x[m][k] * r) * g[k].  xq receives exactly
 * skg_quantize_act_q8_1 of those xn values.
 *
 * x  : float32 [M][K] device, 16-byte aligned.
 * g  : float32 [K] device, 16-byte aligned, or NULL for a gain of 1.
 * eps: finite, >= 0.  With eps == 0 an all-zero row has no normalisation
 *      (its outputs are NaN); a row whose sum of squares overflows binary32
 *      is outside the domain.
 * xn : float32 [M][K] device, 16-byte aligned, or NULL (not written).
 * xq : [M][K/32] 36-byte Q8_1 blocks, device, 4-byte aligned, or NULL.
 * At least one of xn and xq is given.  1 <= M <= 2^24; 32 <= K <= 16384,
 * K % 32 == 0.  x must not overlap xn or xq.
 * Errors: SKG_E_SHAPE (M, K), SKG_E_INVALID_ARG (null x, both outputs null,
 * eps negative or not finite), SKG_E_ALIGN.
 */
skg_status skg_rmsnorm_q8_1(int64_t M, int64_t K, const float* x, const float* g, float eps, float* xn, void* xq,
                            hipStream_t stream);

/*
 * Skinny GEMM / GEMV: y[m][n] = sum_k W[n][k] x[m][k], 1 <= M <= 8.
 *
 * fmt   : SKG_BF16_BF16, SKG_Q8_0_F32, SKG_Q4_0_F32, SKG_Q4_0_Q8_1, SKG_Q8_0_Q8_1.
 * W     : packed weights from skg_pack_weights(fmt, N, K) (device).
 * x     : bf16 [M][K] (BF16_BF16), float32 [M][K] (*_F32), or Q8_1 blocks
 *         [M][K/32] (*_Q8_1); device; 16-byte aligned (4-byte for Q8_1).
 * y     : float32 [M][N] device, 4-byte aligned; overwritten.
 * Accumulation is fp32; integer-dot formats sum each block's int8 products
 * exactly in int32 and scale in fp32: per block dW * (dA * sumi - 8 * s) for
 * q4_0, dW * dA * sumi for q8_0.
 * Errors: SKG_E_SHAPE unless 1 <= M <= 8, N >= 1 and K as for packing
 * (M == 0 is SKG_E_SHAPE; use N or M of the real problem).
 */
skg_status skg_gemv(skg_fmt fmt, int64_t M, int64_t K, int64_t N, const void* W, const void* x,
                    float* y, hipStream_t stream);

/*
 * Several matrices that share one activation, in one launch.
 *
 * "Six hypotheses, four refutations" (Hypothesis ledger: fewer, longer
 * kernels) runs the Q, K and V projections in one launch; the RX 6700 XT
 * Llama 2 7B decode write-up (Approach & Methodology) co-dispatches Q/K/V and
 * evaluates gate and up together, writing their SwiGLU result directly.
 *
 * W  : buffer from skg_pack_weights_multi(fmt, n, Ns, K).
 * ys : host array of device output pointers.
 * epi == SKG_EPI_NONE   : n in 1..4, ys[i] = float32 [M][Ns[i]].
 * epi == SKG_EPI_SWIGLU : n == 2 (gate first, then up), Ns[0] == Ns[1],
 *                         ys[0] = float32 [M][Ns[0]] receives
 *                         h = silu(g) * u, silu(z) = z / (1 + e^-z) in fp32.
 * epi == SKG_EPI_SWIGLU_Q8_1 : as SKG_EPI_SWIGLU, and ys[1] (4-byte aligned)
 *                         receives h as [M][Ns[0] / 32] Q8_1 blocks, the bits
 *                         skg_quantize_act_q8_1(M, Ns[0], ys[0]) would write.
 *                         The workgroup that computes 32 consecutive outputs
 *                         quantises them, so the down projection reads Q8_1
 *                         without a separate quantisation launch (the RX 6700
 *                         XT write-up, Approach & Methodology, has the
 *                         producer of an activation emit its Q8_1 form).
 *                         fmt must be SKG_Q4_0_Q8_1 or SKG_Q8_0_Q8_1 and
 *                         Ns[0] % 32 == 0 (else SKG_E_UNSUPPORTED / SKG_E_SHAPE).
 * Other arguments and errors as skg_gemv.
 */
skg_status skg_gemv_multi(skg_fmt fmt, int64_t M, int64_t K, int n, const int64_t* Ns, const void* W,
                          const void* x, float* const* ys, skg_epi epi, hipStream_t stream);

/*
 * Tiled prefill GEMM on MFMA: y[m][n] = sum_k W[n][k] x[m][k] for large M.
 *
 * "Chapter 2.2 - speed - 64-lane Metal" (the tile; the +1) stops re-reading
 * the weights once per activation row: each 64x64 weight tile is decoded once
 * into padded on-chip memory and serves every row of its output tile.
 *
 * fmt : SKG_Q4_0_BF16, SKG_Q8_0_BF16 (the q8_0 tile of the same page's
 *       q8_0 measurements), SKG_Q4_K_BF16 or SKG_Q6_K_BF16 (the q4_K / q6_K
 *       weights the same page's tile is built for).
 * W   : skg_pack_weights(fmt, N, K) output.
 * x   : bf16 [M][K] device, 16-byte aligned.  y : float32 [M][N], overwritten.
 * Weights are decoded to bf16 (w = bf16_rne(d * (c - 8)) for q4_0,
 * bf16_rne(d * q) for q8_0, both exact before the rounding; for q4_K
 * bf16_rne(fp32_rn(d sc q - dmin m)) and for q6_K
 * bf16_rne(fp32_rn(d sc (q - 32))), the value formed once in binary32) and
 * multiplied on bf16 MFMA with fp32 accumulation.  1 <= M <= 2^31 - 1,
 * N >= 1, K % 32 == 0 (K % 256 == 0 for q4_K/q6_K), and the output must fit
 * one launch: ceil(M / 256) * ceil(N / 112) <= 2^31 - 1 (else SKG_E_SHAPE).
 * q8_0, q4_K and q6_K weights run on the pipelined organisations
 * (skg_gemm_tiled_set_variant 3 or 4); with another organisation selected
 * such a call returns SKG_E_UNSUPPORTED.
 *
 * fmt SKG_Q4_0_Q8_1 / SKG_Q8_0_Q8_1 runs the integer matrix-core tile (the
 * int8 arm of the same tile): x is then the Q8_1 blocks of the activation
 * ([M][K/32] blocks of 36 bytes, 4-byte aligned, as skg_quantize_act_q8_1
 * writes them), each 32-element block's integer dot is exact, and
 * y = sum over blocks of dW * dA * dot in fp32 (q4_0: dot of the codes
 * minus 8).  K % 64 == 0 (else SKG_E_SHAPE), one launch takes
 * ceil(M / 256) * ceil(N / 64) <= 2^31 - 1 tiles, and the organisation
 * selected by skg_gemm_tiled_set_variant does not apply.
 */
skg_status skg_gemm_tiled(skg_fmt fmt, int64_t M, int64_t K, int64_t N, const void* W, const void* x,
                          float* y, hipStream_t stream);

/*
 * Test hook: the int32 block dot products sum_i code_i * qa_i (q4_0) or
 * sum_i q_i * qa_i (q8_0) of rows [n0, n0 + nr) against one Q8_1 activation
 * row, computed by the same device function the gemv kernels use.
 * fmt : SKG_Q4_0_Q8_1 or SKG_Q8_0_Q8_1.  W : packed N x K.  xq : K/32 blocks.
 * out : int32 [nr][K/32] device.  0 <= n0, nr >= 1, n0 + nr <= N.
 */
skg_status skg_debug_block_dots(skg_fmt fmt, int64_t N, int64_t K, int64_t n0, int64_t nr, const void* W,
                                const void* xq, int32_t* out, hipStream_t stream);

/*
 * Streaming-read ceiling: reads `bytes` of `buf` once with 16-byte loads and
 * no arithmetic to speak of, the achievable-bandwidth reference that
 * "Six hypotheses, four refutations" (What the failure left behind) measures
 * with a trivially parallel kernel.  buf : device, 16-byte aligned; bytes a
 * positive multiple of 16.  out : one uint32 (device) that receives a value
 * only when the data hash to an impossible value (it keeps the reads live).
 */
skg_status skg_stream_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

/*
 * Launch-floor reference: enqueues one kernel of `grid` workgroups of `block`
 * threads that does nothing, so back-to-back launches of it measure the fixed
 * cost every launch pays ("Six hypotheses, four refutations", Hypothesis
 * ledger: the per-kernel floor that the dispatch count multiplies).
 * grid : 1 .. 2^31 - 1.  block : a multiple of 64 in 64 .. 1024.  Touches no
 * memory.  SKG_E_SHAPE for any other grid or block.
 */
skg_status skg_empty_launch(int64_t grid, int block, hipStream_t stream);


/*
 * Tuning hooks (measurement only).  The GEMV kernels are compiled in several
 * variants; occupancy and rows per wave are chosen by measurement, not
 * maximised ("Six hypotheses, four refutations", Four traps: full occupancy
 * is a cliff; the hardware maximum is a cliff).
 *
 * skg_gemv_set_variant: use the compiled variant with `ro` output rows per
 *   row group, `j` 16-byte units per lane per K chunk, activation staged in
 *   LDS (x_lds = 1) or registers (0), `waves` waves per workgroup and `kw`
 *   waves sharing each row group (each takes every kw-th K chunk; partial sums
 *   meet in LDS) for every later gemv / gemv_multi call with this
 *   (fmt, M, epi); ro = 0 restores the default.  SKG_E_UNSUPPORTED if that
 *   variant is not compiled; a later call returns SKG_E_UNSUPPORTED if the
 *   selected variant does not take its K.
 *   x_lds = 2 names the matrix-core kernel of the fp32-activation quantised
 *   formats (SKG_Q8_0_F32, SKG_Q4_0_F32, SKG_Q4_K_F32; also the Q8_1 formats
 *   of q4_0 and q8_0 on the integer matrix cores): ro = 16 output rows per tile, j =
 *   fp16 terms carrying each activation (2: ~22 bits; 1: one rounding to
 *   fp16, relative error 2^-11), waves = most waves per workgroup, kw =
 *   quantisation blocks per wave; it takes K with (K / 32) % kw == 0 and
 *   K / 32 <= waves * kw.
 *   x_lds = 3 names the same matrix-core computation with the weight tiles
 *   copied by direct global-to-LDS transfers into a ring of two or three
 *   16-row slots (the activation as for x_lds = 2; formats q4_0 / q8_0 x fp32
 *   and q4_0 / q8_0 / q4_K / q6_K x Q8_1); compiled for K = 4096 only
 *   (waves * kw = 128 blocks), so a call with any other K returns
 *   SKG_E_UNSUPPORTED while it is selected.
 *   x_lds = 4 names the same matrix-core computation with a private weight
 *   ring per wave (each wave copies its own 16-block slice of every tile into
 *   `depth` LDS slots; no workgroup barrier until the last tile); it takes K
 *   with (K / 32) % 16 == 0 and K / 32 <= 128.
 *   x_lds = 5 names the ring kernel of x_lds = 3 for fp32 activations with
 *   several quantisation blocks per chain of MFMAs (a block-diagonal A
 *   operand: four blocks for M <= 4 and two for M = 5..8 with j = 1; two
 *   blocks of four hi and four lo rows, or a second chain of lo operands,
 *   with j = 2; q4_0, q8_0, q4_K, and q6_K by block-halves); compiled for
 *   K = 4096 only, like x_lds = 3.
 *   depth: weight tiles in flight (1 for the vector kernels; the prefetch
 *   depth of x_lds = 2, 1 or 2; the ring slots of x_lds = 3 or 5, 2 or 3, or
 *   4 for q4_0 weights); 0 matches any depth.
 * skg_gemv_variants: writes up to max_entries records of SKG_VARIANT_FIELDS
 *   ints {fmt, M, epi, ro, j, x_lds, waves, kw, depth} to out (host) and
 *   returns the number of compiled variants.  For each (fmt, M, epi) and K
 *   the default is the first record whose variant takes that K.
 * skg_set_lds_pad: extra dynamic LDS bytes (0..65536) requested by every gemv
 *   launch, which lowers occupancy without changing the code (the MI50 case
 *   study's diagnostic control).  Initial value: $SKG_LDS_PAD_BYTES or 0.
 *   The environment value must be a base-10 integer in 0..65536 (blanks
 *   around it allowed); any other value makes every skg_gemv and
 *   skg_gemv_multi call return SKG_E_INVALID_ARG, before any HIP call, until
 *   skg_set_lds_pad sets a valid pad.
 * These settings are process-wide and must not change while another thread
 * is launching gemv work.
 */
#define SKG_VARIANT_FIELDS 9
skg_status skg_gemv_set_variant(skg_fmt fmt, int M, skg_epi epi, int ro, int j, int x_lds, int waves, int kw,
                                int depth);
int skg_gemv_variants(int* out, int max_entries);
/* skg_gemv_default_variant: the record (SKG_VARIANT_FIELDS ints, as skg_gemv_variants) of the
 * variant a skg_gemv / skg_gemv_multi call with this (fmt, M, epi, K) runs
 * now, honouring skg_gemv_set_variant; out is host memory.  SKG_E_UNSUPPORTED
 * when no compiled variant takes K; SKG_E_INVALID_ARG / SKG_E_SHAPE for an
 * unknown fmt or epilogue or M outside 1..8.  Host only, no HIP call. */
skg_status skg_gemv_default_variant(skg_fmt fmt, int M, skg_epi epi, int64_t K, int* out);
skg_status skg_set_lds_pad(int64_t bytes);
/* skg_gemm_tiled_set_variant: prefill kernel organisation, 0 = every wave
 * decodes weights and runs MFMAs, 1 = producer waves decode, consumer waves
 * run MFMAs, 4 consumer waves of 64 rows, 2 = as 1 with 8 consumer waves of
 * 32 rows, 3 = as 1 with a triple-buffered weight tile so fragment reads
 * overlap the MFMAs, 4 = as 3 with the activation slices copied straight
 * from global memory into LDS (default); -1 restores the default.
 * Process-wide. */
skg_status skg_gemm_tiled_set_variant(int variant);

#ifdef __cplusplus
}
#endif

#endif /* SKG_H */
