"""GPU parity of the skinny GEMM / GEMV entry points against the CPU oracle.

Small shapes span several K chunks, ragged row groups and K tails; every
compiled kernel variant is checked; outputs are NaN-poisoned first so rows a
kernel fails to write show up.  Float outputs must satisfy
|y - y_ref| <= 2e-3 * sum|w x| + 1e-6; integer block dots and the Q8_1
quantiser must match exactly."""

import numpy as np
import pytest

import oracle
from synth import inputs as si
from tests._gpu import assert_close, dev, host, note, poisoned, sample_rows
from tests._q8_1_check import q8_1_violations

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def skg():
    import skinny_gemm_decode_amd as m
    return m


def wkind(skg, fmt):
    return skg.WEIGHT_KIND[fmt]


def is_q8_1(skg, fmt):
    return fmt in skg.Q8_1_FMTS


def is_kquant(fmt):
    return fmt >= 7


def k_of(skg, fmt, bf16_k=4104, q_k=4128, kq_k=4352):
    """A K with a ragged last chunk for each weight kind (K-quants: a
    multiple of 256)."""
    return bf16_k if fmt == skg.BF16_BF16 else (kq_k if is_kquant(fmt) else q_k)


def make_inputs(skg, fmt, M, N, K, seed):
    rng = si.rng_for(0, 99, seed)
    W = si.weights(wkind(skg, fmt), rng, N, K)
    x = si.activations_bf16(rng, M, K) if fmt == skg.BF16_BF16 else si.activations_f32(rng, M, K)
    return W, x


def gpu_activation(skg, fmt, x):
    """Device activation in the format the kernel reads (Q8_1 quantised on the
    GPU and checked bit-exactly against the oracle's quantiser first)."""
    xd = dev(x)
    if not is_q8_1(skg, fmt):
        return xd, None
    import torch
    xq = poisoned((x.shape[0], x.shape[1] // 32, 36), dtype=torch.uint8)
    skg.quantize_act_q8_1(xd, xq)
    ref = oracle.quantize_q8_1(x)
    assert np.array_equal(host(xq), ref), "Q8_1 activation differs from the oracle"
    return xq, ref


def reference(skg, fmt, W, x, xq_ref):
    kind = wkind(skg, fmt)
    if fmt == skg.Q4_0_Q8_1:
        y, _, bound = oracle.gemv_q4_0_q8_1_ref(W, xq_ref)
        return y, bound
    if fmt == skg.Q8_0_Q8_1:
        return oracle.gemv_q8_0_q8_1_ref(W, xq_ref)
    if is_q8_1(skg, fmt):
        return oracle.gemv_ref(oracle.dequantize(kind, W), oracle.decode_q8_1(xq_ref))
    return oracle.gemv_ref_fmt(kind, W, x, x_kind="bf16" if fmt == skg.BF16_BF16 else "f32")


def run_gemv(skg, fmt, M, N, K, W, x):
    note(f"gemv fmt={skg.FMT_NAMES[fmt]} M={M} N={N} K={K}")
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    xin, xq_ref = gpu_activation(skg, fmt, x)
    y = poisoned((M, N))
    skg.gemv(fmt, M, K, N, Wp, xin, y)
    return host(y), xq_ref


GEMV_FMTS = [0, 1, 2, 3, 4, 7, 8, 9, 10]


def shapes_for(fmt):
    if fmt == 0:
        return [(1, 8), (5, 40), (17, 520), (131, 4104)]
    if is_kquant(fmt):
        return [(1, 256), (3, 512), (17, 768), (131, 4352)]
    return [(1, 32), (3, 96), (17, 288), (131, 4128)]


@pytest.mark.parametrize("fmt", GEMV_FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_small_shapes(skg, fmt, M):
    for i, (N, K) in enumerate(shapes_for(fmt)):
        W, x = make_inputs(skg, fmt, M, N, K, seed=1000 + 100 * fmt + 10 * M + i)
        y, xq_ref = run_gemv(skg, fmt, M, N, K, W, x)
        y_ref, bound = reference(skg, fmt, W, x, xq_ref)
        assert_close(y, y_ref, bound, f"fmt={fmt} M={M} N={N} K={K}")


def test_every_compiled_variant(skg):
    """Each compiled kernel variant, selected through the tuning hook, on a
    shape with ragged row groups and a K tail."""
    variants = skg.gemv_variants()
    assert variants
    cache = {}
    try:
        for v in variants:
            fmt, M, epi = v["fmt"], v["M"], v["epi"]
            N = 320 if epi == skg.EPI_SWIGLU_Q8_1 else 300
            # the matrix-core variants (x_lds 2..5) take K % 512 == 0, K <= 4096
            K = 4096 if v["x_lds"] in (2, 3, 4, 5) else k_of(skg, fmt)
            if v["x_lds"] == 1 and v["kw"] > 1:
                # every K class walks the same number of chunks, the last one partial
                K = 32 * (64 * v["j"] * (2 * v["kw"] - 1) + (8 if is_kquant(fmt) else 10))
            key = (fmt, M, epi, K)
            if key not in cache:
                W0, x = make_inputs(skg, fmt, M, N, K, seed=5000 + 10 * fmt + M)
                W1, _ = make_inputs(skg, fmt, 1, N, K, seed=6000 + 10 * fmt + M)
                cache[key] = (W0, W1, x)
            W0, W1, x = cache[key]
            skg.gemv_select(v)
            note(f"variant {v}")
            xin, xq_ref = gpu_activation(skg, fmt, x)
            if epi == skg.EPI_NONE:
                Wp = skg.pack_weights(fmt, N, K, dev(W0))
                y = poisoned((M, N))
                skg.gemv(fmt, M, K, N, Wp, xin, y)
                y_ref, bound = reference(skg, fmt, W0, x, xq_ref)
                assert_close(host(y), y_ref, bound, f"variant {v}")
            else:
                Wp = skg.pack_weights_multi(fmt, [N, N], K, [dev(W0), dev(W1)])
                h = poisoned((M, N))
                outs = [h]
                if epi == skg.EPI_SWIGLU_Q8_1:
                    outs.append(poisoned_q8_1(M, N))
                skg.gemv_multi(fmt, M, K, [N, N], Wp, xin, outs, epi=epi)
                g_ref, bg = reference(skg, fmt, W0, x, xq_ref)
                u_ref, bu = reference(skg, fmt, W1, x, xq_ref)
                tol = oracle.swiglu_tolerance(g_ref, u_ref, oracle.tolerance(bg), oracle.tolerance(bu))
                ok, worst = oracle.check_close(host(h), oracle.swiglu_ref(g_ref, u_ref), tol)
                assert ok, f"variant {v}: worst {worst}"
                if epi == skg.EPI_SWIGLU_Q8_1:
                    assert_q8_1_of(host(outs[1]), host(h), f"variant {v}")
            skg.gemv_set_variant(fmt, M, epi, 0)
    finally:
        for v in variants:
            skg.gemv_set_variant(v["fmt"], v["M"], v["epi"], 0)


@pytest.mark.parametrize("fmt", GEMV_FMTS)
def test_gemv_multi_qkv_three_outputs(skg, fmt):
    K = k_of(skg, fmt)
    Ns = [96, 33, 130]
    Ws = [make_inputs(skg, fmt, 1, n, K, seed=7000 + 10 * fmt + i)[0] for i, n in enumerate(Ns)]
    _, x = make_inputs(skg, fmt, 2, 1, K, seed=7100 + fmt)
    note(f"gemv_multi qkv fmt={fmt}")
    Wp = skg.pack_weights_multi(fmt, Ns, K, [dev(w) for w in Ws])
    xin, xq_ref = gpu_activation(skg, fmt, x)
    ys = [poisoned((2, n)) for n in Ns]
    skg.gemv_multi(fmt, 2, K, Ns, Wp, xin, ys)
    for i, (w, y) in enumerate(zip(Ws, ys)):
        y_ref, bound = reference(skg, fmt, w, x, xq_ref)
        assert_close(host(y), y_ref, bound, f"qkv output {i}")


def poisoned_q8_1(M, N):
    """Q8_1 output buffer [M, N/32, 36] filled with 0xA5 bytes."""
    import torch
    return torch.full((M, N // 32, 36), 0xA5, dtype=torch.uint8, device="cuda")


def assert_q8_1_of(hq, h, what):
    """hq (bytes [M, N/32, 36]) holds exactly the oracle's Q8_1 blocks of h."""
    M, N = h.shape
    ref = oracle.quantize_q8_1(h.astype(np.float32))
    assert np.array_equal(hq.reshape(M, N // 32, 36), np.asarray(ref).reshape(M, N // 32, 36)), \
        f"{what}: Q8_1 blocks of h differ from the oracle's quantisation of h"


@pytest.mark.parametrize("fmt", [3, 4])
@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_swiglu_q8_1_epilogue(skg, fmt, M):
    """SwiGLU whose workgroups also write the Q8_1 blocks of h: h within the
    SwiGLU tolerance of the oracle, its blocks bit-identical to the oracle's
    quantisation of the h the GPU wrote, and the down projection fed from
    them equal (bit for bit) to the one fed from a standalone quantisation."""
    K, N = 4128, 32 * 13
    Wg, x = make_inputs(skg, fmt, M, N, K, seed=9700 + 10 * fmt + M)
    Wu, _ = make_inputs(skg, fmt, M, N, K, seed=9800 + 10 * fmt + M)
    Wd, _ = make_inputs(skg, fmt, 1, 96, N, seed=9900 + 10 * fmt + M)
    note(f"swiglu q8_1 epilogue fmt={fmt} M={M}")
    Wp = skg.pack_weights_multi(fmt, [N, N], K, [dev(Wg), dev(Wu)])
    xin, xq_ref = gpu_activation(skg, fmt, x)
    h, hq = poisoned((M, N)), poisoned_q8_1(M, N)
    skg.gemv_multi(fmt, M, K, [N, N], Wp, xin, [h, hq], epi=skg.EPI_SWIGLU_Q8_1)
    g_ref, bg = reference(skg, fmt, Wg, x, xq_ref)
    u_ref, bu = reference(skg, fmt, Wu, x, xq_ref)
    tol = oracle.swiglu_tolerance(g_ref, u_ref, oracle.tolerance(bg), oracle.tolerance(bu))
    ok, worst = oracle.check_close(host(h), oracle.swiglu_ref(g_ref, u_ref), tol)
    assert ok, f"swiglu worst {worst}"
    assert_q8_1_of(host(hq), host(h), "epilogue")
    # and, with no GPU value as oracle input: valid Q8_1 of values within the
    # SwiGLU tolerance of the oracle's h
    bad = q8_1_violations(host(hq).reshape(M, N // 32, 36), oracle.swiglu_ref(g_ref, u_ref), tol)
    assert not bad, "; ".join(bad[:3])
    Wdp = skg.pack_weights(fmt, 96, N, dev(Wd))
    ya, yb = poisoned((M, 96)), poisoned((M, 96))
    skg.gemv(fmt, M, N, 96, Wdp, hq, ya)
    skg.gemv(fmt, M, N, 96, Wdp, skg.quantize_act_q8_1(h), yb)
    assert np.array_equal(host(ya), host(yb))


@pytest.mark.parametrize("fmt", GEMV_FMTS)
@pytest.mark.parametrize("M", [1, 2, 5])
def test_gemv_multi_swiglu_and_its_halves(skg, fmt, M):
    K = k_of(skg, fmt)
    N = 257
    Wg, x = make_inputs(skg, fmt, M, N, K, seed=8000 + 10 * fmt + M)
    Wu, _ = make_inputs(skg, fmt, M, N, K, seed=8100 + 10 * fmt + M)
    note(f"gemv_multi swiglu fmt={fmt} M={M}")
    Wp = skg.pack_weights_multi(fmt, [N, N], K, [dev(Wg), dev(Wu)])
    xin, xq_ref = gpu_activation(skg, fmt, x)
    h = poisoned((M, N))
    skg.gemv_multi(fmt, M, K, [N, N], Wp, xin, [h], epi=skg.EPI_SWIGLU)
    # the same packed pair without the epilogue: each half on its own
    g, u = poisoned((M, N)), poisoned((M, N))
    skg.gemv_multi(fmt, M, K, [N, N], Wp, xin, [g, u], epi=skg.EPI_NONE)
    g_ref, bg = reference(skg, fmt, Wg, x, xq_ref)
    u_ref, bu = reference(skg, fmt, Wu, x, xq_ref)
    assert_close(host(g), g_ref, bg, "gate")
    assert_close(host(u), u_ref, bu, "up")
    tol = oracle.swiglu_tolerance(g_ref, u_ref, oracle.tolerance(bg), oracle.tolerance(bu))
    ok, worst = oracle.check_close(host(h), oracle.swiglu_ref(g_ref, u_ref), tol)
    assert ok, f"swiglu worst {worst}"


@pytest.mark.parametrize("fmt", [3, 4])
def test_block_dots_bit_exact(skg, fmt):
    N, K = 37, 4128
    W, x = make_inputs(skg, fmt, 1, N, K, seed=9000 + fmt)
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    xq, xq_ref = gpu_activation(skg, fmt, x)
    note(f"block dots fmt={fmt}")
    import torch
    out = poisoned((N - 3, K // 32), dtype=torch.int32)
    skg.debug_block_dots(fmt, N, K, 3, N - 3, Wp, xq, out)
    ref = (oracle.block_dots_q4_0_q8_1 if fmt == 3 else oracle.block_dots_q8_0_q8_1)(W[3:], xq_ref[0])
    assert np.array_equal(host(out), ref)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_one_hot_activation_is_bit_exact(skg, fmt):
    N, K = 70, 4096 if fmt else 4104
    W, _ = make_inputs(skg, fmt, 1, N, K, seed=9100 + fmt)
    Wd = oracle.dequantize(wkind(skg, fmt), W)
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    for k in (0, 31, 33, K - 1):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        if fmt == skg.BF16_BF16:
            x = np.zeros((1, K), np.uint16)
            x[0, k] = 0x3F80
        note(f"one-hot fmt={fmt} k={k}")
        y = poisoned((1, N))
        skg.gemv(fmt, 1, K, N, Wp, dev(x), y)
        assert np.array_equal(host(y)[0].astype(np.float64), Wd[:, k]), f"k={k}"


def test_q4_0_all_codes_eight(skg):
    """Blocks whose codes are all 8 decode to zero: exactly zero on the float
    path, and the second reference (stored block sum) on the Q8_1 path."""
    N, K = 40, 4096
    W, x = make_inputs(skg, skg.Q4_0_F32, 1, N, K, seed=9200)
    W[..., 2:] = 0x88
    y, _ = run_gemv(skg, skg.Q4_0_F32, 1, N, K, W, x)
    assert np.all(y == 0.0)
    y8, xq_ref = run_gemv(skg, skg.Q4_0_Q8_1, 1, N, K, W, x)
    y_ref, y_ref_s, _ = oracle.gemv_q4_0_q8_1_ref(W, xq_ref)
    assert np.all(y_ref == 0.0)
    dW = oracle.fp16_bits_to_f64(W[..., 0].astype(np.uint16) | (W[..., 1].astype(np.uint16) << 8))
    dA, sA, qa = oracle.q8_1_fields(xq_ref[0])
    bound_s = np.sum(np.abs(dW) * (np.abs(dA) * 8 * np.abs(qa).sum(-1) + 8 * np.abs(sA)), axis=1)[None, :]
    assert_close(y8, y_ref_s, bound_s, "all-8 vs stored-sum reference")


def test_bf16_scale_boundaries(skg):
    """bf16 weights and activations spanning many binades, K = 8 (one unit)."""
    N, K = 9, 8
    W = np.array([[0x3F80, 0xBF80, 0x7F7F, 0x0080, 0x8001, 0x4000, 0x3E00, 0xC2C8]] * N, np.uint16)
    W[:, 2] = 0x4700   # keep products finite
    x = np.array([[0x3F80, 0x3F80, 0x3F00, 0x7000, 0x0000, 0xC000, 0x4100, 0x3C00]], np.uint16)
    y, _ = run_gemv(skg, skg.BF16_BF16, 1, N, K, W, x)
    y_ref, bound = oracle.gemv_ref_fmt("bf16", W, x, x_kind="bf16")
    assert_close(y, y_ref, bound, "bf16 boundaries")


# Shapes the matrix-core kernel takes (K % 512 == 0, K <= 4096): one wave
# (K = 512), a partial workgroup (K = 1536: 3 waves), ragged row tiles, and
# N large enough that workgroups walk 2, 3 and 5+ tiles.  The default-path
# part also runs K = 1280, which the matrix-core kernel does not take.
MFMA_SHAPES = [(1, 512), (19, 512), (300, 4096), (1000, 1536), (37, 1280), (9000, 4096), (20000, 4096)]


def mfma_variants(skg, fmt, M):
    return [v for v in skg.gemv_variants()
            if v["fmt"] == fmt and v["M"] == M and v["epi"] == skg.EPI_NONE and v["x_lds"] in (2, 3, 4, 5)]


@pytest.mark.parametrize("fmt", [1, 2, 3, 4, 7, 8, 9, 10])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemv_mfma_shapes(skg, fmt, M):
    """Default path at the shapes the matrix-core kernel takes, then every
    matrix-core variant against its own precision: with two fp16 activation
    terms (~22 bits) the error stays under 2e-5 of sum|w x|, which fails if the
    low term were lost; with one term it stays under 2^-11 (its rounding) plus
    fp32 accumulation, 8e-4 of sum|w x|; on Q8_1 activations the block dots
    are exact int32 and only the fp32 scaling rounds, 2e-5 of sum|w a|
    (q4_K's min term takes the activation block sum s as the Q8_1 block stores
    it, rounded to fp16, so q4_K x Q8_1 keeps the 2e-3 bound)."""
    cases = []
    for i, (N, K) in enumerate(MFMA_SHAPES):
        W, x = make_inputs(skg, fmt, M, N, K, seed=8000 + 100 * fmt + 10 * M + i)
        xq_ref = oracle.quantize_q8_1(x) if is_q8_1(skg, fmt) else None
        # large cases: the oracle evaluates a sample of rows (both ends, the
        # ragged tail and a seeded sample), the kernel computes them all
        rows = sample_rows(N, seed=M + i) if N * K * M > 20000 * 4096 * 2 else np.arange(N)
        y_ref, bound = reference(skg, fmt, W[rows], x, xq_ref)
        cases.append((N, K, W, x, y_ref, bound, rows))
        y, _ = run_gemv(skg, fmt, M, N, K, W, x)
        assert_close(y[:, rows], y_ref, bound, f"default fmt={fmt} M={M} N={N} K={K}")
    try:
        for v in mfma_variants(skg, fmt, M):
            skg.gemv_select(v)
            rel = (oracle.REL_TOL if fmt == skg.Q4_K_Q8_1 else
                   2e-5 if (v["j"] == 2 or is_q8_1(skg, fmt)) else 8e-4)
            for N, K, W, x, y_ref, bound, rows in cases:
                nb = K // 32
                if nb % v["kw"] or nb > v["waves"] * v["kw"]:
                    continue
                if v["x_lds"] in (3, 5) and nb != v["waves"] * v["kw"]:
                    continue  # the LDS-ring variant is compiled for K = 4096 only
                note(f"variant {v} N={N} K={K}")
                y, _ = run_gemv(skg, fmt, M, N, K, W, x)
                assert_close(y[:, rows], y_ref, bound, f"variant {v} N={N} K={K}", rel=rel)
    finally:
        skg.gemv_set_variant(fmt, M, 0, 0)


def range_activations(rng, M, K):
    """Rows far outside fp16 range, zero, far below it, one huge outlier, a
    half scaled by 1e20 and outliers in every quarter of some blocks."""
    x = si.activations_f32(rng, M, K)
    x[0] *= np.float32(1e6)          # |x| up to ~5e6 (fp16 max is 65504)
    x[1] = 0.0
    x[2] *= np.float32(1e-30)        # far below fp16's smallest subnormal
    x[3, 1234] = np.float32(3e9)     # one outlier dominating its wave's range
    x[4, : K // 2] *= np.float32(1e20)
    # outliers in every quarter of a block (elements 4g..4g+3 and 16+4g..
    # 16+4g+3 go to lane group g of the matrix-core kernels), so a scale
    # taken from part of a row's lanes overflows fp16
    for blk, e in ((3, 13), (40, 30), (77, 6), (100, 21), (126, 0)):
        x[5, 32 * blk + e] = np.float32(7e4 * (1 + blk))
    return x


def zero_weight(kind, W, n, k):
    """Set element k of row n of canonical weights W to the code whose weight
    is exactly zero (q8_0: 0, q4_0: 8, q6_K: 32); returns whether the format
    has one."""
    if kind == "q8_0":
        W[n, k // 32, 2 + k % 32] = 0
    elif kind == "q4_0":
        b, i = k // 32, k % 32
        byte = W[n, b, 2 + i % 16]
        W[n, b, 2 + i % 16] = (byte & 0xF0) | 8 if i < 16 else (byte & 0x0F) | 0x80
    elif kind == "q6_K":
        sb, e = k // 256, k % 256
        h, r = e // 128, e % 128
        g, l = r // 32, r % 32
        qi = 64 * h + 32 * (g & 1) + l        # low four bits: 0
        sh = 4 * (g >> 1)
        W[n, sb, qi] &= np.uint8(~(0xF << sh) & 0xFF)
        hi = 128 + 32 * h + l                 # top two bits: 0b10
        W[n, sb, hi] = (W[n, sb, hi] & np.uint8(~(3 << (2 * g)) & 0xFF)) | np.uint8(2 << (2 * g))
    else:
        return False
    return True


@pytest.mark.parametrize("fmt", [1, 2, 7, 8])
def test_gemv_activation_range_single_rows(skg, fmt):
    """The M = 1 defaults (vector ALU) on each pathological activation row
    alone, with the weights of every other output row made exactly zero at
    the outliers' positions (q8_0 code 0, q4_0 code 8, q6_K code 32): such an
    outlier must contribute nothing, not cancel against itself and erase the
    rest of its block."""
    N, K = 300, 4096
    rng = si.rng_for(0, 99, 8950 + fmt)
    kind = wkind(skg, fmt)
    W = si.weights(kind, rng, N, K)
    x = range_activations(rng, 6, K)
    for k in [1234] + [32 * blk + e for blk, e in ((3, 13), (40, 30), (77, 6), (100, 21), (126, 0))]:
        for n in range(0, N, 2):
            zero_weight(kind, W, n, k)
    if kind in ("q8_0", "q4_0", "q6_K"):
        assert np.all(oracle.dequantize(kind, W)[::2, 1234] == 0.0)
    for m in range(6):
        xm = np.ascontiguousarray(x[m:m + 1])
        y_ref, bound = reference(skg, fmt, W, xm, None)
        y, _ = run_gemv(skg, fmt, 1, N, K, W, xm)
        assert_close(y, y_ref, bound, f"fmt={fmt} M=1 row {m}")
        if m == 1:
            assert np.all(y == 0.0), "all-zero activation row must give exact zeros"


@pytest.mark.parametrize("fmt", [1, 2, 7, 8])
def test_gemv_mfma_activation_range(skg, fmt):
    """Activations far outside fp16 range, far below it, an all-zero row and
    a single huge outlier: the per-wave power-of-two scaling keeps the two
    fp16 terms exact enough everywhere."""
    M, N, K = 6, 300, 4096
    rng = si.rng_for(0, 99, 8900 + fmt)
    W = si.weights(wkind(skg, fmt), rng, N, K)
    x = range_activations(rng, M, K)
    y_ref, bound = reference(skg, fmt, W, x, None)
    y, _ = run_gemv(skg, fmt, M, N, K, W, x)
    assert_close(y, y_ref, bound, f"fmt={fmt} range")
    assert np.all(y[1] == 0.0), "all-zero activation row must give exact zeros"
    try:
        for v in mfma_variants(skg, fmt, M):
            skg.gemv_select(v)
            note(f"range variant {v}")
            y, _ = run_gemv(skg, fmt, M, N, K, W, x)
            assert_close(y, y_ref, bound, f"fmt={fmt} range variant {v}")
            assert np.all(y[1] == 0.0), f"variant {v}: all-zero activation row must give exact zeros"
    finally:
        skg.gemv_reset(fmt, M)


@pytest.mark.parametrize("fmt", [1, 2, 7])
def test_gemv_multi_mfma(skg, fmt):
    """Several matrices in one matrix-core launch (fused QKV shape)."""
    K, M = 4096, 3
    Ns = [96, 33, 130]
    Ws = [make_inputs(skg, fmt, 1, n, K, seed=8800 + 10 * fmt + i)[0] for i, n in enumerate(Ns)]
    _, x = make_inputs(skg, fmt, M, 1, K, seed=8850 + fmt)
    note(f"gemv_multi mfma fmt={fmt}")
    Wp = skg.pack_weights_multi(fmt, Ns, K, [dev(w) for w in Ws])
    ys = [poisoned((M, n)) for n in Ns]
    skg.gemv_multi(fmt, M, K, Ns, Wp, dev(x), ys)
    for W, y in zip(Ws, ys):
        y_ref, bound = reference(skg, fmt, W, x, None)
        assert_close(host(y), y_ref, bound, f"multi mfma fmt={fmt}")


def test_binding_refuses_short_and_strided_buffers(skg):
    """Real device tensors that are too short or not contiguous are refused by
    the binding before anything is launched; the output stays untouched."""
    import torch

    M, N, K = 2, 64, 256
    W, x = make_inputs(skg, 2, M, N, K, seed=9100)
    Wp = skg.pack_weights(2, N, K, dev(W))
    xd = dev(x)
    y = poisoned((M, N))
    before = host(y).copy()
    with pytest.raises(ValueError, match="y holds"):
        skg.gemv(2, M, K, N, Wp, xd, y[:1])
    with pytest.raises(ValueError, match="x holds"):
        skg.gemv(2, M, K, N, Wp, xd[:1], y)
    with pytest.raises(ValueError, match="W holds"):
        skg.gemv(2, M, K, N, Wp[:-16], xd, y)
    with pytest.raises(ValueError, match="contiguous"):
        skg.gemv(2, M, K, N, Wp, torch.cat([xd, xd], dim=1)[:, ::2], y)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), before, equal_nan=True)


@pytest.mark.parametrize("fmt", GEMV_FMTS)
@pytest.mark.parametrize("M", [1, 2, 8])
def test_gemv_long_k(skg, fmt, M):
    """K far beyond the model widths (16384, 32768): rows walk many K chunks,
    and at M >= 2 the matrix-core defaults (K <= 4096) hand the call to the
    vector kernels; ragged N."""
    for i, K in enumerate((16384, 32768)):
        N = 67
        W, x = make_inputs(skg, fmt, M, N, K, seed=9300 + 100 * fmt + 10 * M + i)
        note(f"long K fmt={fmt} M={M} K={K}")
        y, xq_ref = run_gemv(skg, fmt, M, N, K, W, x)
        y_ref, bound = reference(skg, fmt, W, x, xq_ref)
        assert_close(y, y_ref, bound, f"fmt={fmt} M={M} N={N} K={K}")
