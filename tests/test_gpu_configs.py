"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default kernel variants).  Where the oracle would take long,
it computes a sample of output rows (always including the first and last row
and rows of the last, ragged workgroup)."""

import numpy as np
import pytest

import oracle
from synth import inputs as si
from tests._gpu import assert_close, dev, host, note, poisoned, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def skg():
    import skinny_gemm_decode_amd as m
    return m


def test_q8_0_m1_k256_n512(skg):
    N, K = 512, 256
    rng = si.rng_for(0, 1, 0)
    W = si.q8_0_weights(rng, N, K)
    x = si.activations_f32(rng, 1, K)
    note("q8_0 M=1 K=256 N=512")
    Wp = skg.pack_weights(skg.Q8_0_F32, N, K, dev(W))
    y = poisoned((1, N))
    skg.gemv(skg.Q8_0_F32, 1, K, N, Wp, dev(x), y)
    y_ref, bound = oracle.gemv_ref_fmt("q8_0", W, x)
    assert_close(host(y), y_ref, bound, "q8_0 M=1 K=256 N=512")


def test_bf16_m1_k4096_n12288(skg):
    N, K = 12288, 4096
    rng = si.rng_for(0, 2, 0)
    W = si.bf16_weights(rng, N, K)
    x = si.activations_bf16(rng, 1, K)
    note("bf16 M=1 K=4096 N=12288")
    Wp = skg.pack_weights(skg.BF16_BF16, N, K, dev(W))
    y = poisoned((1, N))
    skg.gemv(skg.BF16_BF16, 1, K, N, Wp, dev(x), y)
    y_ref, bound = oracle.gemv_ref_fmt("bf16", W, x, x_kind="bf16")
    assert_close(host(y), y_ref, bound, "bf16 M=1 K=4096 N=12288")


@pytest.mark.parametrize("kind,fmt", [("q8_0", 1), ("q4_0", 2)])
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_skinny_k4096_n14336(skg, kind, fmt, M):
    N, K = 14336, 4096
    rng = si.rng_for(0, 4, 10 * fmt + M)
    W = si.weights(kind, rng, N, K)
    x = si.activations_f32(rng, M, K)
    note(f"{kind} x f32 M={M} K=4096 N=14336")
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    y = poisoned((M, N))
    skg.gemv(fmt, M, K, N, Wp, dev(x), y)
    yh = host(y)
    assert np.all(np.isfinite(yh))
    rows = sample_rows(N, seed=M)
    y_ref, bound = oracle.gemv_ref_fmt(kind, W[rows], x)
    assert_close(yh[:, rows], y_ref, bound, f"{kind} M={M}")


def test_llama2_7b_q4_0_q8_1_layer_chain(skg):
    """One Llama-2-7B-shaped decode layer, M=1: quantize(x) -> fused QKV ->
    fused gate/up + SwiGLU -> quantize(h) -> down.  Each stage is checked where
    it acts; the chain end to end against the oracle's own chain."""
    import torch
    D, F = 4096, 11008
    rng = si.rng_for(0, 3, 0)
    Wq, Wk, Wv = (si.q4_0_weights(rng, D, D) for _ in range(3))
    Wg, Wu = si.q4_0_weights(rng, F, D), si.q4_0_weights(rng, F, D)
    Wd = si.q4_0_weights(rng, D, F)
    x = si.activations_f32(rng, 1, D)
    fmt = skg.Q4_0_Q8_1
    note("layer chain: pack")
    Pqkv = skg.pack_weights_multi(fmt, [D, D, D], D, [dev(Wq), dev(Wk), dev(Wv)])
    Pgu = skg.pack_weights_multi(fmt, [F, F], D, [dev(Wg), dev(Wu)])
    Pd = skg.pack_weights(fmt, D, F, dev(Wd))

    note("layer chain: quantize x")
    xq = skg.quantize_act_q8_1(dev(x))
    xq_ref = oracle.quantize_q8_1(x)
    assert np.array_equal(host(xq), xq_ref)

    note("layer chain: qkv")
    ys = [poisoned((1, D)) for _ in range(3)]
    skg.gemv_multi(fmt, 1, D, [D, D, D], Pqkv, xq, ys)
    rows = sample_rows(D, seed=3)
    for name, W, y in zip("qkv", (Wq, Wk, Wv), ys):
        y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(W[rows], xq_ref)
        assert_close(host(y)[:, rows], y_ref, bound, f"{name} projection")

    note("layer chain: gate/up + swiglu")
    h = poisoned((1, F))
    skg.gemv_multi(fmt, 1, D, [F, F], Pgu, xq, [h], epi=skg.EPI_SWIGLU)
    hh = host(h)
    frows = sample_rows(F, seed=4)
    g_ref, _, bg = oracle.gemv_q4_0_q8_1_ref(Wg[frows], xq_ref)
    u_ref, _, bu = oracle.gemv_q4_0_q8_1_ref(Wu[frows], xq_ref)
    tol = oracle.swiglu_tolerance(g_ref, u_ref, oracle.tolerance(bg), oracle.tolerance(bu))
    ok, worst = oracle.check_close(hh[:, frows], oracle.swiglu_ref(g_ref, u_ref), tol)
    assert ok, f"swiglu worst {worst}"

    note("layer chain: down projection stage on a generated h")
    h_in = si.activations_f32(si.rng_for(0, 3, 1), 1, F) * np.float32(0.05)
    hq = skg.quantize_act_q8_1(dev(h_in))
    hq_ref = oracle.quantize_q8_1(h_in)
    assert np.array_equal(host(hq), hq_ref)
    yd = poisoned((1, D))
    skg.gemv(fmt, 1, F, D, Pd, hq, yd)
    yd_ref, _, bd = oracle.gemv_q4_0_q8_1_ref(Wd[rows], hq_ref)
    assert_close(host(yd)[:, rows], yd_ref, bd, "down projection (K=11008)")

    note("layer chain: end to end")
    hq_gpu = skg.quantize_act_q8_1(h)
    yo = poisoned((1, D))
    skg.gemv(fmt, 1, F, D, Pd, hq_gpu, yo)
    g_all, _, _ = oracle.gemv_q4_0_q8_1_ref(Wg, xq_ref)
    u_all, _, _ = oracle.gemv_q4_0_q8_1_ref(Wu, xq_ref)
    h_ref32 = oracle.swiglu_ref(g_all, u_all).astype(np.float32)
    y_end, _, b_end = oracle.gemv_q4_0_q8_1_ref(Wd[rows], oracle.quantize_q8_1(h_ref32))
    assert_close(host(yo)[:, rows], y_end, b_end, "layer end to end")
    del torch


PREFILL_VARIANTS = [0, 1, 2, 3, 4]


@pytest.fixture(params=PREFILL_VARIANTS)
def prefill_variant(skg, request):
    skg.gemm_tiled_set_variant(request.param)
    yield request.param
    skg.gemm_tiled_set_variant(-1)


def test_prefill_tile_m512_k4096_n14336(skg, prefill_variant):
    M, N, K = 512, 14336, 4096
    rng = si.rng_for(0, 5, 0)
    W = si.q4_0_weights(rng, N, K)
    A = si.activations_bf16(rng, M, K)
    note(f"gemm_tiled M=512 K=4096 N=14336 variant {prefill_variant}")
    Wp = skg.pack_weights(skg.Q4_0_BF16, N, K, dev(W))
    y = poisoned((M, N))
    skg.gemm_tiled(skg.Q4_0_BF16, M, K, N, Wp, dev(A), y)
    yh = host(y)
    assert np.all(np.isfinite(yh))
    mrows = sample_rows(M, n=48, seed=5)
    ncols = sample_rows(N, n=2048, seed=6)
    y_ref, bound, y_b = oracle.gemm_tiled_ref(W[ncols], A[mrows])
    assert_close(yh[np.ix_(mrows, ncols)], y_ref, bound, "tile vs exact weights")
    # the bf16-rounded-weight reference classifies what deviation remains
    assert_close(yh[np.ix_(mrows, ncols)], y_b, bound, "tile vs bf16 weights", rel=1e-4)


@pytest.mark.parametrize("M,N,K", [(2048, 256, 2048), (300, 250, 2080), (1, 1, 32), (17, 129, 96), (257, 113, 4096)])
def test_prefill_tile_ragged_shapes(skg, prefill_variant, M, N, K):
    """Ragged tiles, odd block counts (K tail inside a 64-wide step), and the
    m=2048, n=256, k=2048 attention-projection shape on which the pages'
    Metal tile returned -inf."""
    rng = si.rng_for(0, 5, M + N + K)
    W = si.q4_0_weights(rng, N, K)
    A = si.activations_bf16(rng, M, K)
    note(f"gemm_tiled M={M} N={N} K={K} variant {prefill_variant}")
    Wp = skg.pack_weights(skg.Q4_0_BF16, N, K, dev(W))
    y = poisoned((M, N))
    skg.gemm_tiled(skg.Q4_0_BF16, M, K, N, Wp, dev(A), y)
    yh = host(y)
    assert np.all(np.isfinite(yh))
    mrows = sample_rows(M, n=64, seed=7)
    y_ref, bound, _ = oracle.gemm_tiled_ref(W, A[mrows])
    assert_close(yh[mrows], y_ref, bound, f"tile M={M} N={N} K={K}")


@pytest.mark.parametrize("variant", [3, 4])
@pytest.mark.parametrize("M,N,K", [(512, 14336, 4096), (300, 250, 2080), (17, 129, 96), (2048, 256, 2048)])
def test_prefill_tile_q8_0(skg, variant, M, N, K):
    """The q8_0 weight tile (pipelined organisations), sampled at the
    M=512 workload size, with ragged tiles and a K tail."""
    rng = si.rng_for(0, 6, M + N + K)
    W = si.q8_0_weights(rng, N, K)
    A = si.activations_bf16(rng, M, K)
    note(f"gemm_tiled q8_0 M={M} N={N} K={K} variant {variant}")
    skg.gemm_tiled_set_variant(variant)
    try:
        Wp = skg.pack_weights(skg.Q8_0_BF16, N, K, dev(W))
        y = poisoned((M, N))
        skg.gemm_tiled(skg.Q8_0_BF16, M, K, N, Wp, dev(A), y)
        yh = host(y)
    finally:
        skg.gemm_tiled_set_variant(-1)
    assert np.all(np.isfinite(yh))
    mrows = sample_rows(M, n=32, seed=8)
    ncols = sample_rows(N, n=1024, seed=9) if N > 1024 else np.arange(N)
    y_ref, bound, y_b = oracle.gemm_tiled_ref(W[ncols], A[mrows], "q8_0")
    assert_close(yh[np.ix_(mrows, ncols)], y_ref, bound, "q8_0 tile vs exact weights")
    assert_close(yh[np.ix_(mrows, ncols)], y_b, bound, "q8_0 tile vs bf16 weights", rel=1e-4)


@pytest.mark.parametrize("variant", [3, 4])
@pytest.mark.parametrize("kind", ["q4_K", "q6_K"])
@pytest.mark.parametrize("M,N,K", [(512, 14336, 4096), (300, 250, 2304), (17, 129, 256), (2048, 256, 2048)])
def test_prefill_tile_kquant(skg, variant, kind, M, N, K):
    """q4_K / q6_K weight tiles (pipelined organisations), sampled at the
    M=512 workload size, with ragged tiles; the bf16-weight reference (each
    weight rounded through binary32 to bf16) bounds the remaining deviation
    to summation order."""
    fmt = skg.Q4_K_BF16 if kind == "q4_K" else skg.Q6_K_BF16
    rng = si.rng_for(0, 7, M + N + K + (kind == "q6_K"))
    W = si.weights(kind, rng, N, K)
    A = si.activations_bf16(rng, M, K)
    note(f"gemm_tiled {kind} M={M} N={N} K={K} variant {variant}")
    skg.gemm_tiled_set_variant(variant)
    try:
        Wp = skg.pack_weights(fmt, N, K, dev(W))
        y = poisoned((M, N))
        skg.gemm_tiled(fmt, M, K, N, Wp, dev(A), y)
        yh = host(y)
    finally:
        skg.gemm_tiled_set_variant(-1)
    assert np.all(np.isfinite(yh))
    mrows = sample_rows(M, n=32, seed=10)
    ncols = sample_rows(N, n=1024, seed=11) if N > 1024 else np.arange(N)
    y_ref, bound, y_b = oracle.gemm_tiled_ref(W[ncols], A[mrows], kind)
    assert_close(yh[np.ix_(mrows, ncols)], y_ref, bound, f"{kind} tile vs exact weights")
    assert_close(yh[np.ix_(mrows, ncols)], y_b, bound, f"{kind} tile vs bf16 weights", rel=1e-4)


@pytest.mark.parametrize("fmt", [3, 4])
@pytest.mark.parametrize("M,N,K", [(512, 14336, 4096), (300, 250, 2048), (17, 129, 64), (2048, 256, 2048),
                                   (257, 1000, 4160)])
def test_prefill_tile_q8_1_integer(skg, fmt, M, N, K):
    """The integer matrix-core tile (q4_0 / q8_0 weights x Q8_1 activation
    blocks): every block dot exact, then one binary32 scaling by dA dW per
    block, so the result stays within 2e-5 of sum|w a| of the exact product of
    the decoded operands (which fails if a block's scale, sign or code order
    were wrong); sampled at the M=512 workload size, ragged tiles."""
    kind = "q4_0" if fmt == skg.Q4_0_Q8_1 else "q8_0"
    rng = si.rng_for(0, 8, M + N + K + fmt)
    W = si.weights(kind, rng, N, K)
    x = si.activations_f32(rng, M, K)
    note(f"gemm_tiled Q8_1 {kind} M={M} N={N} K={K}")
    import torch
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    xq = skg.quantize_act_q8_1(dev(x))
    xq_ref = oracle.quantize_q8_1(x)
    assert np.array_equal(host(xq), xq_ref), "Q8_1 activation differs from the oracle"
    y = poisoned((M, N))
    skg.gemm_tiled(fmt, M, K, N, Wp, xq, y)
    yh = host(y)
    assert np.all(np.isfinite(yh))
    mrows = sample_rows(M, n=32, seed=12)
    ncols = sample_rows(N, n=1024, seed=13) if N > 1024 else np.arange(N)
    xs = xq_ref.reshape(M, K // 32, 36)[mrows]
    if fmt == skg.Q4_0_Q8_1:
        y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(W[ncols], xs)
    else:
        y_ref, bound = oracle.gemv_q8_0_q8_1_ref(W[ncols], xs)
    assert_close(yh[np.ix_(mrows, ncols)], y_ref, bound, f"Q8_1 tile {kind}", rel=2e-5)
    del torch
