"""Parity of the fused RMSNorm -> Q8_1 dispatch with the oracle (GPU).

xn is compared element by element with the float64 RMSNorm, within the
binary32 bound the oracle states.  xq must be bit-identical to the oracle's
Q8_1 quantiser applied to the xn the GPU stored: the integer decision is taken
from the same binary32 values on both sides.
"""

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

NORM_WORKLOAD = 6

# Several 1024-element chunks per thread and ragged tails (K not a multiple of
# 1024), one block (K = 32), the largest K, and a prefill-sized M.
SHAPES = [(1, 4096), (2, 4096), (8, 4096), (1, 11008), (3, 32), (1, 1056), (5, 2080), (2, 16384), (512, 4096)]


def _inputs(M, K, seed, outliers=False):
    rng = si.rng_for(seed, NORM_WORKLOAD, 0)
    x = si.activations_f32_outliers(rng, M, K) if outliers else si.activations_f32(rng, M, K)
    g = si.norm_gain_f32(si.rng_for(seed, NORM_WORKLOAD, 1), K)
    return x, g


def _check_xn(xn, x, g, eps, what):
    ref = oracle.rmsnorm(x, g, eps)
    tol = oracle.rmsnorm_tolerance(ref)
    err = np.abs(xn.astype(np.float64) - ref)
    bad = ~(err <= tol)
    if np.any(bad):
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"{what}: xn[{i}] = {xn[i]!r}, ref {ref[i]!r}, err/tol {err[i] / tol[i]:.3g}")


def _check_xq(xq, xn, what, x=None, g=None, eps=None):
    """Bit-exact against the quantiser of the stored xn (the stage check) and,
    when the inputs are given, valid Q8_1 of values within the norm's
    tolerance of the float64 reference (a check with no GPU value as oracle
    input)."""
    expect = oracle.quantize_q8_1(xn)
    if not np.array_equal(xq, expect):
        m, b = np.argwhere(np.any(xq != expect, axis=2))[0]
        raise AssertionError(f"{what}: Q8_1 block ({m}, {b}) differs from the quantiser of the stored xn")
    if x is not None:
        ref = oracle.rmsnorm(x, g, eps)
        bad = q8_1_violations(xq, ref, oracle.rmsnorm_tolerance(ref))
        assert not bad, f"{what}: " + "; ".join(bad[:3])


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("eps", [1e-5, 1e-6])
def test_rmsnorm_q8_1_parity(skg, M, K, eps):
    import torch
    x, g = _inputs(M, K, seed=M * 7 + K)
    note(f"rmsnorm_q8_1 M={M} K={K} eps={eps}")
    # One extra row in each output stays poisoned: nothing past M is written.
    xn_buf = poisoned((M + 1, K))
    xq_buf = poisoned((M + 1, K // 32, 36), dtype=torch.uint8)
    skg.rmsnorm_q8_1(dev(x), dev(g), eps, xn=xn_buf[:M], xq=xq_buf[:M])
    xn_all, xq_all = host(xn_buf), host(xq_buf)
    assert np.all(np.isnan(xn_all[M])) and np.all(xq_all[M] == 0xFF)
    xn, xq = xn_all[:M], xq_all[:M]
    _check_xn(xn, x, g, eps, f"M={M} K={K}")
    _check_xq(xq, xn, f"M={M} K={K}", x, g, eps)


def test_outlier_channels(skg):
    M, K = 4, 4096
    x, g = _inputs(M, K, seed=5, outliers=True)
    note("rmsnorm_q8_1 outlier channels")
    xn, xq = skg.rmsnorm_q8_1(dev(x), dev(g), 1e-5)
    xn, xq = host(xn), host(xq)
    _check_xn(xn, x, g, 1e-5, "outliers")
    _check_xq(xq, xn, "outliers", x, g, 1e-5)


def test_modes_and_repeats_give_identical_bits(skg):
    """xn-only, xq-only and both-output calls, a gain of None and of ones, and
    repeated calls all produce the same bits (one fixed reduction order)."""
    import torch
    M, K = 3, 11008
    x, g = _inputs(M, K, seed=9)
    xd, gd = dev(x), dev(g)
    note("rmsnorm_q8_1 output modes")
    xn_b, xq_b = skg.rmsnorm_q8_1(xd, gd, 1e-5)
    xn_o, none_q = skg.rmsnorm_q8_1(xd, gd, 1e-5, xq=None)
    none_n, xq_o = skg.rmsnorm_q8_1(xd, gd, 1e-5, xn=None)
    assert none_q is None and none_n is None
    xn_r, xq_r = skg.rmsnorm_q8_1(xd, gd, 1e-5)
    for a, b in ((xn_b, xn_o), (xn_b, xn_r)):
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))
    for a, b in ((xq_b, xq_o), (xq_b, xq_r)):
        assert np.array_equal(host(a), host(b))
    xn_1, xq_1 = skg.rmsnorm_q8_1(xd, None, 1e-5)
    xn_ones, xq_ones = skg.rmsnorm_q8_1(xd, torch.ones(K, dtype=torch.float32, device="cuda"), 1e-5)
    assert np.array_equal(host(xn_1).view(np.uint32), host(xn_ones).view(np.uint32))
    assert np.array_equal(host(xq_1), host(xq_ones))
    _check_xn(host(xn_1), x, None, 1e-5, "no gain")
    _check_xq(host(xq_1), host(xn_1), "no gain", x, None, 1e-5)


def test_degenerate_rows(skg):
    """An all-zero row (eps > 0) normalises to zeros and Q8_1 blocks with
    d = s = 0; a constant row gives g * c / sqrt(c^2 + eps)."""
    K = 1024
    x = np.zeros((3, K), dtype=np.float32)
    x[1] = np.float32(-2.0)
    x[2] = si.activations_f32(si.rng_for(1, NORM_WORKLOAD, 2), 1, K)[0]
    g = si.norm_gain_f32(si.rng_for(1, NORM_WORKLOAD, 3), K)
    note("rmsnorm_q8_1 degenerate rows")
    xn, xq = skg.rmsnorm_q8_1(dev(x), dev(g), 5.0)
    xn, xq = host(xn), host(xq)
    assert not np.any(xn[0]) and not np.any(xq[0])
    assert np.allclose(xn[1], g.astype(np.float64) * (-2.0 / 3.0), rtol=4e-6, atol=0)
    _check_xn(xn, x, g, 5.0, "degenerate rows")
    _check_xq(xq, xn, "degenerate rows", x, g, 5.0)


@pytest.mark.parametrize("scale", [2.0 ** -60, 2.0 ** 40])
def test_extreme_magnitudes_without_eps(skg, scale):
    """With eps = 0 the result does not depend on the scale of the row, down
    to squares near the binary32 normal range and up to sums near 2^100."""
    M, K = 2, 4096
    x, g = _inputs(M, K, seed=13)
    xs = (x * np.float32(scale)).astype(np.float32)
    note(f"rmsnorm_q8_1 scale {scale}")
    xn, xq = skg.rmsnorm_q8_1(dev(xs), dev(g), 0.0)
    xn, xq = host(xn), host(xq)
    _check_xn(xn, xs, g, 0.0, f"scale {scale}")
    _check_xq(xq, xn, f"scale {scale}", xs, g, 0.0)


def test_full_layer_with_fused_norms(skg):
    """Every weight product of a Llama-2-7B-shaped layer with both norms fused
    into Q8_1 producers: norm -> QKV; quantize(attention output) -> O;
    norm -> gate/up + SwiGLU with Q8_1 output -> down.  Each stage is checked
    on its own input: Q8_1 blocks bit-exactly against the quantiser of the
    values the GPU stored, products against the oracle's integer-dot reference
    on the GPU's blocks.  Attention and the residual adds are not part of the
    path; seeded stand-ins take their place."""
    D, F = 4096, 11008
    rng = si.rng_for(0, 3, 0)
    Wq, Wk, Wv, Wo = (si.q4_0_weights(rng, D, D) for _ in range(4))
    Wg, Wu = si.q4_0_weights(rng, F, D), si.q4_0_weights(rng, F, D)
    Wd = si.q4_0_weights(rng, D, F)
    x, g1 = _inputs(1, D, seed=17, outliers=True)
    x2, g2 = _inputs(1, D, seed=18)
    att = si.activations_f32(si.rng_for(19, NORM_WORKLOAD, 4), 1, D)
    fmt = skg.Q4_0_Q8_1
    note("full layer: pack")
    Pqkv = skg.pack_weights_multi(fmt, [D, D, D], D, [dev(Wq), dev(Wk), dev(Wv)])
    Po = skg.pack_weights(fmt, D, D, dev(Wo))
    Pgu = skg.pack_weights_multi(fmt, [F, F], D, [dev(Wg), dev(Wu)])
    Pd = skg.pack_weights(fmt, D, F, dev(Wd))
    rows = sample_rows(D, seed=21)
    frows = sample_rows(F, seed=22)

    note("full layer: attention norm -> qkv")
    xn, xq = skg.rmsnorm_q8_1(dev(x), dev(g1), 1e-5)
    xn_h, xq_h = host(xn), host(xq)
    _check_xn(xn_h, x, g1, 1e-5, "attention norm")
    _check_xq(xq_h, xn_h, "attention norm", x, g1, 1e-5)
    ys = [poisoned((1, D)) for _ in range(3)]
    skg.gemv_multi(fmt, 1, D, [D, D, D], Pqkv, xq, ys)
    for name, W, y in zip("qkv", (Wq, Wk, Wv), ys):
        y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(W[rows], xq_h)
        assert_close(host(y)[:, rows], y_ref, bound, f"{name} after fused norm")

    note("full layer: attention output projection")
    aq = skg.quantize_act_q8_1(dev(att))
    aq_ref = oracle.quantize_q8_1(att)
    assert np.array_equal(host(aq), aq_ref)
    yo = poisoned((1, D))
    skg.gemv(fmt, 1, D, D, Po, aq, yo)
    y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(Wo[rows], aq_ref)
    assert_close(host(yo)[:, rows], y_ref, bound, "O projection")

    note("full layer: feed-forward norm -> gate/up + SwiGLU (Q8_1 out)")
    xn2, xq2 = skg.rmsnorm_q8_1(dev(x2), dev(g2), 1e-5)
    xn2_h, xq2_h = host(xn2), host(xq2)
    _check_xn(xn2_h, x2, g2, 1e-5, "feed-forward norm")
    _check_xq(xq2_h, xn2_h, "feed-forward norm", x2, g2, 1e-5)
    h, hq = skg.gemv_multi(fmt, 1, D, [F, F], Pgu, xq2, epi=skg.EPI_SWIGLU_Q8_1)
    h_h, hq_h = host(h), host(hq)
    g_ref, _, bg = oracle.gemv_q4_0_q8_1_ref(Wg[frows], xq2_h)
    u_ref, _, bu = oracle.gemv_q4_0_q8_1_ref(Wu[frows], xq2_h)
    tol = oracle.swiglu_tolerance(g_ref, u_ref, oracle.tolerance(bg), oracle.tolerance(bu))
    ok, worst = oracle.check_close(h_h[:, frows], oracle.swiglu_ref(g_ref, u_ref), tol)
    assert ok, f"swiglu worst {worst}"
    assert np.array_equal(hq_h.reshape(1, F // 32, 36), oracle.quantize_q8_1(h_h))

    note("full layer: down projection")
    yd = poisoned((1, D))
    skg.gemv(fmt, 1, F, D, Pd, hq, yd)
    y_ref, _, bound = oracle.gemv_q4_0_q8_1_ref(Wd[rows], hq_h.reshape(1, F // 32, 36))
    assert_close(host(yd)[:, rows], y_ref, bound, "down projection")
