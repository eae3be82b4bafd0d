"""Pins for the oracle's products (CPU only): exact rational brute force on tiny
shapes, closed forms, and consistency between the integer-dot and float forms."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import inputs as si
from tests import _exact as ex


def _exact_gemv(kind, W, x_vals, N, K):
    rows = [ex.row_values(kind, W[n].tobytes(), K) for n in range(N)]
    y = [[sum(r[k] * xm[k] for k in range(K)) for r in rows] for xm in x_vals]
    b = [[sum(abs(r[k] * xm[k]) for k in range(K)) for r in rows] for xm in x_vals]
    return y, b


@pytest.mark.parametrize("kind", ["bf16", "q8_0", "q4_0"])
@pytest.mark.parametrize("N,K,M", [(1, 32, 1), (3, 64, 2), (2, 128, 1), (3, 96, 2)])
def test_gemv_equals_exact_rational_sum(kind, N, K, M):
    rng = si.rng_for(0, 99, N * 1000 + K + M)
    W = si.weights(kind, rng, N, K)
    x = si.activations_f32(rng, M, K)
    y, bound = oracle.gemv_ref_fmt(kind, W, x)
    assert y.shape == (M, N)
    xv = [[ex.f32_value(float(v)) for v in x[m]] for m in range(M)]
    ye, be = _exact_gemv(kind, W, xv, N, K)
    for m in range(M):
        for n in range(N):
            scale = float(be[m][n]) + 1e-300
            assert abs(float(ye[m][n]) - y[m, n]) <= 1e-13 * scale
            assert abs(float(be[m][n]) - bound[m, n]) <= 1e-13 * scale


def test_gemv_bf16_activations_are_decoded():
    rng = si.rng_for(0, 99, 5)
    W = si.bf16_weights(rng, 3, 64)
    xb = si.activations_bf16(rng, 1, 64)
    y, _ = oracle.gemv_ref_fmt("bf16", W, xb, x_kind="bf16")
    xv = [[ex.bf16_value(int(v)) for v in xb[0]]]
    ye, _ = _exact_gemv("bf16", W, xv, 3, 64)
    for n in range(3):
        assert abs(float(ye[0][n]) - y[0, n]) <= 1e-13 * abs(float(ye[0][n])) + 1e-300


@pytest.mark.parametrize("kind", ["bf16", "q8_0", "q4_0"])
def test_one_hot_activation_selects_a_column(kind):
    rng = si.rng_for(0, 99, 6)
    N, K = 5, 128
    W = si.weights(kind, rng, N, K)
    Wd = oracle.dequantize(kind, W)
    for k in [0, 17, 31, 32, 127]:
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y, _ = oracle.gemv_ref_fmt(kind, W, x)
        assert np.array_equal(y[0], Wd[:, k])


def test_q4_0_all_codes_eight_gives_zero():
    W = si.q4_0_weights(si.rng_for(0, 99, 7), 4, 256)
    W[..., 2:] = 0x88
    x = si.activations_f32(si.rng_for(0, 99, 8), 2, 256)
    y, _ = oracle.gemv_ref_fmt("q4_0", W, x)
    assert np.all(y == 0)


def test_constant_blocks_closed_form():
    # q8_0 row with every code 3 and every scale 0.25 against x = 1: y = K * 0.75
    N, K = 3, 256
    W = np.zeros((N, K // 32, 34), dtype=np.uint8)
    W[..., 0:2] = [0x00, 0x34]    # 0.25
    W[..., 2:] = 3
    y, _ = oracle.gemv_ref_fmt("q8_0", W, np.ones((1, K), np.float32))
    assert np.all(y == K * 0.75)
    # q4_0 row with codes 10 (value 2d), scale 0.5 against x = 1: y = K * 1.0
    W4 = np.zeros((N, K // 32, 18), dtype=np.uint8)
    W4[..., 0:2] = [0x00, 0x38]
    W4[..., 2:] = 0xAA
    y4, _ = oracle.gemv_ref_fmt("q4_0", W4, np.ones((1, K), np.float32))
    assert np.all(y4 == K * 1.0)


def test_gemv_orientation_non_square():
    # W is N x K and y = W x: a 2 x 64 matrix with a single 1 at (1, 40)
    W = np.zeros((2, 64), dtype=np.uint16)
    W[1, 40] = 0x3F80
    x = np.arange(64, dtype=np.float32)[None, :]
    y, _ = oracle.gemv_ref_fmt("bf16", W, x)
    assert y.shape == (1, 2) and y[0, 0] == 0 and y[0, 1] == 40.0


def test_linearity_in_activation():
    rng = si.rng_for(0, 99, 9)
    W = si.q4_0_weights(rng, 8, 256)
    a = si.activations_f32(rng, 1, 256)
    b = si.activations_f32(rng, 1, 256)
    ya, ba = oracle.gemv_ref_fmt("q4_0", W, a)
    yb, bb = oracle.gemv_ref_fmt("q4_0", W, b)
    yab, _ = oracle.gemv_ref_fmt("q4_0", W, (a.astype(np.float64) + b).astype(np.float32))
    assert np.all(np.abs(yab - (ya + yb)) <= 1e-6 * (ba + bb) + 1e-9)


def test_block_dots_q4_0_q8_1_brute_force():
    rng = si.rng_for(0, 99, 10)
    N, K = 3, 128
    W = si.q4_0_weights(rng, N, K)
    xq = oracle.quantize_q8_1(si.activations_f32(rng, 1, K))[0]
    dots = oracle.block_dots_q4_0_q8_1(W, xq)
    for n in range(N):
        for b in range(K // 32):
            codes = ex.q4_0_block_codes(W[n, b].tobytes())
            _, _, qa = ex.q8_1_block_fields(xq[b].tobytes())
            assert dots[n, b] == sum(c * a for c, a in zip(codes, qa))
    # the ramp block against all-ones codes: sum of 0..15 twice
    blk = np.frombuffer(bytes.fromhex("00bcf0e1d2c3b4a5968778695a4b3c2d1e0f"), np.uint8).reshape(1, 1, 18)
    ones = np.zeros((1, 36), np.uint8)
    ones[0, 4:] = 1
    assert oracle.block_dots_q4_0_q8_1(blk, ones)[0, 0] == 240


def test_block_dots_q8_0_q8_1_brute_force():
    rng = si.rng_for(0, 99, 11)
    W = si.q8_0_weights(rng, 2, 64)
    xq = oracle.quantize_q8_1(si.activations_f32(rng, 1, 64))[0]
    dots = oracle.block_dots_q8_0_q8_1(W, xq)
    for n in range(2):
        for b in range(2):
            qw = [ex.int8(v) for v in W[n, b, 2:]]
            _, _, qa = ex.q8_1_block_fields(xq[b].tobytes())
            assert dots[n, b] == sum(c * a for c, a in zip(qw, qa))


def test_q4_0_q8_1_reference_is_the_decoded_dot():
    rng = si.rng_for(0, 99, 12)
    N, K, M = 16, 512, 2
    W = si.q4_0_weights(rng, N, K)
    xq = oracle.quantize_q8_1(si.activations_f32(rng, M, K))
    y, y_s, bound = oracle.gemv_q4_0_q8_1_ref(W, xq)
    y2, b2 = oracle.gemv_ref(oracle.decode_q4_0(W), oracle.decode_q8_1(xq))
    assert np.allclose(y, y2, rtol=0, atol=1e-12 * np.max(b2))
    assert np.allclose(bound, b2, rtol=1e-14)
    # the stored block sum differs from d*sum(q) only by its fp16 rounding
    assert np.all(np.abs(y - y_s) <= 2e-3 * bound)
    # exact rational check on one row
    n = 5
    row = ex.row_values("q4_0", W[n].tobytes(), K)
    d, s, q = [], [], []
    acts = []
    for b in range(K // 32):
        db, sb, qb = ex.q8_1_block_fields(xq[0, b].tobytes())
        acts += [db * v for v in qb]
    assert abs(float(sum(r * a for r, a in zip(row, acts))) - y[0, n]) <= 1e-13 * bound[0, n]


def test_q4_0_q8_1_second_reference_on_adversarial_blocks():
    # all codes 8: the decoded dot is 0, only the -8*s term of y_ref_s remains
    N, K = 2, 64
    W = np.zeros((N, K // 32, 18), np.uint8)
    W[..., 0:2] = [0x00, 0x3C]
    W[..., 2:] = 0x88
    xq = oracle.quantize_q8_1(si.activations_f32(si.rng_for(0, 99, 13), 1, K))
    y, y_s, _ = oracle.gemv_q4_0_q8_1_ref(W, xq)
    assert np.all(y == 0)
    d, s, q = oracle.q8_1_fields(xq[0])
    expect_s = np.sum(d * q.sum(axis=-1) * 8 - 8 * s)   # dW = 1: dA*sum(code*qa) = 8 dA sum qa
    assert np.allclose(y_s[0], expect_s, rtol=1e-12, atol=1e-15)


def test_silu_and_swiglu():
    z = np.array([0.0, 1.0, -1.0, 20.0, -40.0, 3.5])
    ref = [v / (1 + math.exp(-v)) for v in z]
    assert np.allclose(oracle.silu(z), ref, rtol=1e-15, atol=0)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([50.0]))[0] - 50.0) < 1e-15 * 50
    g = np.array([1.0, -2.0, 0.0])
    u = np.array([2.0, 3.0, 5.0])
    h = oracle.swiglu_ref(g, u)
    assert np.allclose(h, [2 / (1 + math.exp(-1)), 3 * -2 / (1 + math.exp(2)), 0.0], rtol=1e-15)
    # Lipschitz constant of silu is below 1.1
    zz = np.linspace(-20, 20, 200001)
    deriv = np.gradient(oracle.silu(zz), zz)
    assert np.max(np.abs(deriv)) < oracle.gemv.SILU_LIPSCHITZ


def test_swiglu_tolerance_covers_perturbed_inputs():
    rng = np.random.default_rng(4)
    g = rng.normal(0, 3, 1000)
    u = rng.normal(0, 3, 1000)
    tg = np.abs(rng.normal(0, 1e-3, 1000))
    tu = np.abs(rng.normal(0, 1e-3, 1000))
    gp = g + tg * rng.choice([-1, 1], 1000)
    up = u + tu * rng.choice([-1, 1], 1000)
    err = np.abs(oracle.swiglu_ref(gp, up) - oracle.swiglu_ref(g, u))
    assert np.all(err <= oracle.swiglu_tolerance(g, u, tg, tu))


@pytest.mark.parametrize("kind", ["q4_0", "q8_0"])
def test_gemm_tiled_reference_brute_force_tile(kind):
    rng = si.rng_for(0, 99, 14)
    M, N, K = 64, 64, 64
    W = si.weights(kind, rng, N, K)
    A = si.activations_bf16(rng, M, K)
    y, bound, y_b = oracle.gemm_tiled_ref(W, A, kind)
    Wd = [[float(v) for v in ex.row_values(kind, W[n].tobytes(), K)] for n in range(N)]
    Ad = [[float(ex.bf16_value(int(v))) for v in A[m]] for m in range(M)]
    for m in range(0, M, 7):
        for n in range(N):
            yy = math.fsum(Wd[n][k] * Ad[m][k] for k in range(K))
            assert abs(yy - y[m, n]) <= 1e-13 * bound[m, n] + 1e-300
    # bf16-rounded weights stay within the bf16 unit roundoff of the exact product
    assert np.all(np.abs(y_b - y) <= 2.0**-8 * bound + 1e-30)


def test_tolerance_helpers():
    ok, worst = oracle.check_close([1.0, 2.0], [1.0, 2.001], oracle.tolerance(np.array([1.0, 1.0])))
    assert ok and worst <= 1.0
    ok, _ = oracle.check_close([1.0], [1.01], oracle.tolerance(np.array([1.0])))
    assert not ok
    ok, _ = oracle.check_close([np.nan], [0.0], oracle.tolerance(np.array([1.0])))
    assert not ok


BF16 = (8, -126)   # significand bits incl. the hidden bit, minimum normal exponent


@pytest.mark.parametrize("N,K,M", [(3, 96, 2), (2, 64, 1)])
def test_q8_0_q8_1_reference_exact_rational(N, K, M):
    """gemv_q8_0_q8_1_ref against exact rational sums of the decoded
    operands: q8_0 values d*q from the block bytes, Q8_1 values dA*qa from the
    activation block bytes, multiplied and summed as Fractions."""
    rng = si.rng_for(0, 99, 15 + N + K)
    W = si.q8_0_weights(rng, N, K)
    xq = oracle.quantize_q8_1(si.activations_f32(rng, M, K))
    y, bound = oracle.gemv_q8_0_q8_1_ref(W, xq)
    assert y.shape == (M, N) and bound.shape == (M, N)
    for m in range(M):
        acts = []
        for b in range(K // 32):
            dA, _, qa = ex.q8_1_block_fields(xq[m, b].tobytes())
            acts += [dA * v for v in qa]
        for n in range(N):
            row = ex.row_values("q8_0", W[n].tobytes(), K)
            ye = sum(r * a for r, a in zip(row, acts))
            be = sum(abs(r * a) for r, a in zip(row, acts))
            assert abs(float(ye) - y[m, n]) <= 1e-13 * float(be) + 1e-300
            assert abs(float(be) - bound[m, n]) <= 1e-13 * float(be) + 1e-300


def test_q8_0_q8_1_reference_hand_block():
    """One hand-worked block pair: weights d=0.5 with codes 1..32, activation
    d=0.25 with codes all 2 (block sum irrelevant to the decoded dot):
    y = 0.5 * 0.25 * 2 * (1 + ... + 32) = 0.25 * 528 = 132."""
    W = np.zeros((1, 1, 34), np.uint8)
    W[0, 0, 0:2] = [0x00, 0x38]                      # fp16 0.5
    W[0, 0, 2:] = np.arange(1, 33, dtype=np.uint8)
    xq = np.zeros((1, 1, 36), np.uint8)
    xq[0, 0, 0:2] = [0x00, 0x34]                     # fp16 0.25
    xq[0, 0, 4:] = 2
    y, bound = oracle.gemv_q8_0_q8_1_ref(W, xq)
    assert y[0, 0] == 132.0 and bound[0, 0] == 132.0
    xq[0, 0, 4:] = np.uint8(0xFE)                    # codes -2: the sign flips
    y, bound = oracle.gemv_q8_0_q8_1_ref(W, xq)
    assert y[0, 0] == -132.0 and bound[0, 0] == 132.0


@pytest.mark.parametrize("kind", ["q4_0", "q8_0"])
def test_gemm_tiled_bf16_weight_reference_exact(kind):
    """y_bf16w of gemm_tiled_ref: every decoded weight rounded to bf16 by
    exact integer arithmetic (nearest, ties to even), then the exact rational
    product; a truncating or ties-away rounding fails the tie rows below."""
    rng = si.rng_for(0, 99, 16)
    M, N, K = 3, 6, 64
    W = si.weights(kind, rng, N, K)
    # rows whose decoded weights sit exactly halfway between two bf16 values
    # (both tie directions), one that rounds up into the next binade and one
    # that rounds down; the other rows keep their random blocks
    half = {"q4_0": (18, 9), "q8_0": (34, 1)}[kind]
    blk, code = half
    for n, dbits in ((0, 0x3C04), (1, 0x3C0C), (2, 0x3FFF), (3, 0x3C01)):
        W[n, :, 0] = dbits & 0xFF
        W[n, :, 1] = dbits >> 8
        if kind == "q4_0":
            W[n, :, 2:] = 0x99 if n < 3 else W[n, :, 2:]   # codes 9: w = d
        else:
            W[n, :, 2:] = code if n < 3 else W[n, :, 2:]   # codes 1: w = d
    assert W.shape[-1] == blk
    A = si.activations_bf16(rng, M, K)
    _, _, y_b = oracle.gemm_tiled_ref(W, A, kind)
    for n in range(N):
        wr = [ex.round_binary(v, BF16) for v in ex.row_values(kind, W[n].tobytes(), K)]
        if n == 0:   # d = 1 + 2^-8: halfway between 1 and 1 + 2^-7; the even one is 1
            assert wr[0] == 1
        if n == 1:   # d = 1 + 3*2^-8: halfway between 1 + 2^-7 and 1 + 2^-6; the even one is 1 + 2^-6
            assert wr[0] == 1 + Fraction(1, 64)
        if n == 2:   # d = 2 - 2^-10 rounds up into the next binade
            assert wr[0] == 2
        for m in range(M):
            av = [ex.bf16_value(int(v)) for v in A[m]]
            ye = sum(w * a for w, a in zip(wr, av))
            be = sum(abs(w * a) for w, a in zip(wr, av))
            assert abs(float(ye) - y_b[m, n]) <= 1e-13 * float(be) + 1e-300, (m, n)
