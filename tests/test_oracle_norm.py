"""Pins for the oracle's RMSNorm (CPU only).

The pages print no normalised values, so the definition is pinned by exact
hand-worked rows, closed forms, invariants that a dropped or misplaced term
breaks (unit mean square, scale invariance, odd symmetry, the role of eps and
of the gain) and a pure-Python evaluation on small rows.
"""

import math

import numpy as np
import pytest

import oracle

SQRT2 = math.sqrt(2.0)


def _row_34(K=32):
    x = np.zeros(K, dtype=np.float32)
    x[0], x[1] = 3.0, 4.0
    return x


def test_hand_worked_eps_completes_unit_mean_square():
    # mean(x^2) = 25/32 and eps = 7/32 give a denominator of exactly 1.
    xn = oracle.rmsnorm(_row_34(), eps=7.0 / 32.0)[0]
    assert xn[0] == 3.0 and xn[1] == 4.0 and not np.any(xn[2:])


def test_hand_worked_no_eps():
    # 1 / sqrt(25/32) = 4 sqrt(2) / 5.
    xn = oracle.rmsnorm(_row_34(), eps=0.0)[0]
    assert xn[0] == pytest.approx(12 * SQRT2 / 5, rel=1e-15)
    assert xn[1] == pytest.approx(16 * SQRT2 / 5, rel=1e-15)
    assert not np.any(xn[2:])


def test_hand_worked_gain():
    g = np.ones(32, dtype=np.float32)
    g[0], g[1], g[5] = 2.0, -0.5, 0.0
    xn = oracle.rmsnorm(_row_34(), g=g, eps=0.0)[0]
    assert xn[0] == pytest.approx(24 * SQRT2 / 5, rel=1e-15)
    assert xn[1] == pytest.approx(-8 * SQRT2 / 5, rel=1e-15)


@pytest.mark.parametrize("c,eps,expect", [
    (2.0 ** -10, 2.0 ** -20, 1 / SQRT2),   # c^2 == eps
    (-2.0, 5.0, -2.0 / 3.0),              # sqrt(4 + 5) = 3
    (0.0, 1e-5, 0.0),                     # a zero row stays zero when eps > 0
])
def test_constant_row_closed_form(c, eps, expect):
    x = np.full(64, c, dtype=np.float32)
    xn = oracle.rmsnorm(x, eps=eps)[0]
    assert np.allclose(xn, expect, rtol=1e-14, atol=0)


def test_unit_mean_square_without_eps():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 4096)).astype(np.float32) * np.float32(7.5)
    xn = oracle.rmsnorm(x, eps=0.0)
    assert np.allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-13, atol=0)


def test_scale_invariance_and_odd_symmetry():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 1024)).astype(np.float32)
    ref = oracle.rmsnorm(x, eps=0.0)
    for a in (2.0 ** -20, 8.0, 2.0 ** 30):   # powers of two scale binary32 inputs exactly
        xa = (x * np.float32(a)).astype(np.float32)
        assert np.allclose(oracle.rmsnorm(xa, eps=0.0), ref, rtol=1e-14, atol=0)
    assert np.array_equal(oracle.rmsnorm(-x, eps=0.0), -ref)


def test_gain_multiplies_each_channel():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    plain = oracle.rmsnorm(x, eps=1e-5)
    assert np.array_equal(oracle.rmsnorm(x, g=g, eps=1e-5), plain * g.astype(np.float64))


def test_rows_are_independent():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    whole = oracle.rmsnorm(x, eps=1e-6)
    for m in range(5):
        assert np.array_equal(oracle.rmsnorm(x[m], eps=1e-6)[0], whole[m])


def test_pure_python_rows():
    rng = np.random.default_rng(15)
    for K in (32, 64, 96):
        x = rng.standard_normal(K).astype(np.float32)
        g = rng.standard_normal(K).astype(np.float32)
        eps = float(np.float32(1e-5))
        xs = [float(v) for v in x]
        den = math.sqrt(math.fsum(v * v for v in xs) / K + eps)
        expect = [float(gk) * v / den for v, gk in zip(xs, g)]
        got = oracle.rmsnorm(x, g=g, eps=1e-5)[0]
        assert np.allclose(got, expect, rtol=1e-14, atol=1e-300)


def test_tolerance_rejects_a_slipped_divisor():
    # Dividing the sum of squares by K - 1 instead of K moves every element by
    # about 1/(2K) relatively, far outside the binary32 bound.
    rng = np.random.default_rng(16)
    x = rng.standard_normal((1, 4096)).astype(np.float32)
    ref = oracle.rmsnorm(x, eps=1e-5)
    x64 = x.astype(np.float64)
    slip = x64 / np.sqrt(np.sum(x64 * x64) / 4095 + np.float64(np.float32(1e-5)))
    assert np.any(np.abs(slip - ref) > oracle.rmsnorm_tolerance(ref))
    # ... and the same for eps added outside the square root.
    eps = np.float64(np.float32(1e-2))
    y = (x * np.float32(0.05)).astype(np.float32)
    ref_y = oracle.rmsnorm(y, eps=1e-2)
    y64 = y.astype(np.float64)
    outside = y64 / (np.sqrt(np.mean(y64 * y64)) + eps)
    assert np.any(np.abs(outside - ref_y) > oracle.rmsnorm_tolerance(ref_y))


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        oracle.rmsnorm(np.zeros(32, dtype=np.float32), eps=0.0)
    with pytest.raises(ValueError):
        oracle.rmsnorm(np.ones(32, dtype=np.float32), eps=-1.0)
    x = np.ones(32, dtype=np.float32)
    x[3] = np.inf
    with pytest.raises(ValueError):
        oracle.rmsnorm(x)


def test_q8_1_validity_check_accepts_the_quantiser_and_rejects_slips():
    """The no-GPU-input Q8_1 check used on the fused norm: it accepts the
    oracle's quantisation of the binary32-rounded reference and rejects a code
    moved by one, a wrong block sum and a block that misses the full range."""
    from tests._q8_1_check import q8_1_violations
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 1024)).astype(np.float32)
    g = (1 + 0.25 * rng.standard_normal(1024)).astype(np.float32)
    ref = oracle.rmsnorm(x, g, 1e-5)
    tol = oracle.rmsnorm_tolerance(ref)
    xq = oracle.quantize_q8_1(ref.astype(np.float32))
    assert q8_1_violations(xq, ref, tol) == []
    # one code moved by one: pick the element with the smallest residual
    d, _, q = oracle.q8_1_fields(xq)
    resid = np.abs(d[..., None] * q - ref.reshape(3, 32, 32))
    m, b, i = np.unravel_index(np.argmin(np.where(np.abs(q) < 120, resid, np.inf)), resid.shape)
    bad = xq.copy()
    bad[m, b, 4 + i] = np.uint8((int(q[m, b, i]) + 1) & 0xFF)
    assert q8_1_violations(bad, ref, tol)
    # block sum off by a few fp16 ulps
    bad = xq.copy()
    s = int(bad[1, 5, 2]) | (int(bad[1, 5, 3]) << 8)
    s += 8
    bad[1, 5, 2], bad[1, 5, 3] = s & 0xFF, s >> 8
    assert q8_1_violations(bad, ref, tol)
    # a block whose codes were all halved (scale doubled) misses the full range
    bad = xq.copy()
    qq = bad[2, 7, 4:].view(np.int8).astype(int) // 2
    bad[2, 7, 4:] = (qq & 0xFF).astype(np.uint8)
    assert q8_1_violations(bad, ref, tol)
