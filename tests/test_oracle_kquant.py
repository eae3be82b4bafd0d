"""Pins for the oracle's K-quant super-block decoders (q4_K, q6_K), CPU only:
hand-worked blocks (tests/golden/), a byte-by-byte exact decoder written the
other way round (walking code bytes, not elements), closed forms that reduce
a super-block to a plain per-block code, and exact rational GEMVs."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import kquant
from synth import inputs as si
from tests import _exact as ex

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, f"{name}_blocks.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("kind", ["q4_K", "q6_K"])
def test_golden_blocks(kind):
    g = _golden(kind)
    assert g["cite"]
    for b in g["blocks"]:
        raw = bytes.fromhex(b["hex"])
        B = np.frombuffer(raw, np.uint8).reshape(1, 1, -1)
        w = oracle.dequantize(kind, B)[0]
        for k, v in b["values"].items():
            assert w[int(k)] == float(Fraction(v)), (kind, k)
        if kind == "q4_K":
            _, _, sc, m = kquant.q4_K_scales_mins(B[0, 0])
            assert sc.tolist() == b["scales"] and m.tolist() == b["mins"]
            assert ex.q4_K_block_scales_mins(raw) == (b["scales"], b["mins"])
        exact = ex.q4_K_block_values(raw) if kind == "q4_K" else ex.q6_K_block_values(raw)
        for k, v in b["values"].items():
            assert exact[int(k)] == Fraction(v), (kind, k)


@pytest.mark.parametrize("kind", ["q4_K", "q6_K"])
def test_decode_equals_byte_walk_on_random_blocks(kind):
    """Every element of random super-blocks (all scale bytes, all code bytes
    random) against the independent byte-by-byte decoder."""
    rng = si.rng_for(0, 99, 30 + (kind == "q6_K"))
    W = si.weights(kind, rng, 3, 512)
    Wd = oracle.dequantize(kind, W)
    assert Wd.shape == (3, 512)
    for n in range(3):
        vals = ex.row_values(kind, W[n].tobytes(), 512)
        assert [Fraction(float(v)) for v in Wd[n]] == vals


def test_q4_K_unit_scales_give_the_codes():
    """d = 1, dmin = 0, every sc = 1: w = q, the codes in element order
    (element 64c + i is the low nibble of byte 32c + i, 64c + 32 + i its high
    nibble), checked on a ramp of code bytes."""
    B = np.zeros((1, 1, 144), np.uint8)
    B[..., 0:2] = [0x00, 0x3C]
    sc = [1] * 8
    m = [0] * 8
    s = bytearray(12)
    for j in range(4):
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = m[j] | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    B[0, 0, 4:16] = np.frombuffer(bytes(s), np.uint8)
    B[0, 0, 16:] = (np.arange(128) * 3 % 256).astype(np.uint8)
    w = oracle.dequantize("q4_K", B)[0]
    qs = B[0, 0, 16:].astype(int)
    for c in range(4):
        for i in range(32):
            assert w[64 * c + i] == qs[32 * c + i] & 15
            assert w[64 * c + 32 + i] == qs[32 * c + i] >> 4


def test_q4_K_min_is_subtracted_per_sub_block():
    """All codes 0: w = -dmin m_j, constant on each 32-element sub-block."""
    B = np.zeros((1, 1, 144), np.uint8)
    B[..., 0:2] = [0x00, 0x3C]          # d = 1
    B[..., 2:4] = [0x00, 0x40]          # dmin = 2
    mins = [5, 6, 7, 8, 33, 34, 63, 16]
    s = bytearray(12)
    for j in range(4):
        s[j + 4] = mins[j] | ((mins[j + 4] >> 4) << 6)
        s[j + 8] = (mins[j + 4] & 15) << 4
    B[0, 0, 4:16] = np.frombuffer(bytes(s), np.uint8)
    w = oracle.dequantize("q4_K", B)[0].reshape(8, 32)
    for j in range(8):
        assert np.all(w[j] == -2.0 * mins[j])


def test_q6_K_unit_scale_gives_codes_minus_32():
    """d = 1, every scale 1: w = q - 32 with q's low bits from ql and high
    bits from qh; a single set high-bit pair moves exactly one element by 16,
    32 or 48."""
    B = np.zeros((1, 1, 210), np.uint8)
    B[0, 0, 192:208] = 1
    B[0, 0, 208:210] = [0x00, 0x3C]
    w = oracle.dequantize("q6_K", B)[0]
    assert np.all(w == -32.0)
    for (byte, val, elem, delta) in ((128 + 5, 0b01, 5, 16), (128 + 5, 0b10 << 2, 37, 32),
                                     (128 + 40, 0b11 << 6, 128 + 8 + 96, 48), (128 + 63, 0b01 << 4, 255 - 32, 16)):
        C = B.copy()
        C[0, 0, byte] = val
        wc = oracle.dequantize("q6_K", C)[0]
        changed = np.nonzero(wc != w)[0]
        assert changed.tolist() == [elem] and wc[elem] == -32.0 + delta


@pytest.mark.parametrize("kind", ["q4_K", "q6_K"])
def test_kquant_gemv_exact_rational(kind):
    rng = si.rng_for(0, 99, 40 + (kind == "q6_K"))
    N, K, M = 2, 512, 2
    W = si.weights(kind, rng, N, K)
    x = si.activations_f32(rng, M, K)
    y, bound = oracle.gemv_ref_fmt(kind, W, x)
    for m in range(M):
        xv = [ex.f32_value(float(v)) for v in x[m]]
        for n in range(N):
            row = ex.row_values(kind, W[n].tobytes(), K)
            ye = sum(r * a for r, a in zip(row, xv))
            be = sum(abs(r * a) for r, a in zip(row, xv))
            assert abs(float(ye) - y[m, n]) <= 1e-13 * float(be) + 1e-300
            assert abs(float(be) - bound[m, n]) <= 1e-13 * float(be) + 1e-300


@pytest.mark.parametrize("kind", ["q4_K", "q6_K"])
def test_kquant_one_hot_and_linearity(kind):
    rng = si.rng_for(0, 99, 50 + (kind == "q6_K"))
    W = si.weights(kind, rng, 5, 256)
    Wd = oracle.dequantize(kind, W)
    for k in (0, 31, 32, 100, 255):
        x = np.zeros((1, 256), np.float32)
        x[0, k] = 1.0
        y, _ = oracle.gemv_ref_fmt(kind, W, x)
        assert np.array_equal(y[0], Wd[:, k])
    a, b = si.activations_f32(rng, 1, 256), si.activations_f32(rng, 1, 256)
    ya, ba = oracle.gemv_ref_fmt(kind, W, a)
    yb, bb = oracle.gemv_ref_fmt(kind, W, b)
    yab, _ = oracle.gemv_ref_fmt(kind, W, (a.astype(np.float64) + b).astype(np.float32))
    assert np.all(np.abs(yab - (ya + yb)) <= 1e-6 * (ba + bb) + 1e-12)


def test_kquant_block_sizes():
    """144 and 210 bytes per 256 elements: 4.5 and 6.5625 bits per weight."""
    assert kquant.Q4_K_BLOCK_BYTES * 8 / kquant.QK_K == 4.5
    assert kquant.Q6_K_BLOCK_BYTES * 8 / kquant.QK_K == 6.5625
    for kind, nbytes in (("q4_K", 144), ("q6_K", 210)):
        assert si.weights(kind, si.rng_for(0, 99, 60), 3, 768).shape == (3, 3, nbytes)


@pytest.mark.parametrize("kind", ["q4_K", "q6_K"])
def test_tile_bf16_weight_reference_rounds_through_binary32(kind):
    """y_bf16w of the tile reference for K-quant weights: each decoded weight
    rounded to binary32 (nearest-even) and then to bf16 (nearest-even), exact
    rational products.  The q4_K row 0 is built so the two roundings differ
    from one: w = (1 + 2^-8) - (-2^-24) = 1 + 2^-8 + 2^-24 lies half a binary32
    ulp above 1 + 2^-8, which rounds to even (1 + 2^-8), a bf16 tie that
    rounds to even again: 1, where rounding the exact value once would give
    1 + 2^-7."""
    rng = si.rng_for(0, 99, 70 + (kind == "q6_K"))
    M, N, K = 2, 4, 256
    W = si.weights(kind, rng, N, K)
    if kind == "q4_K":
        W[0, 0, 0:2] = [0x04, 0x3C]          # d = 1 + 2^-8
        W[0, 0, 2:4] = [0x01, 0x80]          # dmin = -2^-24 (smallest subnormal, negative)
        W[0, 0, 4] = (W[0, 0, 4] & 0xC0) | 1     # sc_0 = 1
        W[0, 0, 8] = (W[0, 0, 8] & 0xC0) | 1     # m_0 = 1
        W[0, 0, 16] = (W[0, 0, 16] & 0xF0) | 1   # element 0: code 1
    A = si.activations_bf16(rng, M, K)
    _, _, y_b = oracle.gemm_tiled_ref(W, A, kind)
    for n in range(N):
        vals = ex.row_values(kind, W[n].tobytes(), K)
        wr = [ex.round_binary(ex.round_binary(v, ex.F32), (8, -126)) for v in vals]
        if kind == "q4_K" and n == 0:
            assert vals[0] == 1 + Fraction(1, 256) + Fraction(1, 2 ** 24)
            assert ex.round_binary(vals[0], (8, -126)) == 1 + Fraction(1, 128)
            assert wr[0] == 1
        for m in range(M):
            av = [ex.bf16_value(int(v)) for v in A[m]]
            ye = sum(w * a for w, a in zip(wr, av))
            be = sum(abs(w * a) for w, a in zip(wr, av))
            assert abs(float(ye) - y_b[m, n]) <= 1e-13 * float(be) + 1e-300, (m, n)
