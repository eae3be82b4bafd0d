"""Pins for the oracle's format decoders (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import _exact as ex


def _block(hexstr):
    return np.frombuffer(bytes.fromhex(hexstr.replace(" ", "")), dtype=np.uint8)


def test_fp16_decoder_matches_ieee_binary16_for_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 10) & 0x1F) != 31
    bits = bits[finite]
    ours = oracle.fp16_bits_to_f64(bits)
    lib = bits.view(np.float16).astype(np.float64)           # numpy's binary16
    assert np.array_equal(ours, lib)
    # and a few by exact definition
    for b in [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0x3555, 0x2E66]:
        assert Fraction(float(oracle.fp16_bits_to_f64(np.uint16(b)))) == ex.f16_value(b)


def test_fp16_decoder_rejects_inf_nan():
    with pytest.raises(ValueError):
        oracle.fp16_bits_to_f64(np.array([0x7C00], dtype=np.uint16))


def test_bf16_decoder_constants_and_exhaustive():
    for bits, val in [(0x3F80, 1.0), (0xC040, -3.0), (0x0000, 0.0), (0x8000, -0.0),
                      (0x3F00, 0.5), (0x4049, 3.140625), (0x0001, 2.0**-133)]:
        assert oracle.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0] == val
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    ours = oracle.bf16_bits_to_f64(bits)
    sample = bits[::97]
    for b, v in zip(sample, ours[::97]):
        assert Fraction(float(v)) == ex.bf16_value(int(b))


def test_q4_0_golden_blocks(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "q4_0_blocks.json")))
    for blk in g["blocks"]:
        b = _block(blk["hex"])
        vals = oracle.decode_q4_0(b.reshape(1, 1, 18))[0]
        if "values_all" in blk:
            expect = [Fraction(v) for v in blk["values_all"]]
        else:
            expect = [Fraction(blk["others"])] * 32
            for k, v in blk["values"].items():
                expect[int(k)] = Fraction(v)
        assert [Fraction(float(v)) for v in vals] == expect, blk["name"]
    # the worked one-block dot product
    b = _block(g["blocks"][g["dot"]["block"]]["hex"]).reshape(1, 1, 18)
    x = np.arange(1, 33, dtype=np.float32)[None, :]
    y, _ = oracle.gemv_ref_fmt("q4_0", b, x)
    assert Fraction(float(y[0, 0])) == Fraction(g["dot"]["y"])


def test_q8_0_golden_blocks(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "q8_0_blocks.json")))
    for blk in g["blocks"]:
        b = _block(blk["hex"])
        vals = oracle.decode_q8_0(b.reshape(1, 1, 34))[0]
        expect = [Fraction(blk["others"])] * 32
        for k, v in blk["values"].items():
            expect[int(k)] = Fraction(v)
        assert [Fraction(float(v)) for v in vals] == expect, blk["name"]


@pytest.mark.parametrize("kind", ["q8_0", "q4_0", "bf16"])
def test_decoders_equal_bytewise_exact_decode(kind):
    from synth import inputs as si
    rng = si.rng_for(0, 99, 1)
    N, K = 3, 96
    W = si.weights(kind, rng, N, K)
    ours = oracle.dequantize(kind, W)
    for n in range(N):
        row = W[n].tobytes()
        exact = ex.row_values(kind, row, K)
        assert [Fraction(float(v)) for v in ours[n]] == exact


def test_q4_0_code_order_low_nibble_first():
    blk = np.zeros((1, 1, 18), dtype=np.uint8)
    blk[0, 0, 2] = 0x21   # byte 0: low nibble 1 -> element 0, high nibble 2 -> element 16
    c = oracle.q4_0_codes(blk)[0, 0]
    assert c[0] == 1 and c[16] == 2 and c[1] == 0 and c[17] == 0


def test_q8_1_field_layout():
    blk = np.zeros((1, 1, 36), dtype=np.uint8)
    blk[0, 0, 0:2] = [0x00, 0x3C]   # d = 1
    blk[0, 0, 2:4] = [0x00, 0x40]   # s = 2
    blk[0, 0, 4] = 0x81             # q0 = -127
    blk[0, 0, 35] = 0x05            # q31 = 5
    d, s, q = oracle.q8_1_fields(blk)
    assert d[0, 0] == 1.0 and s[0, 0] == 2.0 and q[0, 0, 0] == -127 and q[0, 0, 31] == 5
    a = oracle.decode_q8_1(blk)[0]
    assert a[0] == -127.0 and a[31] == 5.0 and np.all(a[1:31] == 0)
