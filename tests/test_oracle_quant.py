"""Pins for the oracle's quantisers (CPU only)."""

import json
import os
import struct
from fractions import Fraction

import numpy as np

import oracle
from tests import _exact as ex


def _hexfloat(s):
    return float.fromhex(s) if "0x" in s else float(Fraction(s))


def test_q8_1_golden_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "q8_1_quantize.json")))
    for case in g["cases"]:
        x = np.zeros(32, dtype=np.float32)
        for k, v in case["x"].items():
            x[int(k)] = np.float32(_hexfloat(v))
        blk = oracle.quantize_q8_1(x[None, :])[0, 0]
        d_bits = int(blk[0]) | (int(blk[1]) << 8)
        s_bits = int(blk[2]) | (int(blk[3]) << 8)
        q = blk[4:].view(np.int8).astype(int)
        expect_q = np.zeros(32, dtype=int)
        for k, v in case["q"].items():
            expect_q[int(k)] = v
        assert d_bits == int(case["d_bits"], 16), case["name"]
        assert s_bits == int(case["s_bits"], 16), case["name"]
        assert np.array_equal(q, expect_q), case["name"]


def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    xs = []
    for i in range(n):
        kind = i % 5
        if kind == 0:
            x = rng.normal(0, 1, 32)
        elif kind == 1:
            x = rng.normal(0, 1e-6, 32)                    # tiny: subnormal fp16 scales
        elif kind == 2:
            x = rng.integers(-254, 255, 32) / 2.0           # many exact ties
            x[0] = 127.0
        elif kind == 3:
            x = rng.normal(0, 300, 32)                       # large magnitudes
        else:
            x = rng.normal(0, 1, 32) * (rng.random(32) < 0.2)  # mostly zeros
        xs.append(x.astype(np.float32))
    return np.stack(xs)


def test_q8_1_equals_exactly_rounded_steps_on_random_blocks():
    X = _random_blocks(250, seed=7)
    out = oracle.quantize_q8_1(X.reshape(1, -1))[0]
    for b in range(X.shape[0]):
        d16, s16, q = ex.q8_1_quantize_block([float(v) for v in X[b]])
        blk = out[b]
        assert ex.f16_value(int(blk[0]) | (int(blk[1]) << 8)) == d16, b
        assert ex.f16_value(int(blk[2]) | (int(blk[3]) << 8)) == s16, b
        assert list(blk[4:].view(np.int8).astype(int)) == q, b


def test_q8_1_invariants():
    X = _random_blocks(500, seed=11)
    out = oracle.quantize_q8_1(X.reshape(1, -1))[0]
    d, s, q = oracle.q8_1_fields(out)
    for b in range(X.shape[0]):
        amax = float(np.max(np.abs(X[b])))
        if amax > 0:
            assert np.max(np.abs(q[b])) == 127
        else:
            assert np.all(q[b] == 0) and d[b] == 0 and s[b] == 0
        # reconstruction: |x - d16 q| <= d/2 + |q| |d - d16| (+ binary32 slack)
        d32 = np.float32(amax) / np.float32(127)
        err = np.abs(X[b].astype(np.float64) - d[b] * q[b])
        bound = 0.5 * float(d32) * (1 + 1e-6) + np.abs(q[b]) * abs(float(d32) - d[b]) + 1e-30
        assert np.all(err <= bound + 1e-12 * amax), b


def test_q8_1_shapes_and_row_independence():
    rng = np.random.default_rng(3)
    X = rng.normal(0, 1, (3, 128)).astype(np.float32)
    full = oracle.quantize_q8_1(X)
    assert full.shape == (3, 4, 36)
    for m in range(3):
        assert np.array_equal(full[m], oracle.quantize_q8_1(X[m])[0])


def test_q8_0_round_trip_on_blocks_with_full_range_code():
    from synth import inputs as si
    W = si.q8_0_weights(si.rng_for(0, 99, 2), 8, 256)
    W[..., 2] = np.uint8(0x81)          # force code -127 into every block
    x = oracle.decode_q8_0(W).astype(np.float32)     # exact in binary32
    assert np.array_equal(oracle.quantize_q8_0(x), W)


def test_q4_0_round_trip_on_blocks_with_code_zero():
    from synth import inputs as si
    W = si.q4_0_weights(si.rng_for(0, 99, 3), 8, 256)
    W[..., 2] &= np.uint8(0xF0)         # element 0 of every block gets code 0
    x = oracle.decode_q4_0(W).astype(np.float32)
    assert np.array_equal(oracle.quantize_q4_0(x), W)


def test_q4_0_quantizer_hand_worked():
    # m = -4 at element 3 -> d = 0.5, codes = round(x/0.5)+8
    x = np.zeros(32, dtype=np.float32)
    x[3] = -4.0
    x[0] = 1.25      # 2.5 -> 3 (ties away) -> code 11
    x[20] = 3.5      # 7 -> code 15
    blk = oracle.quantize_q4_0(x[None, :])[0, 0]
    assert (int(blk[0]) | (int(blk[1]) << 8)) == 0x3800
    codes = oracle.q4_0_codes(blk.reshape(1, 1, 18))[0, 0]
    assert codes[3] == 0 and codes[0] == 11 and codes[20] == 15 and codes[1] == 8


def test_round_half_away_trap():
    v = np.array([struct.unpack("<f", struct.pack("<I", 0x3EFFFFFF))[0], 0.5, -0.5, 1.5, 2.5, -2.5],
                 dtype=np.float32)
    assert list(oracle.round_half_away_f32(v)) == [0, 1, -1, 2, 3, -3]
