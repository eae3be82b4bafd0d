"""GPU parity: Q8_1 activation quantisation must match the oracle bit for bit."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import inputs as si
from tests._gpu import dev, host, note, poisoned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def skg():
    import skinny_gemm_decode_amd as m
    return m


def _quant_gpu(skg, x):
    M, K = x.shape
    note(f"quantize_act_q8_1 M={M} K={K}")
    xq = poisoned((M, K // 32, 36), dtype=__import__("torch").uint8)
    skg.quantize_act_q8_1(dev(x), xq)
    return host(xq)


@pytest.mark.parametrize("M,K", [(1, 32), (1, 4096), (3, 4096), (1, 11008), (8, 4096), (2, 96)])
def test_q8_1_bit_exact_random(skg, M, K):
    x = si.activations_f32(si.rng_for(0, 3, 100 + M * 7 + K), M, K)
    got = _quant_gpu(skg, x)
    ref = oracle.quantize_q8_1(x)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), f"{np.sum(np.any(got != ref, axis=-1))} blocks differ"


def _adversarial_blocks():
    rng = np.random.default_rng(5)
    blocks = []
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "q8_1_quantize.json")))
    for case in g["cases"]:
        x = np.zeros(32, np.float32)
        for k, v in case["x"].items():
            x[int(k)] = np.float32(float.fromhex(v) if "0x" in v else float(Fraction(v)))
        blocks.append(x)
    for _ in range(64):
        b = (rng.integers(-254, 255, 32) / 2.0).astype(np.float32)    # half-integer ties
        b[rng.integers(0, 32)] = 127.0
        blocks.append(b)
    for scale in (1e-8, 1e-6, 1e-4, 1e2, 3e2):     # subnormal fp16 d .. large d (s stays finite)
        for _ in range(16):
            blocks.append((rng.normal(0, 1, 32) * scale).astype(np.float32))
    blocks.append(np.zeros(32, np.float32))
    for _ in range(16):                                                # a single nonzero
        b = np.zeros(32, np.float32)
        b[rng.integers(0, 32)] = np.float32(rng.normal(0, 10))
        blocks.append(b)
    return np.concatenate(blocks)[None, :]


def test_q8_1_bit_exact_adversarial(skg):
    x = _adversarial_blocks()
    got = _quant_gpu(skg, x)
    ref = oracle.quantize_q8_1(x)
    bad = np.nonzero(np.any(got[0] != ref[0], axis=-1))[0]
    assert bad.size == 0, f"blocks {bad[:10]} differ: got {got[0, bad[0]]} ref {ref[0, bad[0]]}"


def _double_rounding_blocks(n_want=24, seed=11):
    """Blocks whose block sum s = fp16(f32(d * sum q)) differs from rounding
    the exact product straight to fp16: a kernel that fuses the multiply into
    the conversion fails exactly these.  Found on the CPU with exact float64
    products (24 + 12 significant bits fit in 53)."""
    rng = np.random.default_rng(seed)
    found = []
    while len(found) < n_want:
        X = rng.normal(0, 1, (4096, 32)).astype(np.float32)
        q = oracle.quantize_q8_1(X.reshape(1, -1))[0]
        amax = np.max(np.abs(X), axis=1)
        d32 = (amax / np.float32(127)).astype(np.float32)
        sumq = q[:, 4:].view(np.int8).astype(np.int64).sum(axis=1)
        exact = d32.astype(np.float64) * sumq
        single = exact.astype(np.float16)
        double = (d32 * sumq.astype(np.float32)).astype(np.float32).astype(np.float16)
        idx = np.nonzero(single != double)[0]
        found.extend(X[i] for i in idx)
    return np.concatenate(found[:n_want])[None, :]


def test_q8_1_block_sum_rounds_the_binary32_product(skg):
    x = _double_rounding_blocks()
    got = _quant_gpu(skg, x)
    ref = oracle.quantize_q8_1(x)
    bad = np.nonzero(np.any(got[0] != ref[0], axis=-1))[0]
    assert bad.size == 0, f"{bad.size} of {ref.shape[1]} double-rounding blocks differ"
