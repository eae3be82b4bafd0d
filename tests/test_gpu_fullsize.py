"""GPU parity of every small-batch GEMV default, and of every matrix-core
variant, at the workload's full size K=4096, N=14336 (and a ragged
N=14331), M = 1..8, for all four quantised formats, on EVERY output row.

At this size the persistent matrix-core kernels give each workgroup two to
four 16-row tiles, so the paths that only run from a workgroup's second tile
on (the register reloads of the rolling prefetch, the reuse of an LDS ring
slot, the double-buffered reduction) run under test here, in the launch
configuration the benchmark times.  The oracle decodes the whole matrix once
per format and evaluates y = x W^T in float64 ("Chapter 2.2 - speed - 64-lane
Metal", the negative: test the dispatch the model actually uses, at its real
shape)."""

import numpy as np
import pytest

import oracle
from synth import inputs as si
from tests._gpu import assert_close, dev, host, note, poisoned

pytestmark = pytest.mark.gpu

K = 4096
N_FULL = 14336
N_RAGGED = 14331          # last tile holds 11 rows
KIND = {1: "q8_0", 2: "q4_0", 3: "q4_0", 4: "q8_0", 7: "q4_K", 8: "q6_K", 9: "q4_K", 10: "q6_K"}
SEED = {"q8_0": 2, "q4_0": 1, "q4_K": 3, "q6_K": 4}
FMTS = [1, 2, 3, 4, 7, 8, 9, 10]


@pytest.fixture(scope="module")
def skg():
    import skinny_gemm_decode_amd as m
    return m


_CACHE = {}


def weights(skg, fmt, N):
    """(canonical W, packed W on the device, decoded float64 W), once per
    (weight kind, N) for the module."""
    key = (KIND[fmt], N)
    if key not in _CACHE:
        _CACHE.clear()  # one matrix (~470 MB decoded) at a time
        rng = si.rng_for(0, 4, 500 + N + SEED[KIND[fmt]])
        W = si.weights(KIND[fmt], rng, N, K)
        Wd = oracle.dequantize(KIND[fmt], W)
        _CACHE[key] = (W, {}, Wd)
    W, packed, Wd = _CACHE[key]
    if fmt not in packed:
        note(f"full size: pack fmt={fmt} N={N}")
        packed[fmt] = skg.pack_weights(fmt, N, K, dev(W))
    return W, packed[fmt], Wd


def activation(skg, fmt, M, seed):
    """Device activation as the kernel reads it, and the decoded float64
    activation the reference multiplies (Q8_1 blocks checked bit-exactly
    against the oracle's quantiser first)."""
    x = si.activations_f32(si.rng_for(0, 4, 900 + seed), M, K)
    if fmt in skg.Q8_1_FMTS:
        xq = skg.quantize_act_q8_1(dev(x))
        ref = oracle.quantize_q8_1(x)
        assert np.array_equal(host(xq), ref), "Q8_1 activation differs from the oracle"
        return xq, oracle.decode_q8_1(ref)
    return dev(x), x.astype(np.float64)


def variants_at_k4096(skg, fmt, M):
    out = []
    for v in skg.gemv_variants():
        if v["fmt"] != fmt or v["M"] != M or v["epi"] != skg.EPI_NONE or v["x_lds"] not in (2, 3, 4, 5):
            continue
        nb = K // 32
        if v["x_lds"] in (3, 5) and v["waves"] * v["kw"] != nb:
            continue
        if v["x_lds"] in (2, 4) and (nb % v["kw"] or nb > v["waves"] * v["kw"]):
            continue
        out.append(v)
    return out


def rel_of(skg, fmt, v):
    """Tolerance a matrix-core variant is held to: two fp16 activation terms
    or exact int8 block dots 2e-5 of sum|w x|; one fp16 term (one rounding of
    2^-11 relative per element plus fp32 accumulation) 8e-4; q4_K x Q8_1 the
    2e-3 bound (its min term takes the Q8_1 block sum as stored, in fp16)."""
    if fmt == skg.Q4_K_Q8_1:
        return oracle.REL_TOL
    return 2e-5 if (v["j"] == 2 or fmt in skg.Q8_1_FMTS) else 8e-4


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_full_size_every_row(skg, fmt, M):
    W, Wp, Wd = weights(skg, fmt, N_FULL)
    xin, xd = activation(skg, fmt, M, 10 * fmt + M)
    y_ref, bound = oracle.gemv_ref(Wd, xd)
    dv = skg.gemv_default_variant(fmt, M, skg.EPI_NONE, K)
    note(f"full size default fmt={fmt} M={M} variant {dv}")
    y = poisoned((M, N_FULL))
    skg.gemv(fmt, M, K, N_FULL, Wp, xin, y)
    assert_close(host(y), y_ref, bound, f"default fmt={fmt} M={M} {dv}")
    try:
        for v in variants_at_k4096(skg, fmt, M):
            skg.gemv_select(v)
            note(f"full size fmt={fmt} M={M} variant {v}")
            y = poisoned((M, N_FULL))
            skg.gemv(fmt, M, K, N_FULL, Wp, xin, y)
            assert_close(host(y), y_ref, bound, f"variant {v}", rel=rel_of(skg, fmt, v))
    finally:
        skg.gemv_set_variant(fmt, M, skg.EPI_NONE, 0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [3, 8])
def test_ragged_full_size_every_row(skg, fmt, M):
    """N = 14331: the last 16-row tile is partial (its rows past N are
    clamped on load and never stored)."""
    W, Wp, Wd = weights(skg, fmt, N_RAGGED)
    xin, xd = activation(skg, fmt, M, 100 + 10 * fmt + M)
    y_ref, bound = oracle.gemv_ref(Wd, xd)
    cases = [None] + variants_at_k4096(skg, fmt, M)
    try:
        for v in cases:
            if v is not None:
                skg.gemv_select(v)
            note(f"ragged full size fmt={fmt} M={M} variant {v}")
            y = poisoned((M, N_RAGGED))
            skg.gemv(fmt, M, K, N_RAGGED, Wp, xin, y)
            rel = oracle.REL_TOL if v is None else rel_of(skg, fmt, v)
            assert_close(host(y), y_ref, bound, f"ragged variant {v}", rel=rel)
    finally:
        skg.gemv_set_variant(fmt, M, skg.EPI_NONE, 0)
