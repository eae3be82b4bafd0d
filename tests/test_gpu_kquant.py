"""GPU checks specific to the K-quant super-block formats (q4_K, q6_K; the
reading of "Chapter 2.2 - speed - 64-lane Metal", In twenty seconds - The fix,
as the 256-element GGUF super-blocks): the packed layout byte for byte,
exactly rounded one-hot products, and the exact cancellation of codes that
decode to zero.  The GEMV parity at small, long-K and full sizes runs with
the other formats."""

import numpy as np
import pytest

import oracle
from oracle import kquant
from synth import inputs as si
from tests._gpu import dev, host, note, poisoned

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def skg():
    import skinny_gemm_decode_amd as m
    return m


def align256(v):
    return (v + 255) // 256 * 256


def expected_packed(kind, W):
    """{offset: bytes} of the packed layout, derived from the codes the oracle
    reads out of the canonical blocks: per row one 16-byte unit per 32
    elements with element i in the low nibble of byte i and element 16 + i in
    its high nibble (q6_K: the low four bits of each code); q6_K then one
    8-byte unit per 32 elements with the top two bits (dword t, byte b: of
    elements 8t + b, 16 + 8t + b at bits 4, 6 and of 8t + 4 + b,
    20 + 8t + b at bits 0, 2); the q4_K super-block headers, or the q6_K int8
    scales and fp16 d, in their own streams."""
    N, nsb, _ = W.shape
    nb = nsb * 8
    if kind == "q4_K":
        c = kquant.q4_K_codes(W).reshape(N, nb, 32)
    else:
        c = kquant.q6_K_codes(W).reshape(N, nb, 32)
    lo = (c[..., :16] & 15) | ((c[..., 16:] & 15) << 4)           # [N, nb, 16]
    regions = {}
    if kind == "q4_K":
        payload = lo.astype(np.uint8).reshape(N, nb * 16)
        row_bytes = nb * 16
        regions[0] = payload.tobytes()
        scale_off = align256(N * row_bytes)
        regions[scale_off] = np.ascontiguousarray(W[..., :16]).tobytes()
        total = align256(scale_off + N * nb * 2)
    else:
        hi = c >> 4                                                  # [N, nb, 32]
        hb = np.zeros((N, nb, 8), np.int64)
        for t in range(2):
            for b in range(4):
                k0, k1 = 2 * t, 2 * t + 1
                hb[..., 4 * t + b] = ((hi[..., 4 * k0 + b] << 4) | (hi[..., 16 + 4 * k0 + b] << 6)
                                      | (hi[..., 4 * k1 + b] << 0) | (hi[..., 16 + 4 * k1 + b] << 2))
        payload = np.concatenate([lo.astype(np.uint8).reshape(N, nb * 16), hb.astype(np.uint8).reshape(N, nb * 8)],
                                 axis=1)
        row_bytes = nb * 24
        regions[0] = payload.tobytes()
        scale_off = align256(N * row_bytes)
        regions[scale_off] = np.ascontiguousarray(W[..., 192:208]).tobytes()
        d_off = align256(scale_off + N * nb * 2)
        regions[d_off] = np.ascontiguousarray(W[..., 208:210]).tobytes()
        total = align256(d_off + N * nsb * 2)
    return regions, total


@pytest.mark.parametrize("fmt", [7, 8])
@pytest.mark.parametrize("N,K", [(1, 256), (5, 768), (33, 4096)])
def test_pack_layout_bit_exact(skg, fmt, N, K):
    kind = skg.WEIGHT_KIND[fmt]
    W = si.weights(kind, si.rng_for(0, 7, 100 + fmt + N), N, K)
    regions, total = expected_packed(kind, W)
    assert skg.packed_size(fmt, N, K) == total
    note(f"pack layout fmt={fmt} N={N} K={K}")
    Wp = host(skg.pack_weights(fmt, N, K, dev(W)))
    for off, ref in regions.items():
        got = Wp[off:off + len(ref)].tobytes()
        assert got == ref, f"region at {off}: first difference at byte {next(i for i in range(len(ref)) if got[i] != ref[i])}"


@pytest.mark.parametrize("fmt", [7, 8])
def test_one_hot_is_the_rounded_weight(skg, fmt):
    """x = e_k: every product is exact before the kernel's last fused
    multiply-add, so y equals the weight rounded once to binary32."""
    kind = skg.WEIGHT_KIND[fmt]
    N, K = 70, 1024
    W = si.weights(kind, si.rng_for(0, 7, 200 + fmt), N, K)
    Wd = oracle.dequantize(kind, W)
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    for k in (0, 15, 16, 31, 32, 130, 200, 255, 256, 700, K - 1):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        note(f"one-hot fmt={fmt} k={k}")
        y = poisoned((1, N))
        skg.gemv(fmt, 1, K, N, Wp, dev(x), y)
        assert np.array_equal(host(y)[0], Wd[:, k].astype(np.float32)), f"k={k}"


@pytest.mark.parametrize("fmt", [8, 10])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_q6_K_codes_32_cancel_exactly(skg, fmt, M):
    """Every code 32 (low bits 0, high bits 2) decodes to w = 0: the output is
    exactly zero whatever the scales and the activation."""
    N, K = 40, 2048
    W = si.weights("q6_K", si.rng_for(0, 7, 300 + fmt + M), N, K)
    W[..., 0:128] = 0x00
    W[..., 128:192] = 0xAA
    assert np.all(oracle.dequantize("q6_K", W) == 0.0)
    x = si.activations_f32(si.rng_for(0, 7, 310 + M), M, K)
    Wp = skg.pack_weights(fmt, N, K, dev(W))
    xin = dev(x) if fmt == skg.Q6_K_F32 else skg.quantize_act_q8_1(dev(x))
    note(f"q6_K codes 32 fmt={fmt} M={M}")
    y = poisoned((M, N))
    skg.gemv(fmt, M, K, N, Wp, xin, y)
    assert np.all(host(y) == 0.0)
