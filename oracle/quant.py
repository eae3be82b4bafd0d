"""Block quantisers (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

quantize_q8_1 is the activation quantiser on the decode path: the RX 6700 XT
Llama 2 7B decode write-up (austxu.dev, Approach & Methodology) feeds Q8_1
activations (int8 codes, a scale and a block sum per 32 elements) to its
Q4_0 x Q8_1 integer-dot matvec, produced by a standalone quantisation dispatch
or fused into the RMSNorm that precedes it.  The pages do not print the
quantiser's arithmetic; the stated reading, carried out here one IEEE binary32
operation at a time so the integer result is unique, is, per 32-element block:

1. amax = max_i |x_i|
2. d    = amax / 127                 (binary32 division, round-to-nearest-even)
3. id   = 1 / d if d != 0 else 0     (binary32 division)
4. q_i  = round_half_away(x_i * id)  (binary32 product, ties away from zero)
5. stored d: binary16(d), nearest-even
6. stored s: binary16(d * float32(sum_i q_i)), the binary32 product of the
   unrounded d and the code sum, then nearest-even to binary16

quantize_q8_0 / quantize_q4_0 are weight quantisers used only to state the
round-trip invariants of the weight formats; the library takes weights that are
already quantised.
"""

from __future__ import annotations

import numpy as np

from .formats import QK

_F32 = np.float32


def round_half_away_f32(p: np.ndarray) -> np.ndarray:
    """Round binary32 values to the nearest integer, ties away from zero.

    |p| + 0.5 is formed in float64, where it is exact for every binary32 p of
    magnitude below 2^52, so 0.49999997f rounds to 0 (in binary32 that sum would
    round up to 1.0).
    """
    p64 = np.asarray(p, dtype=np.float32).astype(np.float64)
    return (np.sign(p64) * np.floor(np.abs(p64) + 0.5)).astype(np.int64)


def _blocks(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    if K % QK:
        raise ValueError("K must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")
    return x.reshape(M, K // QK, QK)


def _scale_and_codes(xb: np.ndarray, qmax: int):
    """Steps 1-4 above for qmax = 127; returns (d float32, codes int64)."""
    amax = np.max(np.abs(xb), axis=-1)                       # exact
    d = (amax / _F32(qmax)).astype(_F32)                     # step 2
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = (_F32(1.0) / d[nz]).astype(_F32)               # step 3
    p = (xb * inv[..., None]).astype(_F32)                   # step 4, product
    q = round_half_away_f32(p)
    q = np.clip(q, -qmax, qmax)                              # guard; never active
    return d, q


def _f16_le_bytes(v: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(v, dtype=np.float32).astype("<f2")
    return h.view(np.uint8).reshape(*np.shape(v), 2)


def quantize_q8_1(x) -> np.ndarray:
    """float32 [M, K] (or [K]) -> uint8 [M, K/32, 36] Q8_1 blocks {d, s, q[32]}."""
    xb = _blocks(x)
    d, q = _scale_and_codes(xb, 127)
    sumq = q.sum(axis=-1).astype(_F32)                       # exact integer <= 4064
    s = (d * sumq).astype(_F32)                              # step 6 product
    out = np.empty((*xb.shape[:2], 36), dtype=np.uint8)
    out[..., 0:2] = _f16_le_bytes(d)                         # step 5
    out[..., 2:4] = _f16_le_bytes(s)                         # step 6 rounding
    out[..., 4:] = q.astype(np.int8).view(np.uint8)
    return out


def quantize_q8_0(x) -> np.ndarray:
    """float32 [N, K] -> uint8 [N, K/32, 34] q8_0 blocks (steps 1-5 above)."""
    xb = _blocks(x)
    d, q = _scale_and_codes(xb, 127)
    out = np.empty((*xb.shape[:2], 34), dtype=np.uint8)
    out[..., 0:2] = _f16_le_bytes(d)
    out[..., 2:] = q.astype(np.int8).view(np.uint8)
    return out


def quantize_q4_0(x) -> np.ndarray:
    """float32 [N, K] -> uint8 [N, K/32, 18] q4_0 blocks.

    Per block: m = the signed element of largest magnitude (the first on ties);
    d = m / -8 (binary32); id = 1/d (0 if d == 0);
    code_i = clamp(round_half_away(x_i * id) + 8, 0, 15); stored d = binary16(d).
    Code element i < 16 goes to the low nibble of byte i, element i + 16 to its
    high nibble.  This maps m itself to code 0, so the whole -8..7 range is used.
    """
    xb = _blocks(x)
    idx = np.argmax(np.abs(xb), axis=-1)                     # first on ties
    m = np.take_along_axis(xb, idx[..., None], axis=-1)[..., 0]
    d = (m / _F32(-8.0)).astype(_F32)
    nz = d != 0
    inv = np.zeros_like(d)
    inv[nz] = (_F32(1.0) / d[nz]).astype(_F32)
    p = (xb * inv[..., None]).astype(_F32)
    c = np.clip(round_half_away_f32(p) + 8, 0, 15).astype(np.uint8)
    out = np.empty((*xb.shape[:2], 18), dtype=np.uint8)
    out[..., 0:2] = _f16_le_bytes(d)
    out[..., 2:] = c[..., :16] | (c[..., 16:] << 4)
    return out
