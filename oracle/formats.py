"""Exact decoders for the canonical weight and activation formats (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Formats (all little-endian, row n of an N x K matrix holds its K/32 blocks in
order along K):

* bf16: the upper 16 bits of an IEEE binary32 value.  The decode GEMV of
  "The Shape That Actually Matters" (The shape a decode step actually runs;
  Round 1) streams bf16 weights of shape N=12288 x K=4096.
* q8_0, 34-byte block: fp16 scale d, then 32 int8 codes q; w_i = d * q_i.
  "The Shape That Actually Matters" (Round 1, Round 2) also quantises to 8 bits
  with one scale per 32 elements, but its byte counts (56.6 MB for the
  12288 x 4096 matrix, 0.563 of bf16) put 36 bytes in each block, i.e. a wider
  scale; the block used here is the 34-byte one with an fp16 scale.
* q4_0, 18-byte block: fp16 scale d, then 16 bytes of 4-bit codes; element i
  (i < 16) is the low nibble of byte i, element i + 16 the high nibble of byte
  i; w_i = d * (code_i - 8).  "Six hypotheses, four refutations" (Hypothesis
  ledger) names the 18-byte q4_0 block; the value rule and the nibble order are
  this project's stated reading of that format.
* Q8_1 activation block, 36 bytes: fp16 scale d, fp16 block sum s, then 32
  int8 codes; a_i = d * q_i.  The RX 6700 XT Llama 2 7B decode write-up
  (austxu.dev, Approach & Methodology) feeds Q8_1 activations to the Q4_0 integer-dot matvec.
"""

from __future__ import annotations

import numpy as np

QK = 32
BF16_BYTES = 2
Q8_0_BLOCK_BYTES = 34
Q4_0_BLOCK_BYTES = 18
Q8_1_BLOCK_BYTES = 36


def fp16_bits_to_f64(bits) -> np.ndarray:
    """Decode IEEE binary16 bit patterns to float64, from the definition.

    sign bit 15, 5-bit biased exponent e (bias 15), 10-bit fraction f:
    e == 0 -> (-1)^s * f * 2^-24 (zero and subnormals);
    0 < e < 31 -> (-1)^s * (1024 + f) * 2^(e - 25).
    Infinities and NaNs (e == 31) are rejected: the inputs are finite.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    if np.any(e == 31):
        raise ValueError("fp16 infinity/NaN in an input that must be finite")
    mag = np.where(e == 0, f.astype(np.float64) * 2.0**-24,
                   (1024 + f).astype(np.float64) * np.exp2((e - 25).astype(np.float64)))
    return np.where(s == 1, -mag, mag)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns: they are the top half of a binary32 value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    v = b.view(np.float32) if b.flags["C_CONTIGUOUS"] else np.ascontiguousarray(b).view(np.float32)
    out = v.astype(np.float64)
    if not np.all(np.isfinite(out)):
        raise ValueError("bf16 infinity/NaN in an input that must be finite")
    return out


def _le16(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    return lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)


def decode_bf16(W) -> np.ndarray:
    """uint16 [..., K] bf16 -> float64 [..., K]."""
    return bf16_bits_to_f64(W)


def decode_q8_0(B) -> np.ndarray:
    """uint8 [N, nb, 34] -> float64 [N, nb*32]; w_i = d * q_i."""
    B = np.asarray(B, dtype=np.uint8)
    assert B.shape[-1] == Q8_0_BLOCK_BYTES
    d = fp16_bits_to_f64(_le16(B[..., 0], B[..., 1]))
    q = B[..., 2:].view(np.int8).astype(np.float64)
    w = d[..., None] * q
    return w.reshape(*B.shape[:-2], B.shape[-2] * QK)


def q4_0_codes(B) -> np.ndarray:
    """uint8 [N, nb, 18] -> int64 [N, nb, 32] 4-bit codes in element order.

    Element i < 16 is the low nibble of code byte i; element i >= 16 is the
    high nibble of code byte i - 16.
    """
    B = np.asarray(B, dtype=np.uint8)
    assert B.shape[-1] == Q4_0_BLOCK_BYTES
    qs = B[..., 2:].astype(np.int64)
    return np.concatenate([qs & 0x0F, qs >> 4], axis=-1)


def decode_q4_0(B) -> np.ndarray:
    """uint8 [N, nb, 18] -> float64 [N, nb*32]; w_i = d * (code_i - 8)."""
    B = np.asarray(B, dtype=np.uint8)
    d = fp16_bits_to_f64(_le16(B[..., 0], B[..., 1]))
    c = q4_0_codes(B)
    w = d[..., None] * (c - 8).astype(np.float64)
    return w.reshape(*B.shape[:-2], B.shape[-2] * QK)


def q8_1_fields(B):
    """uint8 [M, nb, 36] -> (d float64 [M, nb], s float64 [M, nb], q int64 [M, nb, 32])."""
    B = np.asarray(B, dtype=np.uint8)
    assert B.shape[-1] == Q8_1_BLOCK_BYTES
    d = fp16_bits_to_f64(_le16(B[..., 0], B[..., 1]))
    s = fp16_bits_to_f64(_le16(B[..., 2], B[..., 3]))
    q = B[..., 4:].view(np.int8).astype(np.int64)
    return d, s, q


def decode_q8_1(B) -> np.ndarray:
    """uint8 [M, nb, 36] -> float64 [M, nb*32]; a_i = d * q_i."""
    d, _, q = q8_1_fields(B)
    a = d[..., None] * q.astype(np.float64)
    return a.reshape(*np.asarray(B).shape[:-2], np.asarray(B).shape[-2] * QK)


def dequantize(kind: str, W) -> np.ndarray:
    """Exact float64 values of canonical weights of the named kind."""
    if kind == "bf16":
        return decode_bf16(W)
    if kind == "q8_0":
        return decode_q8_0(W)
    if kind == "q4_0":
        return decode_q4_0(W)
    if kind in ("q4_K", "q6_K"):
        from . import kquant
        return kquant.decode_q4_K(W) if kind == "q4_K" else kquant.decode_q6_K(W)
    raise ValueError(f"unknown weight kind {kind!r}")
