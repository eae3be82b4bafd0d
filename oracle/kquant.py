"""K-quant super-block weight formats, q4_K and q6_K (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's oracle leg, never by the product path.

"Chapter 2.2 - speed - 64-lane Metal" (In twenty seconds - The fix; the free
2x) tiles its prefill GEMM for q4_K and q6_K weights and counts the q4_K and
q6_K tensors of its model file, but does not define either encoding.  The
reading taken here is that they are the GGUF super-block formats of 256
elements, the ones such model files carry:

* q4_K, 144 bytes: fp16 d, fp16 dmin, 12 bytes holding eight 6-bit sub-block
  scales sc_j and eight 6-bit mins m_j, then 128 bytes of 4-bit codes q.
  Sub-block j covers elements 32 j .. 32 j + 31 and w = d sc_j q - dmin m_j.
  The 12 bytes s[0..11]: for j < 4, sc_j = s[j] & 63 and m_j = s[j + 4] & 63;
  for j >= 4, sc_j = (s[j + 4] & 15) | (s[j - 4] >> 6) << 4 and
  m_j = (s[j + 4] >> 4) | (s[j] >> 6) << 4.  Codes: element 64 c + i
  (c = 0..3, i < 32) is the low nibble of code byte 32 c + i and element
  64 c + 32 + i its high nibble.
* q6_K, 210 bytes: 128 bytes ql (low 4 bits of each code), 64 bytes qh (high
  2 bits), 16 int8 scales, fp16 d.  For element e, with h = e // 128,
  r = e % 128, g = r // 32 and l = r % 32: low bits = nibble (g >> 1) of
  ql[64 h + 32 (g & 1) + l], high bits = bits 2 g, 2 g + 1 of qh[32 h + l],
  q = low | high << 4, and w = d scales[e // 16] (q - 32).

Every decode below is exact in float64: d and dmin are fp16 values, the
scales small integers, the codes at most 6 bits.
"""

from __future__ import annotations

import numpy as np

from .formats import fp16_bits_to_f64

QK_K = 256
Q4_K_BLOCK_BYTES = 144
Q6_K_BLOCK_BYTES = 210


def _le16(lo, hi) -> np.ndarray:
    return np.asarray(lo, dtype=np.uint16) | (np.asarray(hi, dtype=np.uint16) << 8)


def q4_K_scales_mins(B):
    """uint8 [..., 144] -> (d, dmin float64 [...], sc, m int64 [..., 8])."""
    B = np.asarray(B, dtype=np.uint8)
    assert B.shape[-1] == Q4_K_BLOCK_BYTES
    d = fp16_bits_to_f64(_le16(B[..., 0], B[..., 1]))
    dmin = fp16_bits_to_f64(_le16(B[..., 2], B[..., 3]))
    s = B[..., 4:16].astype(np.int64)
    sc = np.empty(B.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            m[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
            m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return d, dmin, sc, m


def q4_K_codes(B) -> np.ndarray:
    """uint8 [..., 144] -> int64 [..., 256] 4-bit codes in element order."""
    B = np.asarray(B, dtype=np.uint8)
    qs = B[..., 16:].astype(np.int64).reshape(B.shape[:-1] + (4, 32))    # [.., chunk c, byte i]
    lo, hi = qs & 15, qs >> 4
    return np.stack([lo, hi], axis=-2).reshape(B.shape[:-1] + (QK_K,))  # [.., c, (lo|hi), i]


def decode_q4_K(B) -> np.ndarray:
    """uint8 [N, nsb, 144] -> float64 [N, nsb*256]: w = d sc_j q - dmin m_j."""
    B = np.asarray(B, dtype=np.uint8)
    d, dmin, sc, m = q4_K_scales_mins(B)
    q = q4_K_codes(B).reshape(B.shape[:-1] + (8, 32)).astype(np.float64)
    a = (d[..., None] * sc.astype(np.float64))[..., None]               # [.., j, 1]
    b = (dmin[..., None] * m.astype(np.float64))[..., None]
    w = a * q - b
    return w.reshape(*B.shape[:-2], B.shape[-2] * QK_K)


def q6_K_codes(B) -> np.ndarray:
    """uint8 [..., 210] -> int64 [..., 256] 6-bit codes (0..63) in element order."""
    B = np.asarray(B, dtype=np.uint8)
    assert B.shape[-1] == Q6_K_BLOCK_BYTES
    ql = B[..., 0:128].astype(np.int64)
    qh = B[..., 128:192].astype(np.int64)
    e = np.arange(QK_K)
    h, r = e // 128, e % 128
    g, l = r // 32, r % 32
    low = (ql[..., 64 * h + 32 * (g & 1) + l] >> (4 * (g >> 1))) & 15
    high = (qh[..., 32 * h + l] >> (2 * g)) & 3
    return low | (high << 4)


def q6_K_fields(B):
    """uint8 [..., 210] -> (d float64 [...], scales int64 [..., 16])."""
    B = np.asarray(B, dtype=np.uint8)
    d = fp16_bits_to_f64(_le16(B[..., 208], B[..., 209]))
    sc = B[..., 192:208].view(np.int8).astype(np.int64)
    return d, sc


def decode_q6_K(B) -> np.ndarray:
    """uint8 [N, nsb, 210] -> float64 [N, nsb*256]: w = d scale_(e//16) (q - 32)."""
    B = np.asarray(B, dtype=np.uint8)
    d, sc = q6_K_fields(B)
    q = q6_K_codes(B).reshape(B.shape[:-1] + (16, 16)) - 32
    w = d[..., None, None] * sc[..., None].astype(np.float64) * q.astype(np.float64)
    return w.reshape(*B.shape[:-2], B.shape[-2] * QK_K)
