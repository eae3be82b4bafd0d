"""Exact rational arithmetic used to pin the oracle.

Everything here is written independently of the oracle and of numpy's float
arithmetic: bytes are parsed by hand, IEEE values become ``Fraction``s, and
rounding to binary32 / binary16 is done with integer arithmetic from the IEEE
754 definition (round to nearest, ties to even, gradual underflow).
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

F32 = (24, -126)   # (significand bits incl. hidden bit, minimum normal exponent)
F16 = (11, -14)


def round_binary(v: Fraction, fmt=F32) -> Fraction:
    """Round an exact rational to the nearest value of a binary format (ties to even)."""
    p, emin = fmt
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f16_value(bits: int) -> Fraction:
    """Exact value of a binary16 bit pattern (finite only)."""
    s = (bits >> 15) & 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    assert e != 31
    mag = Fraction(f, 2**24) if e == 0 else Fraction(1024 + f) * Fraction(2) ** (e - 25)
    return -mag if s else mag


def f16_bits(v: Fraction) -> int:
    """Bit pattern of a value that is exactly representable in binary16."""
    if v == 0:
        return 0
    s = 0x8000 if v < 0 else 0
    a = abs(v)
    for e in range(1, 31):
        m = a / (Fraction(2) ** (e - 25))
        if m.denominator == 1 and 1024 <= m < 2048:
            return s | (e << 10) | (int(m) - 1024)
    m = a * 2**24
    assert m.denominator == 1 and m < 1024, "not representable"
    return s | int(m)


def f32_value(x: float) -> Fraction:
    """Exact value of a Python float that holds a binary32 value."""
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    s = (b >> 31) & 1
    e = (b >> 23) & 0xFF
    f = b & 0x7FFFFF
    assert e != 255
    mag = Fraction(f, 2**149) if e == 0 else Fraction(2**23 + f) * Fraction(2) ** (e - 150)
    return -mag if s else mag


def bf16_value(bits: int) -> Fraction:
    """Exact value of a bf16 bit pattern: the top half of a binary32 pattern."""
    b = (bits & 0xFFFF) << 16
    s = (b >> 31) & 1
    e = (b >> 23) & 0xFF
    f = b & 0x7FFFFF
    assert e != 255
    mag = Fraction(f, 2**149) if e == 0 else Fraction(2**23 + f) * Fraction(2) ** (e - 150)
    return -mag if s else mag


def half_away(v: Fraction) -> int:
    """Nearest integer, ties away from zero."""
    a = abs(v)
    n = math.floor(a + Fraction(1, 2))
    return -n if v < 0 else n


def int8(b: int) -> int:
    b = int(b)
    return b - 256 if b >= 128 else b


# --- block decoders, byte by byte -------------------------------------------

def q8_0_block_values(block: bytes) -> list[Fraction]:
    d = f16_value(block[0] | (block[1] << 8))
    return [d * int8(block[2 + i]) for i in range(32)]


def q4_0_block_codes(block: bytes) -> list[int]:
    codes = [0] * 32
    for i in range(16):
        codes[i] = block[2 + i] & 0x0F
        codes[i + 16] = block[2 + i] >> 4
    return codes


def q4_0_block_values(block: bytes) -> list[Fraction]:
    d = f16_value(block[0] | (block[1] << 8))
    return [d * (c - 8) for c in q4_0_block_codes(block)]


def q8_1_block_fields(block: bytes):
    d = f16_value(block[0] | (block[1] << 8))
    s = f16_value(block[2] | (block[3] << 8))
    q = [int8(block[4 + i]) for i in range(32)]
    return d, s, q


def q8_1_quantize_block(xs: list[float]):
    """Q8_1 of one 32-element binary32 block with every step rounded exactly:
    d = f32(amax/127), id = f32(1/d), q_i = half_away(f32(x_i id)),
    stored d = f16(d), stored s = f16(f32(d * sum q))."""
    xv = [f32_value(v) for v in xs]
    amax = max(abs(v) for v in xv)
    d = round_binary(amax / 127, F32)
    inv = round_binary(1 / d, F32) if d != 0 else Fraction(0)
    q = [half_away(round_binary(v * inv, F32)) for v in xv]
    q = [max(-127, min(127, c)) for c in q]
    d16 = round_binary(d, F16)
    s16 = round_binary(round_binary(d * sum(q), F32), F16)
    return d16, s16, q


def row_values(kind: str, row_bytes: bytes, K: int) -> list[Fraction]:
    """Exact values of one canonical weight row."""
    if kind == "bf16":
        return [bf16_value(row_bytes[2 * k] | (row_bytes[2 * k + 1] << 8)) for k in range(K)]
    if kind == "q8_0":
        out = []
        for b in range(K // 32):
            out += q8_0_block_values(row_bytes[34 * b: 34 * b + 34])
        return out
    if kind == "q4_0":
        out = []
        for b in range(K // 32):
            out += q4_0_block_values(row_bytes[18 * b: 18 * b + 18])
        return out
    if kind == "q4_K":
        out = []
        for b in range(K // 256):
            out += q4_K_block_values(row_bytes[144 * b: 144 * b + 144])
        return out
    if kind == "q6_K":
        out = []
        for b in range(K // 256):
            out += q6_K_block_values(row_bytes[210 * b: 210 * b + 210])
        return out
    raise ValueError(kind)


# --- K-quant super-blocks (256 elements), byte by byte -----------------------

def q4_K_block_scales_mins(block: bytes):
    """(sc, m) lists of the eight 6-bit sub-block scales and mins, read bit by
    bit from the 12 packed bytes s = block[4:16]: the low six bits of s[j]
    (scale) and s[j+4] (min) for j < 4; for j >= 4 the low / high nibble of
    s[j+4] below the top two bits of s[j-4] (scale) and s[j] (min)."""
    s = block[4:16]
    sc, m = [], []
    for j in range(8):
        if j < 4:
            sc.append(s[j] % 64)
            m.append(s[j + 4] % 64)
        else:
            sc.append(s[j + 4] % 16 + 16 * (s[j - 4] // 64))
            m.append(s[j + 4] // 16 + 16 * (s[j] // 64))
    return sc, m


def q4_K_block_values(block: bytes) -> list[Fraction]:
    """Walks the 128 code bytes: byte 32c + i gives element 64c + i (low
    nibble) and element 64c + 32 + i (high nibble)."""
    assert len(block) == 144
    d = f16_value(block[0] | (block[1] << 8))
    dmin = f16_value(block[2] | (block[3] << 8))
    sc, m = q4_K_block_scales_mins(block)
    out = [None] * 256
    for byte_index in range(128):
        b = block[16 + byte_index]
        c, i = divmod(byte_index, 32)
        for e, code in ((64 * c + i, b % 16), (64 * c + 32 + i, b // 16)):
            j = e // 32
            out[e] = d * sc[j] * code - dmin * m[j]
    return out


def q6_K_block_values(block: bytes) -> list[Fraction]:
    """Walks the ql bytes of each 128-element half: ql[64h + l] holds elements
    l (low nibble) and l + 64 (high nibble), ql[64h + 32 + l] elements l + 32
    and l + 96 (l < 32, relative to the half); qh[32h + l] holds the top two
    bits of those four elements at bit pairs 0, 1 (element l), 2, 3 (l + 32),
    4, 5 (l + 64), 6, 7 (l + 96)."""
    assert len(block) == 210
    ql, qh = block[0:128], block[128:192]
    sc = [int8(v) for v in block[192:208]]
    d = f16_value(block[208] | (block[209] << 8))
    out = [None] * 256
    for h in range(2):
        for l in range(32):
            a, b, hb = ql[64 * h + l], ql[64 * h + 32 + l], qh[32 * h + l]
            lows = (a % 16, b % 16, a // 16, b // 16)
            for k in range(4):
                e = 128 * h + l + 32 * k
                q = lows[k] + 16 * ((hb >> (2 * k)) % 4)
                out[e] = d * sc[e // 16] * (q - 32)
    return out
