"""Seeded synthetic inputs for the skinny decode GEMM / GEMV workloads.

This module only draws random numbers and lays them out in the canonical byte
formats; it performs none of the method's arithmetic (no dequantisation, no
quantisation, no dot products).  Both the CPU oracle and the GPU path consume
what it produces, so it is the one piece of code they share.

Canonical formats (row n of an N x K weight matrix holds blocks b = 0..K/32-1
in order, K contiguous):

* bf16 weights / activations: uint16 bit patterns, [rows][K].
* q8_0 block, 34 bytes: fp16 scale d (little-endian) then 32 int8 codes.
* q4_0 block, 18 bytes: fp16 scale d (little-endian) then 16 bytes of codes.
  Random code bytes are drawn uniformly over 0..255, which makes both 4-bit
  codes of every byte independent and uniform over 0..15; which code of the
  byte is which element is the decoder's business, not the generator's.
* q4_K super-block, 144 bytes, and q6_K super-block, 210 bytes (256 elements
  each): the field layout is the decoder's business; the generator fills the
  fp16 scale fields with scale-like values and every other byte uniformly.
* fp32 activations: float32 [M][K].

Value distributions follow the decode workloads of the source pages (token
decode on Llama-2-7B-shaped layers; see the RX 6700 XT Llama 2 7B decode write-up
(austxu.dev), Approach & Methodology, and "The Shape That Actually
Matters", The shape a decode step actually runs): int8 codes uniform in
[-127, 127] with fp16 scales uniform in [1e-3, 1e-2]; 4-bit codes uniform in
0..15 with fp16 scales |N(0, 0.01)|; bf16 weights N(0, 0.02); activations
N(0, 1).  Every draw is keyed by (seed, workload id, buffer index) through
numpy's SeedSequence so any buffer can be regenerated on its own.
"""

from __future__ import annotations

import numpy as np

QK = 32  # elements per quantisation block along K

#: workload ids used to key the random streams
WORKLOAD_IDS = {
    "q8_0_m1_k256_n512": 1,
    "bf16_m1_k4096_n12288": 2,
    "llama2_7b_q4_0_q8_1_layer": 3,
    "skinny_m1to8_k4096_n14336": 4,
    "prefill_q4_0_bf16_m512": 5,
    "test": 99,
}


def rng_for(seed: int, workload: int, buffer_idx: int, stream: int = 0) -> np.random.Generator:
    """Independent generator for (seed, workload id, buffer index, sub-stream)."""
    return np.random.default_rng(np.random.SeedSequence([seed, workload, buffer_idx, stream]))


def _f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _fp16_bytes(v: np.ndarray) -> np.ndarray:
    """fp16 (round-nearest-even) little-endian bytes of float values, shape [..., 2]."""
    h = np.ascontiguousarray(v, dtype=np.float32).astype("<f2")
    return h.view(np.uint8).reshape(*v.shape, 2)


def q8_0_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint8 [N, K/32, 34]: int8 codes uniform in [-127, 127], fp16 scales U[1e-3, 1e-2]."""
    assert K % QK == 0
    nb = K // QK
    q = rng.integers(-127, 128, size=(N, nb, QK), dtype=np.int16).astype(np.int8)
    d = rng.uniform(1e-3, 1e-2, size=(N, nb)).astype(np.float32)
    out = np.empty((N, nb, 34), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(d)
    out[..., 2:] = q.view(np.uint8)
    return out


def q4_0_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint8 [N, K/32, 18]: uniform random code bytes, fp16 scales |N(0, 0.01)|."""
    assert K % QK == 0
    nb = K // QK
    qs = rng.integers(0, 256, size=(N, nb, 16), dtype=np.uint16).astype(np.uint8)
    d = np.abs(rng.normal(0.0, 0.01, size=(N, nb))).astype(np.float32)
    out = np.empty((N, nb, 18), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(d)
    out[..., 2:] = qs
    return out


QK_K = 256  # elements per K-quant super-block


def q4_K_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint8 [N, K/256, 144]: fp16 d and dmin |N(0, 1e-4)|, 12 uniform random
    bytes of packed 6-bit sub-block scales and mins, 128 uniform random code
    bytes.  The pages do not characterise K-quant tensors; these magnitudes put
    typical weights near those of the other formats (|w| ~ 0.02)."""
    assert K % QK_K == 0
    nsb = K // QK_K
    out = np.empty((N, nsb, 144), dtype=np.uint8)
    out[..., 0:2] = _fp16_bytes(np.abs(rng.normal(0.0, 1e-4, size=(N, nsb))).astype(np.float32))
    out[..., 2:4] = _fp16_bytes(np.abs(rng.normal(0.0, 1e-4, size=(N, nsb))).astype(np.float32))
    out[..., 4:] = rng.integers(0, 256, size=(N, nsb, 140), dtype=np.uint16).astype(np.uint8)
    return out


def q6_K_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """uint8 [N, K/256, 210]: 192 uniform random code bytes (low and high
    planes), 16 int8 sub-block scales uniform in [-128, 127], fp16 d
    |N(0, 2e-5)| (typical |w| ~ 0.02; stated choices, as for q4_K)."""
    assert K % QK_K == 0
    nsb = K // QK_K
    out = np.empty((N, nsb, 210), dtype=np.uint8)
    out[..., 0:192] = rng.integers(0, 256, size=(N, nsb, 192), dtype=np.uint16).astype(np.uint8)
    out[..., 192:208] = rng.integers(-128, 128, size=(N, nsb, 16), dtype=np.int16).astype(np.int8).view(np.uint8)
    out[..., 208:210] = _fp16_bytes(np.abs(rng.normal(0.0, 2e-5, size=(N, nsb))).astype(np.float32))
    return out


def bf16_weights(rng: np.random.Generator, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """uint16 [N, K] bf16 bit patterns of N(0, std) values."""
    return _f32_to_bf16_bits(rng.normal(0.0, std, size=(N, K)).astype(np.float32))


def activations_f32(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """float32 [M, K] drawn from N(0, 1)."""
    return rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)


def activations_f32_outliers(rng: np.random.Generator, M: int, K: int, channels: int = 8,
                             scale: float = 40.0) -> np.ndarray:
    """float32 [M, K] N(0, 1) with `channels` randomly chosen channels scaled by
    `scale`: a residual stream with a few large channels, which RMSNorm inputs
    have and the pages do not characterise further."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, size=min(channels, K), replace=False)
    x[:, cols] *= np.float32(scale)
    return x


def norm_gain_f32(rng: np.random.Generator, K: int) -> np.ndarray:
    """float32 [K] per-channel RMSNorm gain drawn from N(1, 0.25)."""
    return (1.0 + 0.25 * rng.standard_normal(K)).astype(np.float32)


def activations_bf16(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    """uint16 [M, K] bf16 bit patterns of N(0, 1) values."""
    return _f32_to_bf16_bits(activations_f32(rng, M, K))


def weights(kind: str, rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Canonical weights of the named kind ("bf16", "q8_0" or "q4_0")."""
    if kind == "bf16":
        return bf16_weights(rng, N, K)
    if kind == "q8_0":
        return q8_0_weights(rng, N, K)
    if kind == "q4_0":
        return q4_0_weights(rng, N, K)
    if kind == "q4_K":
        return q4_K_weights(rng, N, K)
    if kind == "q6_K":
        return q6_K_weights(rng, N, K)
    raise ValueError(f"unknown weight kind {kind!r}")


# ---------------------------------------------------------------------------
# Device-side generators for the large rotation sets of the benchmark.  They
# draw the same distributions with torch's seeded device RNG, so gigabytes of
# distinct weight buffers appear in HBM in well under a second.
# ---------------------------------------------------------------------------

def torch_weights(kind: str, N: int, K: int, seed: int, device):
    """Canonical weights of the named kind as a torch uint8/uint16 device tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    nb = K // QK
    if kind == "bf16":
        w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * 0.02
        return w.to(torch.bfloat16).view(torch.int16)
    if kind == "q4_0":
        out = torch.empty((N, nb, 18), dtype=torch.uint8, device=device)
        d = (torch.randn((N, nb), generator=g, device=device) * 0.01).abs().to(torch.float16)
        out[..., 0:2] = d.view(torch.uint8).view(N, nb, 2)
        out[..., 2:] = torch.randint(0, 256, (N, nb, 16), generator=g, device=device, dtype=torch.uint8)
        return out
    if kind == "q8_0":
        out = torch.empty((N, nb, 34), dtype=torch.uint8, device=device)
        d = (torch.rand((N, nb), generator=g, device=device) * 9e-3 + 1e-3).to(torch.float16)
        out[..., 0:2] = d.view(torch.uint8).view(N, nb, 2)
        q = torch.randint(-127, 128, (N, nb, 32), generator=g, device=device, dtype=torch.int8)
        out[..., 2:] = q.view(torch.uint8)
        return out
    if kind in ("q4_K", "q6_K"):
        nsb = K // QK_K
        if kind == "q4_K":
            out = torch.empty((N, nsb, 144), dtype=torch.uint8, device=device)
            for o in (0, 2):
                d = (torch.randn((N, nsb), generator=g, device=device) * 1e-4).abs().to(torch.float16)
                out[..., o:o + 2] = d.view(torch.uint8).view(N, nsb, 2)
            out[..., 4:] = torch.randint(0, 256, (N, nsb, 140), generator=g, device=device, dtype=torch.uint8)
        else:
            out = torch.empty((N, nsb, 210), dtype=torch.uint8, device=device)
            out[..., 0:208] = torch.randint(0, 256, (N, nsb, 208), generator=g, device=device, dtype=torch.uint8)
            d = (torch.randn((N, nsb), generator=g, device=device) * 2e-5).abs().to(torch.float16)
            out[..., 208:210] = d.view(torch.uint8).view(N, nsb, 2)
        return out
    raise ValueError(f"unknown weight kind {kind!r}")
