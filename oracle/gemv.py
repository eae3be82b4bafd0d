"""Reference products of the decode path (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

The operation is the skinny GEMM of token decode, y[m, n] = sum_k W[n, k] x[m, k]
for M = 1..8 activation rows against an N x K weight matrix ("The Shape That
Actually Matters", The shape a decode step actually runs: one activation row
times every weight matrix, M=1, K=4096, N=12288), and the same product at
M = 512 for the tiled prefill GEMM ("Chapter 2.2 - speed - 64-lane Metal",
the tile).  Every result here is the plain definition: operands are decoded
exactly to float64 and the products are summed by numpy's float64 matmul.

Tolerance for float outputs: |y - y_ref| <= 2e-3 * sum_k |W[n,k] x[m,k]| + 1e-6.
Integer block dot products have no tolerance: they are exact integers.
"""

from __future__ import annotations

import numpy as np

from .formats import (
    QK,
    dequantize,
    decode_bf16,
    decode_q4_0,
    decode_q8_0,
    fp16_bits_to_f64,
    q4_0_codes,
    q8_1_fields,
)

REL_TOL = 2e-3
ABS_TOL = 1e-6


def gemv_ref(W: np.ndarray, x: np.ndarray):
    """W float64 [N, K], x float64 [M, K] -> (y [M, N], bound [M, N]).

    y = x W^T and bound = |x| |W|^T, the sum of absolute products that scales
    the tolerance.
    """
    W = np.asarray(W, dtype=np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    assert W.shape[1] == x.shape[1]
    return x @ W.T, np.abs(x) @ np.abs(W).T


def gemv_ref_fmt(kind: str, W_canonical, x, x_kind: str = "f32"):
    """Decode canonical weights ("bf16", "q8_0", "q4_0") and activations
    ("f32" float32 values or "bf16" bit patterns), then gemv_ref."""
    Wd = dequantize(kind, W_canonical)
    if x_kind == "bf16":
        xd = decode_bf16(x)
    elif x_kind == "f32":
        xd = np.asarray(x, dtype=np.float32).astype(np.float64)
    else:
        raise ValueError(x_kind)
    return gemv_ref(Wd, np.atleast_2d(xd))


def tolerance(bound: np.ndarray, rel: float = REL_TOL, abs_: float = ABS_TOL) -> np.ndarray:
    """Allowed |y - y_ref| for fp32-accumulated outputs."""
    return rel * np.asarray(bound, dtype=np.float64) + abs_


def check_close(y, y_ref, allowed) -> tuple[bool, float]:
    """(all within allowed, worst |err| / allowed)."""
    err = np.abs(np.asarray(y, dtype=np.float64) - np.asarray(y_ref, dtype=np.float64))
    allowed = np.asarray(allowed, dtype=np.float64)
    ratio = err / allowed
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(np.isfinite(err)) and worst <= 1.0), worst


# --------------------------------------------------------------------------
# Integer-dot path: q4_0 weights against Q8_1 activations (RX 6700 XT Llama 2
# decode write-up, Approach & Methodology: wave64 integer-dot Q4_0 x Q8_1
# matvec).  Per block b of row n, the integer dot of the 4-bit codes with the
# activation codes is exact; the block's contribution is
# dW_b * dA_b * (sum_i code_i qa_i - 8 sum_i qa_i).
# --------------------------------------------------------------------------

def block_dots_q4_0_q8_1(Wq4, xq) -> np.ndarray:
    """Wq4 uint8 [N, nb, 18], xq uint8 [nb, 36] (one activation row)
    -> int64 [N, nb]: sum_i code_i * qa_i over each block (exact)."""
    c = q4_0_codes(Wq4)                                  # [N, nb, 32]
    _, _, qa = q8_1_fields(np.asarray(xq).reshape(-1, 36))  # [nb, 32]
    return np.einsum("nbi,bi->nb", c, qa)


def block_dots_q8_0_q8_1(Wq8, xq) -> np.ndarray:
    """Wq8 uint8 [N, nb, 34], xq uint8 [nb, 36] -> int64 [N, nb]: sum_i q_i qa_i."""
    qw = np.asarray(Wq8, dtype=np.uint8)[..., 2:].view(np.int8).astype(np.int64)
    _, _, qa = q8_1_fields(np.asarray(xq).reshape(-1, 36))
    return np.einsum("nbi,bi->nb", qw, qa)


def _dW(B) -> np.ndarray:
    B = np.asarray(B, dtype=np.uint8)
    return fp16_bits_to_f64(B[..., 0].astype(np.uint16) | (B[..., 1].astype(np.uint16) << 8))


def gemv_q4_0_q8_1_ref(Wq4, xq):
    """q4_0 [N, nb, 18] x Q8_1 [M, nb, 36] -> (y_ref, y_ref_s, bound), each [M, N].

    y_ref   = sum_b dW dA (sumi - 8 sum_i qa_i): the exact dot of the decoded
              operands, identical to gemv_ref(decode_q4_0(W), decode_q8_1(xq)).
    y_ref_s = sum_b dW (dA sumi - 8 s): the same with the stored block sum s in
              place of dA sum_i qa_i, which is what a kernel reading s computes.
              It is the second reference that tells a rounding artifact of s
              from a computation error ("Six hypotheses, four refutations",
              How the agents searched: a second reference to classify errors).
    bound   = sum_k |w_k a_k| over the decoded operands.
    """
    Wq4 = np.asarray(Wq4, dtype=np.uint8)
    xq = np.asarray(xq, dtype=np.uint8).reshape(-1, Wq4.shape[1], 36)
    dW = _dW(Wq4)                                         # [N, nb]
    c = q4_0_codes(Wq4)                                   # [N, nb, 32]
    ys, yss = [], []
    for m in range(xq.shape[0]):
        dA, sA, qa = q8_1_fields(xq[m])                   # [nb], [nb], [nb, 32]
        sumi = np.einsum("nbi,bi->nb", c, qa).astype(np.float64)
        sq = qa.sum(axis=-1).astype(np.float64)
        ys.append(np.sum(dW * dA[None, :] * (sumi - 8.0 * sq[None, :]), axis=1))
        yss.append(np.sum(dW * (dA[None, :] * sumi - 8.0 * sA[None, :]), axis=1))
    Wd = decode_q4_0(Wq4)
    from .formats import decode_q8_1
    _, bound = gemv_ref(Wd, decode_q8_1(xq))
    return np.stack(ys), np.stack(yss), bound


def gemv_q8_0_q8_1_ref(Wq8, xq):
    """q8_0 [N, nb, 34] x Q8_1 [M, nb, 36] -> (y_ref, bound): exact decoded dot."""
    from .formats import decode_q8_1
    Wd = decode_q8_0(Wq8)
    xq = np.asarray(xq, dtype=np.uint8).reshape(-1, np.asarray(Wq8).shape[1], 36)
    return gemv_ref(Wd, decode_q8_1(xq))


# --------------------------------------------------------------------------
# Gate/up + SwiGLU epilogue (RX 6700 XT Llama 2 decode write-up, Approach &
# Methodology: gate and up projections evaluated together, SwiGLU written
# directly).  The pages name SwiGLU without defining it; the textbook form is
# h = silu(g) * u with silu(z) = z / (1 + e^-z), g the gate (first) matrix.
# --------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu_ref(g, u) -> np.ndarray:
    return silu(g) * np.asarray(u, dtype=np.float64)


#: sup over z of |d silu / dz| (about 1.0998), rounded up
SILU_LIPSCHITZ = 1.1


def swiglu_tolerance(g_ref, u_ref, tol_g, tol_u) -> np.ndarray:
    """Allowed |h - h_ref| when g and u each carry the GEMV tolerance.

    |silu(g')u' - silu(g)u| <= |silu'|max |u| tol_g + |silu(g)| tol_u (first
    order), plus binary32 evaluation of silu and the product (a few units in
    the last place of h) and the absolute floor.
    """
    g_ref = np.asarray(g_ref, dtype=np.float64)
    u_ref = np.asarray(u_ref, dtype=np.float64)
    h_ref = swiglu_ref(g_ref, u_ref)
    first = SILU_LIPSCHITZ * (np.abs(u_ref) + tol_u) * tol_g + np.abs(silu(g_ref)) * tol_u
    return first + 8.0 * 2.0**-24 * np.abs(h_ref) + ABS_TOL


# --------------------------------------------------------------------------
# M = 512 tiled prefill GEMM (Chapter 2.2 - speed - 64-lane Metal, the tile:
# read the weights once per 64x64 tile instead of once per row).
# --------------------------------------------------------------------------

def gemm_tiled_ref(Wq, A_bf16, kind: str = "q4_0"):
    """Quantised weights [N, nb, block] ("q4_0" 18-byte or "q8_0" 34-byte
    blocks, "q4_K" / "q6_K" super-blocks) x bf16 bit patterns [M, K] ->
    (y, bound, y_bf16w) [M, N].

    "Chapter 2.2 - speed - 64-lane Metal" (the tile) decodes each weight tile
    once and multiplies it against every activation row; the product itself
    is the plain definition, y[m][n] = sum_k w[n][k] x[m][k] in fp64.
    y_bf16w rounds every decoded weight to bf16 (nearest-even) before the
    float64 product: the value a kernel that stages bf16 weights computes
    exactly up to summation order.  It is a second reference for classifying
    deviations, not the gate.  The page does not say how a K-quant weight
    reaches bf16; the reading taken here is the plainest one for a kernel
    that decodes in binary32: the decoded value is rounded once to binary32
    (nearest-even; exact for q4_0 and q8_0), then to bf16.
    """
    if kind not in ("q4_0", "q8_0", "q4_K", "q6_K"):
        raise ValueError(f"tile weights are q4_0, q8_0, q4_K or q6_K, not {kind!r}")
    Wd = dequantize(kind, Wq)
    A = decode_bf16(A_bf16)
    y, bound = gemv_ref(Wd, A)
    w32 = Wd.astype(np.float32)                            # exact: 11 + 4 (q4_0) or 11 + 8 (q8_0) bits
    u = w32.view(np.uint32).astype(np.uint64)
    wb = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    y_bf16w, _ = gemv_ref(decode_bf16(wb), A)
    return y, bound, y_bf16w
