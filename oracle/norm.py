"""RMSNorm with a per-channel gain (test oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

The RX 6700 XT Llama 2 7B decode write-up (austxu.dev, Approach & Methodology)
lets the RMSNorm-plus-scale dispatch that precedes a Q4_0 matvec also write
that matvec's Q8_1 activation, so no separate quantisation dispatch runs;
"Six hypotheses, four refutations" (Hypothesis ledger: fewer, longer kernels)
counts the same fusion, normalisation writing the quantised format directly,
among its launch savings.  Neither page writes the normalisation out.  The
reading taken is the textbook root-mean-square normalisation with a learned
gain per channel, for each row m of an M x K activation:

    xn[m, k] = g[k] * x[m, k] / sqrt( (1/K) * sum_j x[m, j]^2 + eps )

computed here in float64 from the float32 inputs (g = 1 when no gain is
given).  The Q8_1 output of the fused step is ``quantize_q8_1`` applied to the
normalised values the GPU stores in binary32, so the integer decision is taken
in the same precision on both sides.
"""

from __future__ import annotations

import numpy as np

# Tolerance of a binary32 evaluation against the float64 definition, per
# element: xn = (x * r) * g with r = 1 / sqrt(ss / K + eps).  A binary32 sum of
# (positive) squares whose longest chain of dependent additions has depth D is
# off by at most D * u relatively (u = 2^-24); r inherits half of that plus one
# rounding each for / K, + eps, sqrt and 1 / (4 u), and the two products add
# 2 u.  For D <= 80 that is 40 u + 6 u = 46 u ~ 2.7e-6; the gate is 4e-6 of
# |xn| plus an absolute floor for zero and underflowing outputs.
RMS_REL_TOL = 4e-6
RMS_ABS_TOL = 1e-30


def _rows(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")
    return x


def rmsnorm(x, g=None, eps: float = 1e-5) -> np.ndarray:
    """float64 [M, K]: g * x / sqrt(mean(x^2) + eps), row by row."""
    x64 = _rows(x).astype(np.float64)
    K = x64.shape[1]
    if eps < 0 or not np.isfinite(eps):
        raise ValueError("eps must be finite and >= 0")
    ms = np.sum(x64 * x64, axis=1, keepdims=True) / K
    den = np.sqrt(ms + np.float64(np.float32(eps)))
    if np.any(den == 0):
        raise ValueError("an all-zero row with eps = 0 has no normalisation")
    xn = x64 / den
    if g is not None:
        g64 = np.asarray(g, dtype=np.float32).astype(np.float64).reshape(1, K)
        xn = xn * g64
    return xn


def rmsnorm_tolerance(xn_ref: np.ndarray) -> np.ndarray:
    """Per-element bound on |xn_gpu - xn_ref| for a binary32 evaluation."""
    return RMS_REL_TOL * np.abs(xn_ref) + RMS_ABS_TOL
