"""Validity of Q8_1 blocks against float64 reference values (CPU only).

A GPU producer that quantises values it computed itself (a norm, an
epilogue) is checked bit-exactly against the oracle's quantiser of the values
it stored.  This module adds a check that takes no GPU value as oracle input:
the blocks must be a valid Q8_1 encoding (the quantiser's per-block rules) of
values within the producer's tolerance of the float64 reference.

With d the binary32 block scale and d16 its stored fp16, each code satisfies
|q d - v| <= d (1/2 + 2^-20) for the value v it encodes, |q d16 - q d| <=
127 max(d 2^-11, 2^-25), and |v - ref| <= tol; d itself is at most
(max|ref| + max tol) / 127 over the block, up to one binary32 rounding.  The
stored block sum must be d16 * sum q to within two fp16 roundings, and a block
with a nonzero stored scale uses the full code range (max |q| = 127).
"""

from __future__ import annotations

import numpy as np

import oracle


def q8_1_violations(xq, ref, tol) -> list[str]:
    """Messages for every block of xq [M, nb, 36] that is not a valid Q8_1
    encoding of values within tol [M, K] of ref [M, K]; empty if all are."""
    d16, s16, q = oracle.q8_1_fields(xq)
    M, nb = d16.shape
    ref = np.asarray(ref, dtype=np.float64).reshape(M, nb, 32)
    tol = np.asarray(tol, dtype=np.float64).reshape(M, nb, 32)
    amax = np.max(np.abs(ref), axis=2) + np.max(tol, axis=2)
    d_hi = amax / 127.0 * (1 + 2.0 ** -23)
    bad = []
    err = np.abs(d16[..., None] * q - ref)
    allow = d_hi[..., None] * (0.5 + 2.0 ** -20) + 127 * np.maximum(d_hi[..., None] * 2.0 ** -11, 2.0 ** -25) + tol
    for m, b in np.argwhere(np.any(err > allow, axis=2)):
        i = int(np.argmax(err[m, b] - allow[m, b]))
        bad.append(f"block ({m}, {b}) element {i}: |d q - ref| = {err[m, b, i]:.3g} > {allow[m, b, i]:.3g}")
    qs = np.sum(q, axis=2).astype(np.float64)
    s_err = np.abs(s16 - d16 * qs)
    s_allow = np.abs(d16 * qs) * 2.0 ** -10 + 2.0 ** -24
    for m, b in np.argwhere(s_err > s_allow):
        bad.append(f"block ({m}, {b}): stored sum {s16[m, b]!r} vs d q-sum {d16[m, b] * qs[m, b]!r}")
    full = np.max(np.abs(q), axis=2)
    for m, b in np.argwhere((d16 != 0) & (full != 127)):
        bad.append(f"block ({m}, {b}): nonzero scale but max |q| = {full[m, b]}")
    for m, b in np.argwhere((d16 == 0) & np.any(q != 0, axis=2)):
        bad.append(f"block ({m}, {b}): zero scale with nonzero codes")
    return bad
