"""Helpers for the GPU parity tests: device transfer, poisoned outputs and
oracle comparisons.  Every expected value comes from ``oracle``; nothing the
GPU produced is ever fed to the oracle as an input."""

from __future__ import annotations

import sys

import numpy as np

import oracle


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    """numpy -> contiguous GPU tensor with the same bytes."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16)).cuda()
    return t.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    torch().cuda.synchronize()
    return t.detach().cpu().numpy()


def poisoned(shape, dtype=None):
    """Output buffer pre-filled with a NaN pattern so unwritten elements show up."""
    t = torch()
    dtype = dtype or t.float32
    out = t.empty(shape, dtype=dtype, device="cuda")
    if dtype == t.float32:
        out.fill_(float("nan"))
    else:
        out.fill_(-1)
    return out


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(msg, file=sys.stderr, flush=True)


def assert_close(y, y_ref, bound, what: str, rel=oracle.REL_TOL, abs_=oracle.ABS_TOL):
    ok, worst = oracle.check_close(y, y_ref, oracle.tolerance(bound, rel, abs_))
    if not ok:
        err = np.abs(np.asarray(y, np.float64) - y_ref)
        i = np.unravel_index(np.nanargmax(np.where(np.isfinite(err), err, np.inf)), err.shape)
        raise AssertionError(f"{what}: worst err/tol = {worst:.3g} at {i}: y={np.asarray(y)[i]!r} "
                             f"ref={y_ref[i]!r} bound={bound[i]!r}")
    return worst


def sample_rows(N, n=256, seed=0):
    """Sorted output rows to check at full size: a seeded sample plus both ends
    and the last 40 rows (the ragged tail of any row tiling)."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    rows |= {0, 1, N - 2, N - 1} | set(range(max(0, N - 40), N))
    return np.array(sorted(r for r in rows if 0 <= r < N))
