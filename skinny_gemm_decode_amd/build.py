"""Build libskg.so (gfx950 only) in-tree with hipcc.

Every HIP source is compiled to an object in parallel, then linked into one
shared library next to this file.  Usage: ``python skinny_gemm_decode_amd/build.py``
(run as a file: importing the package would load the library being rebuilt).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libskg.so")

ARCH = "gfx950"
SOURCES = [
    "gemv_mfma_q4_0.hip",
    "gemv_mfma_q8_0.hip",
    "gemv_mfma_q8_1.hip",
    "gemv_q4_0_f32_m68.hip",
    "gemv_q4_0_f32_m35.hip",
    "gemv_q8_0_f32_m38.hip",
    "api.hip",
    "pack.hip",
    "quant.hip",
    "norm.hip",
    "misc.hip",
    "gemm_tiled.hip",
    "gemm_i8.hip",
    "gemv_bf16.hip",
    "gemv_q8_0_f32.hip",
    "gemv_q4_0_f32.hip",
    "gemv_q8_1.hip",
    "gemv_q4_K.hip",
    "gemv_q6_K.hip",
]

# Packed fp32 arithmetic is disabled for every HIP translation unit; the host
# pass warns that it does not know the feature, which is harmless.
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every source and link libskg.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
