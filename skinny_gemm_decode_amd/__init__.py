"""Python binding of libskg, the MI355X (gfx950) skinny decode GEMM / GEMV library.

Argument marshalling only: every function here checks that its tensors are
contiguous GPU tensors large enough for the call (the C ABI sees raw pointers
and cannot), passes raw device pointers and the current HIP stream to the C
ABI declared in ``include/skg.h``, and raises ``SkgError`` on a nonzero status.
All arithmetic happens in the library's HIP kernels; there is no CPU fallback.
Importing this module fails with ImportError when ``libskg.so`` has not been
built (``python skinny_gemm_decode_amd/build.py``).

PyTorch is used for device memory and streams only.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskg.so")

# skg_fmt
BF16_BF16 = 0
Q8_0_F32 = 1
Q4_0_F32 = 2
Q4_0_Q8_1 = 3
Q8_0_Q8_1 = 4
Q4_0_BF16 = 5
Q8_0_BF16 = 6
Q4_K_F32 = 7
Q6_K_F32 = 8
Q4_K_Q8_1 = 9
Q6_K_Q8_1 = 10
Q4_K_BF16 = 11
Q6_K_BF16 = 12
FMT_NAMES = {BF16_BF16: "bf16_bf16", Q8_0_F32: "q8_0_f32", Q4_0_F32: "q4_0_f32",
             Q4_0_Q8_1: "q4_0_q8_1", Q8_0_Q8_1: "q8_0_q8_1", Q4_0_BF16: "q4_0_bf16", Q8_0_BF16: "q8_0_bf16",
             Q4_K_F32: "q4_K_f32", Q6_K_F32: "q6_K_f32", Q4_K_Q8_1: "q4_K_q8_1", Q6_K_Q8_1: "q6_K_q8_1",
             Q4_K_BF16: "q4_K_bf16", Q6_K_BF16: "q6_K_bf16"}
# weight kind of each format (the canonical encoding pack_weights reads)
WEIGHT_KIND = {BF16_BF16: "bf16", Q8_0_F32: "q8_0", Q4_0_F32: "q4_0", Q4_0_Q8_1: "q4_0", Q8_0_Q8_1: "q8_0",
               Q4_0_BF16: "q4_0", Q8_0_BF16: "q8_0", Q4_K_F32: "q4_K", Q6_K_F32: "q6_K", Q4_K_Q8_1: "q4_K",
               Q6_K_Q8_1: "q6_K", Q4_K_BF16: "q4_K", Q6_K_BF16: "q6_K"}
Q8_1_FMTS = (Q4_0_Q8_1, Q8_0_Q8_1, Q4_K_Q8_1, Q6_K_Q8_1)
# skg_epi
EPI_NONE = 0
EPI_SWIGLU = 1
EPI_SWIGLU_Q8_1 = 2  # SwiGLU, and h also written as Q8_1 blocks (ys[1])
# skg_status
OK, E_INVALID_ARG, E_SHAPE, E_ALIGN, E_UNSUPPORTED, E_DEVICE, E_HIP = range(7)

Q8_1_BLOCK_BYTES = 36


class SkgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python skinny_gemm_decode_amd/build.py`")
    # PyTorch's HIP runtime must be loaded first: the library then binds to it
    # by soname, so one process never holds two HIP runtimes (a second copy,
    # loaded through the library's own runpath, does not see the device once
    # PyTorch has initialised it).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "skg_abi_version": (i32, []),
        "skg_status_str": (ctypes.c_char_p, [i32]),
        "skg_last_error": (ctypes.c_char_p, []),
        "skg_packed_size": (sz, [i32, i64, i64]),
        "skg_pack_weights": (i32, [i32, i64, i64, vp, vp, vp]),
        "skg_packed_size_multi": (sz, [i32, i32, ctypes.POINTER(i64), i64]),
        "skg_pack_weights_multi": (i32, [i32, i32, ctypes.POINTER(i64), i64, ctypes.POINTER(vp), vp, vp]),
        "skg_quantize_act_q8_1": (i32, [i64, i64, vp, vp, vp]),
        "skg_rmsnorm_q8_1": (i32, [i64, i64, vp, vp, ctypes.c_float, vp, vp, vp]),
        "skg_gemv": (i32, [i32, i64, i64, i64, vp, vp, vp, vp]),
        "skg_gemv_multi": (i32, [i32, i64, i64, i32, ctypes.POINTER(i64), vp, vp, ctypes.POINTER(vp), i32, vp]),
        "skg_gemm_tiled": (i32, [i32, i64, i64, i64, vp, vp, vp, vp]),
        "skg_debug_block_dots": (i32, [i32, i64, i64, i64, i64, vp, vp, vp, vp]),
        "skg_stream_read": (i32, [vp, sz, vp, vp]),
        "skg_empty_launch": (i32, [i64, i32, vp]),
        "skg_gemv_default_variant": (i32, [i32, i32, i32, i64, ctypes.POINTER(i32)]),
        "skg_gemv_set_variant": (i32, [i32, i32, i32, i32, i32, i32, i32, i32, i32]),
        "skg_gemv_variants": (i32, [ctypes.POINTER(i32), i32]),
        "skg_set_lds_pad": (i32, [i64]),
        "skg_gemm_tiled_set_variant": (i32, [i32]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def abi_version() -> int:
    return lib.skg_abi_version()


def status_str(status: int) -> str:
    return lib.skg_status_str(status).decode()


def last_error() -> str:
    return lib.skg_last_error().decode()


def check(status: int) -> None:
    if status != OK:
        raise SkgError(status, last_error())


def _stream(stream) -> int:
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# Bytes per K element of an activation row, by product format (Q8_1: 36-byte
# blocks of 32 elements), and of a canonical weight row element.
_X_BYTES_PER_32 = {BF16_BF16: 64, Q8_0_F32: 128, Q4_0_F32: 128, Q4_0_Q8_1: 36, Q8_0_Q8_1: 36,
                   Q4_0_BF16: 64, Q8_0_BF16: 64, Q4_K_F32: 128, Q6_K_F32: 128, Q4_K_Q8_1: 36, Q6_K_Q8_1: 36,
                   Q4_K_BF16: 64, Q6_K_BF16: 64}
_W_BYTES_PER_32 = {BF16_BF16: 64, Q8_0_F32: 34, Q4_0_F32: 18, Q4_0_Q8_1: 18, Q8_0_Q8_1: 34,
                   Q4_0_BF16: 18, Q8_0_BF16: 34}
# K-quant super-blocks: bytes per 256 elements
_W_BYTES_PER_256 = {Q4_K_F32: 144, Q4_K_Q8_1: 144, Q4_K_BF16: 144, Q6_K_F32: 210, Q6_K_Q8_1: 210, Q6_K_BF16: 210}


def _need(t, nbytes: int, what: str) -> int:
    """Device pointer of t after checking that it is a contiguous GPU tensor
    holding at least nbytes: the library sees raw pointers only, so a short or
    strided tensor would otherwise be read or written out of bounds."""
    if t is None:
        raise ValueError(f"{what} is required")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call needs {nbytes}")
    return t.data_ptr()


def _x_bytes(fmt: int, M: int, K: int) -> int:
    return M * (K // 32) * _X_BYTES_PER_32.get(fmt, 0) + (M * (K % 32) * 2 if fmt == BF16_BF16 else 0)


def _w_bytes(fmt: int, N: int, K: int) -> int:
    if fmt in _W_BYTES_PER_256:
        return N * (K // 256) * _W_BYTES_PER_256[fmt]
    return N * K * 2 if fmt == BF16_BF16 else N * (K // 32) * _W_BYTES_PER_32.get(fmt, 0)


# ---- packing -----------------------------------------------------------

def packed_size(fmt: int, N: int, K: int) -> int:
    return int(lib.skg_packed_size(fmt, N, K))


def packed_size_multi(fmt: int, Ns: Sequence[int], K: int) -> int:
    arr = (ctypes.c_int64 * len(Ns))(*Ns)
    return int(lib.skg_packed_size_multi(fmt, len(Ns), arr, K))


def pack_weights(fmt: int, N: int, K: int, src, dst=None, stream=None):
    """Pack canonical weights (device tensor) into a new or given uint8 buffer."""
    import torch

    size = packed_size(fmt, N, K)
    if size == 0:
        check(lib.skg_pack_weights(fmt, N, K, None, None, None))
    if dst is None:
        dst = torch.empty(size, dtype=torch.uint8, device=src.device)
    check(lib.skg_pack_weights(fmt, N, K, _need(src, _w_bytes(fmt, N, K), "src"), _need(dst, size, "dst"),
                               _stream(stream)))
    return dst


def pack_weights_multi(fmt: int, Ns: Sequence[int], K: int, srcs, dst=None, stream=None):
    """Pack several canonical matrices sharing K into one buffer (QKV, gate/up)."""
    import torch

    n = len(Ns)
    size = packed_size_multi(fmt, Ns, K)
    arr = (ctypes.c_int64 * n)(*Ns)
    if size == 0:
        check(lib.skg_pack_weights_multi(fmt, n, arr, K, None, None, None))
    if len(srcs) != n:
        raise ValueError(f"{n} sizes but {len(srcs)} source matrices")
    if dst is None:
        dst = torch.empty(size, dtype=torch.uint8, device=srcs[0].device)
    ptrs = (ctypes.c_void_p * n)(*[_need(s, _w_bytes(fmt, N, K), f"srcs[{i}]") for i, (s, N) in enumerate(zip(srcs, Ns))])
    check(lib.skg_pack_weights_multi(fmt, n, arr, K, ptrs, _need(dst, size, "dst"), _stream(stream)))
    return dst


# ---- activation quantisation -------------------------------------------

def quantize_act_q8_1(x, xq=None, stream=None):
    """float32 [M, K] device tensor -> uint8 [M, K/32, 36] Q8_1 blocks."""
    import torch

    if x.dim() == 1:
        x = x.unsqueeze(0)
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K // 32, Q8_1_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    check(lib.skg_quantize_act_q8_1(M, K, _need(x, M * K * 4, "x"), _need(xq, M * (K // 32) * Q8_1_BLOCK_BYTES, "xq"),
                                    _stream(stream)))
    return xq


def rmsnorm_q8_1(x, g=None, eps: float = 1e-5, xn=True, xq=True, stream=None):
    """RMSNorm of float32 [M, K] rows with per-channel gain g (None: 1).

    xn / xq: True to allocate the output, a tensor to write into, or
    None / False to skip it (at least one is produced).  Returns (xn, xq):
    float32 [M, K] and uint8 [M, K/32, 36] Q8_1 blocks of exactly xn.
    """
    import torch

    if x.dim() == 1:
        x = x.unsqueeze(0)
    M, K = x.shape
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 tensor")
    if g is not None and (g.dtype != torch.float32 or not g.is_contiguous() or g.numel() != K):
        raise ValueError("g must be a contiguous float32 tensor of K elements")
    if xn is True:
        xn = torch.empty((M, K), dtype=torch.float32, device=x.device)
    elif xn is False:
        xn = None
    if xq is True:
        xq = torch.empty((M, K // 32, Q8_1_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    elif xq is False:
        xq = None
    check(lib.skg_rmsnorm_q8_1(M, K, _need(x, M * K * 4, "x"), _need(g, K * 4, "g") if g is not None else None,
                               float(eps), _need(xn, M * K * 4, "xn") if xn is not None else None,
                               _need(xq, M * (K // 32) * Q8_1_BLOCK_BYTES, "xq") if xq is not None else None,
                               _stream(stream)))
    return xn, xq


# ---- products -------------------------------------------------------------

def gemv(fmt: int, M: int, K: int, N: int, W, x, y=None, stream=None):
    """y[M, N] = x W^T on packed weights W (skinny GEMM, 1 <= M <= 8)."""
    import torch

    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=W.device)
    check(lib.skg_gemv(fmt, M, K, N, _need(W, packed_size(fmt, N, K), "W"), _need(x, _x_bytes(fmt, M, K), "x"),
                       _need(y, M * N * 4, "y"), _stream(stream)))
    return y


def gemv_multi(fmt: int, M: int, K: int, Ns: Sequence[int], W, x, ys=None, epi: int = EPI_NONE, stream=None):
    """Several packed matrices sharing x in one launch.  SwiGLU writes one
    output h; SwiGLU_Q8_1 writes h and its Q8_1 blocks (uint8 [M, N/32, 36])."""
    import torch

    n = len(Ns)
    nout = {EPI_SWIGLU: 1, EPI_SWIGLU_Q8_1: 2}.get(epi, n)
    if ys is None:
        if epi == EPI_SWIGLU_Q8_1:
            ys = [torch.empty((M, Ns[0]), dtype=torch.float32, device=W.device),
                  torch.empty((M, Ns[0] // 32, 36), dtype=torch.uint8, device=W.device)]
        else:
            ys = [torch.empty((M, Ns[i]), dtype=torch.float32, device=W.device) for i in range(nout)]
    arr = (ctypes.c_int64 * n)(*Ns)
    if len(ys) < nout:
        raise ValueError(f"{nout} outputs needed, {len(ys)} given")
    if epi in (EPI_SWIGLU, EPI_SWIGLU_Q8_1):
        need = [M * Ns[0] * 4, M * (Ns[0] // 32) * Q8_1_BLOCK_BYTES][:nout]
    else:
        need = [M * Ns[i] * 4 for i in range(nout)]
    yp = (ctypes.c_void_p * nout)(*[_need(t, b, f"ys[{i}]") for i, (t, b) in enumerate(zip(ys, need))])
    check(lib.skg_gemv_multi(fmt, M, K, n, arr, _need(W, packed_size_multi(fmt, Ns, K), "W"),
                             _need(x, _x_bytes(fmt, M, K), "x"), yp, epi, _stream(stream)))
    return ys


def gemm_tiled(fmt: int, M: int, K: int, N: int, W, x, y=None, stream=None):
    """y[M, N] = x W^T on MFMA for large M: q4_0, q8_0, q4_K or q6_K weights
    against bf16 x, or q4_0 / q8_0 weights against Q8_1 blocks of x (integer
    matrix cores)."""
    import torch

    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=W.device)
    check(lib.skg_gemm_tiled(fmt, M, K, N, _need(W, packed_size(fmt, N, K), "W"), _need(x, _x_bytes(fmt, M, K), "x"),
                             _need(y, M * N * 4, "y"), _stream(stream)))
    return y


def debug_block_dots(fmt: int, N: int, K: int, n0: int, nr: int, W, xq, out=None, stream=None):
    """int32 [nr, K/32] integer block dots of rows [n0, n0+nr) (test hook)."""
    import torch

    if out is None:
        out = torch.empty((nr, K // 32), dtype=torch.int32, device=W.device)
    check(lib.skg_debug_block_dots(fmt, N, K, n0, nr, _need(W, packed_size(fmt, N, K), "W"),
                                   _need(xq, (K // 32) * Q8_1_BLOCK_BYTES, "xq"),
                                   _need(out, max(nr, 0) * (K // 32) * 4, "out"), _stream(stream)))
    return out


def stream_read(buf, nbytes: int | None = None, out=None, stream=None):
    """Read nbytes of buf once (bandwidth ceiling); returns the sink tensor."""
    import torch

    if out is None:
        out = torch.zeros(1, dtype=torch.int32, device=buf.device)
    nbytes = _nbytes(buf) if nbytes is None else nbytes
    check(lib.skg_stream_read(_need(buf, nbytes, "buf"), nbytes, _need(out, 4, "out"), _stream(stream)))
    return out


def empty_launch(grid: int = 1, block: int = 64, stream=None) -> None:
    """One kernel that does nothing (the launch-floor reference)."""
    check(lib.skg_empty_launch(grid, block, _stream(stream)))


# ---- tuning hooks ------------------------------------------------------

VARIANT_KEYS = ("fmt", "M", "epi", "ro", "j", "x_lds", "waves", "kw", "depth")


def gemv_variants():
    """List of compiled GEMV variants as dicts (first per (fmt, M, epi) = default)."""
    n = lib.skg_gemv_variants(None, 0)
    w = len(VARIANT_KEYS)
    buf = (ctypes.c_int * (w * n))()
    lib.skg_gemv_variants(buf, n)
    return [dict(zip(VARIANT_KEYS, buf[w * i: w * i + w])) for i in range(n)]


def gemv_default_variant(fmt: int, M: int, epi: int = EPI_NONE, K: int = 4096) -> dict:
    """The variant record a gemv call with these arguments runs now."""
    buf = (ctypes.c_int * len(VARIANT_KEYS))()
    check(lib.skg_gemv_default_variant(fmt, M, epi, K, buf))
    return dict(zip(VARIANT_KEYS, buf[:len(VARIANT_KEYS)]))


def gemv_set_variant(fmt: int, M: int, epi: int = EPI_NONE, ro: int = 0, j: int = 0, x_lds: int = 0,
                     waves: int = 4, kw: int = 1, depth: int = 0) -> None:
    check(lib.skg_gemv_set_variant(fmt, M, epi, ro, j, x_lds, waves, kw, depth))


def gemv_select(v: dict) -> None:
    """Select the variant of a record from gemv_variants() for its (fmt, M, epi)."""
    gemv_set_variant(v["fmt"], v["M"], v["epi"], v["ro"], v["j"], v["x_lds"], v["waves"], v["kw"], v["depth"])


def gemv_reset(fmt: int, M: int, epi: int = EPI_NONE) -> None:
    """Back to the default variant of (fmt, M, epi)."""
    gemv_set_variant(fmt, M, epi, 0)


def set_lds_pad(nbytes: int) -> None:
    check(lib.skg_set_lds_pad(nbytes))


def gemm_tiled_set_variant(variant: int) -> None:
    check(lib.skg_gemm_tiled_set_variant(variant))
