"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any HIP
call (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skg.h")


@pytest.fixture(scope="module")
def skg():
    import skinny_gemm_decode_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skg_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["skg_pack_weights", "skg_pack_weights_multi", "skg_packed_size", "skg_packed_size_multi",
                     "skg_quantize_act_q8_1", "skg_rmsnorm_q8_1", "skg_gemv", "skg_gemv_multi", "skg_gemm_tiled",
                     "skg_status_str", "skg_last_error", "skg_debug_block_dots", "skg_stream_read"]:
        assert required in names


def test_library_exports_every_declared_symbol(skg):
    lib = ctypes.CDLL(skg.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version_and_status_strings(skg):
    assert skg.abi_version() == 2
    assert skg.status_str(0) == "SKG_OK"
    assert skg.status_str(2) == "SKG_E_SHAPE"
    assert skg.status_str(99) == "SKG_E_UNKNOWN"


def test_packed_sizes(skg):
    # q4_0 at K=4096, N=14336: 16-byte payload + 2-byte scale per block
    assert skg.packed_size(skg.Q4_0_F32, 14336, 4096) == 14336 * 128 * 18
    assert skg.packed_size(skg.Q8_0_F32, 14336, 4096) == 14336 * 128 * 34
    assert skg.packed_size(skg.BF16_BF16, 12288, 4096) == 12288 * 4096 * 2
    assert skg.packed_size(skg.Q4_0_Q8_1, 4096, 11008) == 4096 * 344 * 18
    assert skg.packed_size(skg.Q4_0_F32, 1, 33) == 0        # K not a multiple of 32
    assert skg.packed_size(skg.BF16_BF16, 0, 64) == 0       # N < 1
    assert skg.packed_size(17, 4, 64) == 0                  # unknown format
    assert skg.packed_size_multi(skg.Q4_0_Q8_1, [4096, 4096, 4096], 4096) == 3 * 4096 * 128 * 18
    # K-quants: q4_K 16-byte units + 16-byte header per 256 elements; q6_K
    # 24 bytes per 32 elements, int8 scale pairs, then fp16 d per 256 elements,
    # each stream starting on a 256-byte boundary
    a256 = lambda v: (v + 255) // 256 * 256
    assert skg.packed_size(skg.Q4_K_F32, 14336, 4096) == 14336 * 128 * 18
    assert skg.packed_size(skg.Q4_K_Q8_1, 3, 256) == a256(a256(3 * 8 * 16) + 3 * 8 * 2)
    q6 = a256(14336 * 128 * 24) + 14336 * 128 * 2
    assert skg.packed_size(skg.Q6_K_F32, 14336, 4096) == a256(q6) + 14336 * 16 * 2
    assert skg.packed_size(skg.Q6_K_Q8_1, 5, 512) == a256(a256(a256(5 * 16 * 24) + 5 * 16 * 2) + 5 * 2 * 2)
    for fmt in (skg.Q4_K_F32, skg.Q6_K_F32, skg.Q4_K_Q8_1, skg.Q6_K_Q8_1):
        assert skg.packed_size(fmt, 4, 4128) == 0           # K not a multiple of 256
        assert skg.packed_size(fmt, 4, 128) == 0
    # three 4096x4096 + two 11008x4096 + one 4096x11008 q4_0 matrices: one decode layer
    layer = (skg.packed_size_multi(3, [4096] * 3, 4096) + skg.packed_size_multi(3, [11008] * 2, 4096)
             + skg.packed_size(3, 4096, 11008))
    assert layer == 104_398_848


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)

# The calls below pass fake device pointers and rely on host validation to
# reject them.  Where a GPU is visible, a mistaken "invalid" case would launch
# a kernel on those pointers, so these tests run only where there is none.
no_gpu = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                            reason="fake-pointer validation tests run only without a GPU")


def call(skg, name, *args):
    return getattr(skg.lib, name)(*args)


@no_gpu
@pytest.mark.parametrize("args,status", [
    ((99, 1, 4096, 4096), 1),            # unknown fmt
    ((5, 1, 4096, 4096), 4),             # gemm format is not a gemv format
    ((2, 0, 4096, 4096), 2),             # M = 0
    ((2, 9, 4096, 4096), 2),             # M > 8
    ((2, 1, 4008, 4096), 2),             # K % 32 != 0
    ((0, 1, 4, 4096), 2),                # bf16 K < 8
    ((2, 1, 4096, 0), 2),                # N = 0
])
def test_gemv_shape_and_fmt_errors(skg, args, status):
    fmt, M, K, N = args
    assert call(skg, "skg_gemv", fmt, M, K, N, FAKE, FAKE, FAKE, None) == status
    assert skg.last_error() != ""


@no_gpu
def test_gemv_pointer_errors(skg):
    assert call(skg, "skg_gemv", 2, 1, 4096, 4096, None, FAKE, FAKE, None) == skg.E_INVALID_ARG
    assert call(skg, "skg_gemv", 2, 1, 4096, 4096, FAKE, FAKE, None, None) == skg.E_INVALID_ARG
    assert call(skg, "skg_gemv", 2, 1, 4096, 4096, MISALIGNED, FAKE, FAKE, None) == skg.E_ALIGN
    assert call(skg, "skg_gemv", 2, 1, 4096, 4096, FAKE, MISALIGNED, FAKE, None) == skg.E_ALIGN
    # Q8_1 activations need only 4-byte alignment; y needs 4
    assert call(skg, "skg_gemv", 3, 1, 4096, 4096, FAKE, ctypes.c_void_p((1 << 20) + 4), MISALIGNED,
                None) == skg.E_ALIGN


@no_gpu
def test_gemv_multi_errors(skg):
    Ns = (ctypes.c_int64 * 4)(64, 64, 64, 64)
    ys = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    g = skg.lib.skg_gemv_multi
    assert g(2, 1, 64, 0, Ns, FAKE, FAKE, ys, 0, None) == skg.E_INVALID_ARG        # n = 0
    assert g(2, 1, 64, 5, Ns, FAKE, FAKE, ys, 0, None) == skg.E_INVALID_ARG        # n > 4
    assert g(2, 1, 64, 3, Ns, FAKE, FAKE, ys, 1, None) == skg.E_INVALID_ARG        # swiglu needs n = 2
    Ns2 = (ctypes.c_int64 * 2)(64, 65)
    assert g(2, 1, 64, 2, Ns2, FAKE, FAKE, ys, 1, None) == skg.E_SHAPE             # gate/up differ
    assert g(2, 1, 64, 2, Ns, FAKE, FAKE, ys, 7, None) == skg.E_INVALID_ARG        # unknown epilogue
    ysn = (ctypes.c_void_p * 2)(FAKE, None)
    assert g(2, 1, 64, 2, Ns, FAKE, FAKE, ysn, 0, None) == skg.E_INVALID_ARG       # null output
    # SwiGLU with Q8_1 output: integer-dot formats, whole 32-row blocks, two outputs
    assert g(2, 1, 64, 2, Ns, FAKE, FAKE, ys, 2, None) == skg.E_UNSUPPORTED        # fp32-activation format
    Ns48 = (ctypes.c_int64 * 2)(48, 48)
    assert g(3, 1, 64, 2, Ns48, FAKE, FAKE, ys, 2, None) == skg.E_SHAPE            # N % 32 != 0
    assert g(3, 1, 64, 2, Ns, FAKE, FAKE, ysn, 2, None) == skg.E_INVALID_ARG       # null Q8_1 output
    ysm = (ctypes.c_void_p * 2)(FAKE, MISALIGNED)
    assert g(3, 1, 64, 2, Ns, FAKE, FAKE, ysm, 2, None) == skg.E_ALIGN             # Q8_1 output alignment
    assert g(3, 1, 64, 3, Ns, FAKE, FAKE, ys, 2, None) == skg.E_INVALID_ARG        # n must be 2


@no_gpu
def test_other_entry_point_errors(skg):
    L = skg.lib
    assert L.skg_quantize_act_q8_1(0, 64, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_quantize_act_q8_1(1, 48, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_quantize_act_q8_1(1, 64, MISALIGNED, FAKE, None) == skg.E_ALIGN
    assert L.skg_quantize_act_q8_1(1, 64, FAKE, None, None) == skg.E_INVALID_ARG
    nrm = L.skg_rmsnorm_q8_1
    assert nrm(0, 4096, FAKE, FAKE, 1e-5, FAKE, FAKE, None) == skg.E_SHAPE            # M = 0
    assert nrm((1 << 24) + 1, 4096, FAKE, FAKE, 1e-5, FAKE, FAKE, None) == skg.E_SHAPE
    assert nrm(1, 48, FAKE, FAKE, 1e-5, FAKE, FAKE, None) == skg.E_SHAPE              # K % 32
    assert nrm(1, 16416, FAKE, FAKE, 1e-5, FAKE, FAKE, None) == skg.E_SHAPE           # K > 16384
    assert nrm(1, 0, FAKE, FAKE, 1e-5, FAKE, FAKE, None) == skg.E_SHAPE
    assert nrm(1, 4096, None, FAKE, 1e-5, FAKE, FAKE, None) == skg.E_INVALID_ARG      # null x
    assert nrm(1, 4096, FAKE, FAKE, 1e-5, None, None, None) == skg.E_INVALID_ARG      # no output
    for eps in (-1e-5, float("nan"), float("inf")):
        assert nrm(1, 4096, FAKE, FAKE, eps, FAKE, FAKE, None) == skg.E_INVALID_ARG
    for args in ((MISALIGNED, FAKE, FAKE, FAKE), (FAKE, MISALIGNED, FAKE, FAKE),
                 (FAKE, FAKE, MISALIGNED, FAKE), (FAKE, FAKE, FAKE, MISALIGNED)):
        x, g, xn, xq = args
        assert nrm(1, 4096, x, g, 1e-5, xn, xq, None) == skg.E_ALIGN
    four = ctypes.c_void_p((1 << 20) + 4)                                          # 4- but not 16-byte aligned
    for args in ((four, FAKE, FAKE, FAKE), (FAKE, four, FAKE, FAKE), (FAKE, FAKE, four, FAKE)):
        x, g, xn, xq = args
        assert nrm(1, 4096, x, g, 1e-5, xn, xq, None) == skg.E_ALIGN
    assert L.skg_gemm_tiled(2, 512, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_UNSUPPORTED
    assert L.skg_gemm_tiled(5, 0, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemm_tiled(5, 512, 4100, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemm_tiled_set_variant(1) == skg.OK
    assert L.skg_gemm_tiled(6, 512, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_UNSUPPORTED  # q8_0: 3, 4 only
    assert L.skg_gemm_tiled_set_variant(-1) == skg.OK
    assert L.skg_gemm_tiled(6, 512, 4100, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemm_tiled_set_variant(1) == skg.OK
    assert L.skg_gemm_tiled(11, 512, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_UNSUPPORTED  # q4_K: 3, 4 only
    assert L.skg_gemm_tiled(12, 512, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_UNSUPPORTED  # q6_K: 3, 4 only
    assert L.skg_gemm_tiled_set_variant(-1) == skg.OK
    assert L.skg_gemm_tiled(11, 512, 4128, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE  # K % 256
    assert L.skg_gemm_tiled(12, 512, 128, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemv(11, 1, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_UNSUPPORTED    # tile format
    assert L.skg_gemm_tiled(3, 512, 4128, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE   # Q8_1 tile: K % 64
    assert L.skg_gemm_tiled(4, 512, 4096, 4096, FAKE, MISALIGNED, FAKE, None) == skg.E_ALIGN
    assert L.skg_gemm_tiled(3, 0, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemv(13, 1, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_INVALID_ARG
    # more output tiles than one launch takes, and M or N beyond 32-bit indices
    assert L.skg_gemm_tiled(5, 1 << 30, 4096, 1 << 20, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemm_tiled(5, 1 << 31, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_gemm_tiled(5, 512, 4096, 1 << 31, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_packed_size(2, 1 << 31, 4096) == 0
    assert L.skg_pack_weights(2, (1 << 31) - 1, 1 << 30, FAKE, FAKE, None) == skg.E_SHAPE  # grid too large
    assert L.skg_pack_weights(2, 4, 64, FAKE, MISALIGNED, None) == skg.E_ALIGN
    assert L.skg_pack_weights(2, 4, 64, ctypes.c_void_p((1 << 20) + 1), FAKE, None) == skg.E_ALIGN
    assert L.skg_pack_weights(2, 4, 60, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_debug_block_dots(2, 8, 64, 0, 1, FAKE, FAKE, FAKE, None) == skg.E_UNSUPPORTED
    assert L.skg_debug_block_dots(3, 8, 64, 6, 3, FAKE, FAKE, FAKE, None) == skg.E_SHAPE
    assert L.skg_stream_read(FAKE, 17, FAKE, None) == skg.E_SHAPE
    assert L.skg_set_lds_pad(1 << 20) == skg.E_INVALID_ARG
    assert L.skg_gemv_set_variant(2, 1, 0, 3, 3, 0, 4, 1, 0) == skg.E_UNSUPPORTED


def test_variant_registry(skg):
    vs = skg.gemv_variants()
    seen = {(v["fmt"], v["M"], v["epi"]) for v in vs}
    for fmt in range(5):
        for M in range(1, 9):
            for epi in (0, 1):
                assert (fmt, M, epi) in seen, (fmt, M, epi)
    for fmt in (3, 4):
        for M in range(1, 9):
            assert (fmt, M, 2) in seen, (fmt, M, 2)
    skg.gemv_set_variant(2, 1, 0, 16, 2, 0, 4, 1)
    skg.gemv_set_variant(2, 1, 0, 0)
    # every record selects itself, depth included; the default query returns
    # the selected record and, after the reset, the first registered one
    for v in vs:
        assert v["depth"] >= 1
    ring = [v for v in vs if v["x_lds"] in (3, 5)]
    assert ring and {v["depth"] for v in ring} <= {2, 3, 4}
    v = ring[-1]
    skg.gemv_select(v)
    try:
        assert skg.gemv_default_variant(v["fmt"], v["M"], v["epi"], 4096) == v
    finally:
        skg.gemv_reset(v["fmt"], v["M"], v["epi"])
    first = next(w for w in vs if (w["fmt"], w["M"], w["epi"]) == (v["fmt"], v["M"], v["epi"]))
    assert skg.gemv_default_variant(v["fmt"], v["M"], v["epi"], 4096) == first
    with pytest.raises(skg.SkgError):
        skg.gemv_set_variant(v["fmt"], v["M"], v["epi"], v["ro"], v["j"], v["x_lds"], v["waves"], v["kw"], 7)


@no_gpu
def test_valid_call_without_gpu_reports_device_error(skg):
    # Arguments are valid, so only the device check can reject the call.
    assert skg.lib.skg_gemv(2, 1, 4096, 4096, FAKE, FAKE, FAKE, None) == skg.E_DEVICE
    assert "device" in skg.last_error().lower()


def test_single_hip_runtime(skg):
    """The library shares PyTorch's HIP runtime: exactly one libamdhip64 is
    mapped into the process after import."""
    with open("/proc/self/maps") as f:
        libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(libs) == 1, libs


class _FakeTensor:
    """Duck-typed stand-in for a device tensor (no GPU here)."""

    def __init__(self, nbytes, cuda=True, contiguous=True):
        self.nbytes_, self.cuda, self.contig = nbytes, cuda, contiguous

    is_cuda = property(lambda self: self.cuda)

    def is_contiguous(self):
        return self.contig

    def numel(self):
        return self.nbytes_

    def element_size(self):
        return 1

    def data_ptr(self):
        return 0x10000


def test_binding_checks_buffer_sizes(skg):
    """The binding refuses host, strided and short tensors before any call:
    the library sees raw pointers and would read or write past them."""
    assert skg._need(_FakeTensor(64), 64, "y") == 0x10000
    for t, msg in ((_FakeTensor(64, cuda=False), "on the GPU"), (_FakeTensor(64, contiguous=False), "contiguous"),
                   (_FakeTensor(63), "63 bytes")):
        with pytest.raises(ValueError, match=msg):
            skg._need(t, 64, "y")
    with pytest.raises(ValueError, match="required"):
        skg._need(None, 4, "x")
    # activation and canonical weight bytes by format
    assert skg._x_bytes(skg.BF16_BF16, 2, 4104) == 2 * 4104 * 2
    assert skg._x_bytes(skg.Q4_0_F32, 3, 4096) == 3 * 4096 * 4
    assert skg._x_bytes(skg.Q8_0_Q8_1, 2, 4096) == 2 * 128 * 36
    assert skg._w_bytes(skg.Q4_0_Q8_1, 5, 4096) == 5 * 128 * 18
    assert skg._w_bytes(skg.Q8_0_F32, 5, 4096) == 5 * 128 * 34
    assert skg._w_bytes(skg.BF16_BF16, 5, 4104) == 5 * 4104 * 2
    # a short output is refused before the library is called
    W, x, y = _FakeTensor(skg.packed_size(skg.Q4_0_F32, 64, 256)), _FakeTensor(4 * 256), _FakeTensor(4 * 64 - 4)
    with pytest.raises(ValueError, match="y holds"):
        skg.gemv(skg.Q4_0_F32, 1, 256, 64, W, x, y)


_PAD_PROBE = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
import skinny_gemm_decode_amd as skg
lib = skg.lib
# W = NULL: rejected on the host by every path, so nothing is ever launched;
# the message tells which check refused the call
st = lib.skg_gemv(2, 1, 4096, 64, None, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None)
print(st, lib.skg_last_error().decode())
st2 = lib.skg_set_lds_pad(ctypes.c_int64(128))
st3 = lib.skg_gemv(2, 1, 4096, 64, None, ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 20), None)
print(st2, st3, lib.skg_last_error().decode())
"""


@pytest.mark.parametrize("value,bad", [("-5", True), ("70000", True), ("12abc", True), ("", True),
                                       ("99999999999999999999999", True), ("0", False), ("1024", False),
                                       (" 4096 ", False), ("65536", False)])
def test_lds_pad_environment_value_is_validated(skg, value, bad):
    """SKG_LDS_PAD_BYTES outside 0..65536 (or not an integer) refuses every
    GEMV call with SKG_E_INVALID_ARG until skg_set_lds_pad sets a valid pad;
    a valid value is accepted (the call then fails only on its null W)."""
    import subprocess
    import sys
    env = dict(os.environ, SKG_LDS_PAD_BYTES=value)
    r = subprocess.run([sys.executable, "-c", _PAD_PROBE.format(root=ROOT)], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    first, second = r.stdout.strip().splitlines()[-2:]
    st, msg = first.split(" ", 1)
    assert int(st) == 1   # SKG_E_INVALID_ARG either way
    if bad:
        assert "SKG_LDS_PAD_BYTES" in msg, msg
    else:
        assert "null W" in msg, msg
    st2, st3, msg3 = second.split(" ", 2)
    assert int(st2) == 0 and int(st3) == 1 and "null W" in msg3, second
