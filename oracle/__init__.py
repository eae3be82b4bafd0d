"""CPU oracle for the skinny decode GEMM / GEMV path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the GPU kernels are checked against.  Only the test suite, the
graft entry point's smoke check and the benchmark's CPU-baseline leg may import
it.  The product path (the HIP library and its Python binding) never imports,
calls or falls back to anything here, and this package imports nothing from the
product path.

Everything is numpy.  Decoding is exact (fp64), products are accumulated in
fp64, and the activation quantiser is emulated step by step in IEEE binary32,
so that the integer codes it produces are the unique result of the stated
operation sequence.

Sources (the four web pages this method is described on):

* "The Shape That Actually Matters" (amarbaro.com): the M=1, K=4096, N=12288
  decode GEMV shape and its bf16 / 8-bit weight arms.
* "Six hypotheses, four refutations, +31% throughput" (MI50 megakernel case
  study): q4_0 matvec with 18-byte blocks; a second, lower-precision reference
  to classify deviations; verification at the stage where a change acts.
* "Chapter 2.2 - speed - 64-lane Metal" (llama-3x-prompt-speed): the 64x64
  tiled prefill GEMM at M=512.
* the RX 6700 XT Llama 2 7B decode write-up (austxu.dev):
  Q4_0 x Q8_1 integer-dot matvec, fused QKV and gate/up + SwiGLU, and the
  RMSNorm-plus-scale that writes the Q8_1 activation directly.

Pins: every function here is checked by the ``-m "not gpu"`` tests against
hand-worked blocks (``tests/golden/``), closed forms, round-trip invariants and
exact rational brute force on tiny inputs.  No function here is "parity
unpinned".
"""

from .formats import (  # noqa: F401
    QK,
    BF16_BYTES,
    Q8_0_BLOCK_BYTES,
    Q4_0_BLOCK_BYTES,
    Q8_1_BLOCK_BYTES,
    fp16_bits_to_f64,
    bf16_bits_to_f64,
    decode_bf16,
    decode_q8_0,
    decode_q4_0,
    decode_q8_1,
    q4_0_codes,
    q8_1_fields,
    dequantize,
)
from .quant import (  # noqa: F401
    quantize_q8_1,
    quantize_q8_0,
    quantize_q4_0,
    round_half_away_f32,
)
from .norm import (  # noqa: F401
    RMS_REL_TOL,
    RMS_ABS_TOL,
    rmsnorm,
    rmsnorm_tolerance,
)
from .gemv import (  # noqa: F401
    REL_TOL,
    ABS_TOL,
    gemv_ref,
    gemv_ref_fmt,
    block_dots_q4_0_q8_1,
    block_dots_q8_0_q8_1,
    gemv_q4_0_q8_1_ref,
    gemv_q8_0_q8_1_ref,
    silu,
    swiglu_ref,
    swiglu_tolerance,
    gemm_tiled_ref,
    tolerance,
    check_close,
)
