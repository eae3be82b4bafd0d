"""Byte counts the source pages print, checked against the formats and the
workload accounting used here (CPU only).

* "The Shape That Actually Matters" (The instrument came first): the bf16
  decode matrix of the M=1, K=4096, N=12288 GEMV is 100.7 MB, and eight
  rotating buffers make an 805 MB working set.
* The same page (Round 1, Round 2): its 8-bit arm is 56.6 MB for that matrix,
  a byte ratio of 0.563 against bf16: both are 36 bytes per 32 elements, not
  the 34-byte q8_0 block this path uses (a different block; see the oracle's
  format notes).
* The RX 6700 XT Llama 2 7B write-up (Approach & Methodology): 62 grouped
  launches, 32 QKV and 30 feed-forward, carry 156 logical projections, i.e.
  three projections per QKV launch and two per gate/up launch, the grouping
  of the fused entry points here.
"""

import oracle
import skinny_gemm_decode_amd as skg

N, K = 12288, 4096


def test_bf16_decode_matrix_bytes():
    size = skg.packed_size(skg.BF16_BF16, N, K)
    assert size == N * K * oracle.BF16_BYTES == 100_663_296
    assert round(size / 1e6, 1) == 100.7
    assert round(8 * size / 1e6) == 805


def test_the_pages_8bit_arm_is_a_36_byte_block():
    q8 = N * K // 32 * 36
    assert round(q8 / 1e6, 1) == 56.6
    assert q8 / (N * K * oracle.BF16_BYTES) == 0.5625   # printed as 0.563 (half rounded up)
    # the q8_0 block of this path is 34 bytes: a different, smaller matrix
    ours = skg.packed_size(skg.Q8_0_F32, N, K)
    assert ours == N * K // 32 * oracle.Q8_0_BLOCK_BYTES == N * K // 32 * 34


def test_grouped_projection_count():
    qkv_launches, ffn_launches = 32, 30
    qkv_per_launch = 3   # gemv_multi with the Q, K and V matrices
    ffn_per_launch = 2   # gemv_multi with gate and up (SwiGLU epilogue)
    assert qkv_launches + ffn_launches == 62
    assert qkv_launches * qkv_per_launch + ffn_launches * ffn_per_launch == 156
    assert skg.packed_size_multi(skg.Q4_0_Q8_1, [4096] * 3, 4096) == 3 * skg.packed_size(skg.Q4_0_Q8_1, 4096, 4096)
