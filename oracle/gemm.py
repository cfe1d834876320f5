"""The consumer linear of the quantized activation: out = dq(A) @ dq(B)^T.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The op's quantized output feeds the next linear directly, without a second
quant of its input (the PR conversation page: quantized linears take the
pre-quantized activation, the static-FP8 kernel passing the FP8 tensor
through, the NVFP4 kernel skipping its own quant).  The consumer computes
out[m, n] = sum_k dq(A)[m, k] * dq(B)[n, k] with B the (N, K) weight in the
same format, stored K-contiguous like the activation, and returns it in bf16.

Dequantization:
  * static FP8: dq(A) = decode_E4M3(A) * a_scale (one fp32 per tensor);
  * MXFP8: dq(A)[m, k] = decode_E4M3(A[m, k]) * 2^(S[m, k // 32] - 127),
    S the E8M0 codes of shape (rows, K / 32) (OCP MX);
  * NVFP4 (the op's NVFP4 output as it stands): dq(A)[m, k] =
    decode_E2M1(c[m, k]) * decode_E4M3(S[m, k // 16]) / gs, c the E2M1 code
    of element k (element 2j in the low nibble of byte j of the row), S read
    from the 128x4-tiled block-scale buffer at swizzle_128x4_offset(m, k //
    16), gs the fp32 global scale the op quantized with (the inverse of the
    quantizer: the op maps y to c with o = gs / decode(S)).

Evaluated in float64 by a library matmul (numpy) of the dequantized
operands: MXFP8 operands and their products are exact in float64 (4-bit
significands times powers of two), static-FP8 operands too (4 + 24 bits);
the products and the K-term sum round at the float64 level (relative error
below K * 2^-52 of sum |a b|, far under the bf16 rounding that follows), and
the result is rounded once to bf16 (round to nearest even).  The pages do
not state the consumer's accumulation precision; the GPU's tolerance is
derived in the parity test.

Parity: pinned by tests/test_oracle_gemm.py against an exact rational
evaluation (Python fractions, element by element) on small inputs, closed
forms (all-ones blocks, a single non-zero product) and the scale laws.
"""

import numpy as np

from .formats import BF16, E2M1, E4M3FN, decode, decode_e8m0, f64_to_bits
from .norm_quant import swizzle_128x4_offset

__all__ = ["dequant_fp8_static", "dequant_mxfp8", "dequant_nvfp4", "gemm_f64", "gemm_fp8_static", "gemm_mxfp8",
           "gemm_nvfp4"]

MX_BLOCK = 32
NVFP4_BLOCK = 16


def dequant_fp8_static(q, scale: float) -> np.ndarray:
    """float64 values of E4M3FN codes times a per-tensor fp32 scale."""
    return decode(np.asarray(q, np.uint8), E4M3FN) * float(np.float32(scale))


def dequant_mxfp8(q, s) -> np.ndarray:
    """float64 values of (rows, K) E4M3FN codes with (rows, K / 32) E8M0
    block scales."""
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.uint8)
    rows, K = q.shape
    if K % MX_BLOCK or s.shape != (rows, K // MX_BLOCK):
        raise ValueError("MXFP8 operand: K % 32 == 0 and scales of shape (rows, K / 32)")
    return decode(q, E4M3FN) * np.repeat(decode_e8m0(s), MX_BLOCK, axis=1)


def dequant_nvfp4(q, s_buf, gs: float, rows: int, K: int) -> np.ndarray:
    """float64 values of (rows, K / 2) packed E2M1 codes with E4M3FN block
    scales in the 128x4-tiled buffer ``s_buf`` (flat uint8) and global scale
    gs: code * scale / gs."""
    q = np.asarray(q, np.uint8)
    if K % (4 * NVFP4_BLOCK) or q.shape != (rows, K // 2):
        raise ValueError("NVFP4 operand: K % 64 == 0 and codes of shape (rows, K / 2)")
    c = np.empty((rows, K), np.uint8)
    c[:, 0::2] = q & 0x0F
    c[:, 1::2] = q >> 4
    mm, bb = np.meshgrid(np.arange(rows), np.arange(K // NVFP4_BLOCK), indexing="ij")
    S = np.asarray(s_buf, np.uint8).reshape(-1)[swizzle_128x4_offset(mm, bb, K)]
    sig = np.repeat(decode(S, E4M3FN), NVFP4_BLOCK, axis=1)
    return decode(c, E2M1) * sig / float(np.float32(gs))


def gemm_f64(a, b) -> np.ndarray:
    """sum_k a[m, k] * b[n, k] in float64 (a library matmul)."""
    return np.asarray(a, np.float64) @ np.asarray(b, np.float64).T


def gemm_fp8_static(a_q, a_scale, b_q, b_scale):
    """(exact float64 result, its bf16 bits) of the static-FP8 consumer."""
    exact = gemm_f64(dequant_fp8_static(a_q, a_scale), dequant_fp8_static(b_q, b_scale))
    return exact, f64_to_bits(exact, BF16)


def gemm_mxfp8(a_q, a_s, b_q, b_s):
    """(exact float64 result, its bf16 bits) of the MXFP8 consumer."""
    exact = gemm_f64(dequant_mxfp8(a_q, a_s), dequant_mxfp8(b_q, b_s))
    return exact, f64_to_bits(exact, BF16)


def gemm_nvfp4(a_q, a_s, a_gs, b_q, b_s, b_gs, M: int, N: int, K: int):
    """(exact float64 result, its bf16 bits) of the NVFP4 consumer."""
    exact = gemm_f64(dequant_nvfp4(a_q, a_s, a_gs, M, K), dequant_nvfp4(b_q, b_s, b_gs, N, K))
    return exact, f64_to_bits(exact, BF16)
