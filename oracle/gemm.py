"""Block-scaled MXFP4 GEMM reference (test infrastructure only).

What it computes ("FP4, FP8 and INT8/INT4" page, tom-jerr.github.io, section
5.1, block-scaled GEMM equation; "NVFP4 / MXFP4 format" page,
charlestar.github.io, section 6): C[m, n] = sum over 32-blocks t of
s^A[m, t] * s^B[n, t] * sum_{k in t} p^A[m, k] * p^B[n, k].

Each dequantized operand value p * 2^e is exact in fp32 (a 2-bit significand
times a power of two), so the product of the oracle-dequantized operands taken
in binary64 equals that sum up to binary64 rounding (relative ~1e-16), far
below any fp32 accumulation error.  numpy's matmul serves as the
binary64 matrix product.

Operand layout: A is [M, K] quantized along K; B is passed transposed as
Bt [N, K], also quantized along K (section 6 of the format page: storing the
weight as N x K makes its last-dimension groups the K groups).
"""
import numpy as np

from . import MX, dequantize


def dequant_matrix(packed: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Oracle MXFP4 dequantization of a [rows, cols] operand into float64."""
    y = dequantize(MX, packed.reshape(-1), scales.reshape(-1))
    return y.astype(np.float64).reshape(rows, cols)


def gemm_f64(a_packed, a_scales, bt_packed, bt_scales, M: int, N: int, K: int) -> np.ndarray:
    """C = A @ B in binary64 from MXFP4 operands A [M, K] and Bt [N, K]."""
    A = dequant_matrix(a_packed, a_scales, M, K)
    Bt = dequant_matrix(bt_packed, bt_scales, N, K)
    return A @ Bt.T


def block_scaled_dot(pa: np.ndarray, sa: np.ndarray, pb: np.ndarray, sb: np.ndarray,
                     group: int) -> float:
    """One output of the block-scaled dot product, summed group by group in
    binary64: sum_g sa[g] * sb[g] * sum_{k in g} pa[k] * pb[k]."""
    total = 0.0
    for g in range(len(sa)):
        sl = slice(g * group, (g + 1) * group)
        total += float(sa[g]) * float(sb[g]) * float(np.dot(pa[sl].astype(np.float64),
                                                            pb[sl].astype(np.float64)))
    return total
