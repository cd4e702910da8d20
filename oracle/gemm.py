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

from . import MX, dequantize, e2m1_value, e4m3_value, unpack


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


# ---- NVFP4 x NVFP4 ------------------------------------------------------------
#
# The same equation with 16-element blocks, E4M3 block scales and one fp32
# tensor scale per operand ("NVFP4 / MXFP4 format" page, section 6:
# Y = a_X a_W sum_g b^X_g b^W_g sum_{k in g} p^X_k p^W_k).  Reading: the
# tensor scales multiply once, outside the sum, as the page factors them; the
# block scales are the exact E4M3 values.  Each dequantized value
# p * b * a carries at most 2 + 4 + 24 significant bits, so it is exact in
# binary64, and the binary64 matrix product equals the equation up to
# binary64 rounding.

def nv_dequant_matrix_exact(packed: np.ndarray, scales: np.ndarray, s_g, rows: int,
                            cols: int) -> np.ndarray:
    """p * E4M3(s_b) * s_g in binary64 for a [rows, cols] NVFP4 operand."""
    codes = unpack(np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1))
    pv = np.array([e2m1_value(c) for c in range(16)])[codes]
    # any E4M3FN byte: the sign bit, then the magnitude code (0x7F is NaN)
    mag = np.array([e4m3_value(c) if c < 127 else np.nan for c in range(128)])
    sv = np.concatenate([mag, -mag])
    sb = sv[np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1)]
    return (pv.reshape(-1, 16) * sb[:, None] * float(np.float32(s_g))).reshape(rows, cols)


def nv_gemm_f64(a_packed, a_scales, sg_a, bt_packed, bt_scales, sg_b, M: int, N: int,
                K: int) -> np.ndarray:
    """C = A @ B in binary64 from NVFP4 operands A [M, K] and Bt [N, K]."""
    A = nv_dequant_matrix_exact(a_packed, a_scales, sg_a, M, K)
    Bt = nv_dequant_matrix_exact(bt_packed, bt_scales, sg_b, N, K)
    return A @ Bt.T


# ---- MFMA operand order (the packed operand layout) ----------------------------
#
# Not a layout the pages fix: OCP leaves the physical arrangement of elements
# and scales to the implementation ("NVFP4 / MXFP4 format" page, section 7).
# It is the arrangement the library's packed GEMM reads.  For row tile rt
# (32 rows, the last padded with zero codes and scale byte 127) and K step ks
# (64 values), lane l of a 64-lane operand holds row 32 rt + l % 32 and K
# block 2 ks + l // 32 (16 code bytes); after all codes, the scale of that
# lane's block in step 8 q + i sits at byte 8 l + i of the tile's 512-byte
# scale group q.

def packed_bytes(rows: int, K: int) -> int:
    nrt = (rows + 31) // 32
    return nrt * 32 * (K // 2) + nrt * 32 * (K // 32)


def pack_operand(codes: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Row-major MXFP4 operand (codes [rows, K/2], scales [rows, K/32]) to the
    packed layout, one byte at a time in the order the layout lists them."""
    nrt, nks = (rows + 31) // 32, K // 64
    c = np.zeros((nrt * 32, K // 2), np.uint8)
    c[:rows] = np.asarray(codes, np.uint8).reshape(rows, K // 2)
    s = np.full((nrt * 32, K // 32), 127, np.uint8)
    s[:rows] = np.asarray(scales, np.uint8).reshape(rows, K // 32)
    out_c = np.zeros((nrt, nks, 64, 16), np.uint8)
    out_s = np.zeros((nrt, nks // 8, 64, 8), np.uint8)
    for l in range(64):
        row = np.arange(nrt)[:, None] * 32 + l % 32          # [nrt, 1]
        blk = 2 * np.arange(nks)[None, :] + l // 32          # [1, nks]
        for b in range(16):
            out_c[:, :, l, b] = c[row, 16 * blk + b]
        for i in range(8):
            step = 8 * np.arange(nks // 8)[None, :] + i
            out_s[:, :, l, i] = s[row, 2 * step + l // 32]
    return np.concatenate([out_c.reshape(-1), out_s.reshape(-1)])


def gemm_from_packed(a_packed: np.ndarray, bt_packed: np.ndarray, M: int, N: int,
                     K: int) -> np.ndarray:
    """C = A @ B in binary64, reading both operands the way the scaled MFMA
    consumes them (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands: lane l
    supplies row or column l % 32 and the 32 K values from 32 (l // 32) of
    the 64-wide step, with its own E8M0 byte): for every pair of row tiles and
    every K step, the 32 x 64 slices from the 64 lanes, multiplied and added.
    Written from the consumer's side, independently of pack_operand."""
    mag = np.array([e2m1_value(c) for c in range(16)])

    def tiles(packed, rows):
        nrt, nks = (rows + 31) // 32, K // 64
        codes = np.asarray(packed[:nrt * nks * 1024], np.uint8).reshape(nrt, nks, 64, 16)
        scl = np.asarray(packed[nrt * nks * 1024:], np.uint8).reshape(nrt, nks // 8, 64, 8)
        vals = np.zeros((nrt, nks, 32, 64))                   # [tile, step, row, K in step]
        for l in range(64):
            lo, hi = codes[:, :, l, :] & 15, codes[:, :, l, :] >> 4
            v = np.stack([mag[lo], mag[hi]], axis=-1).reshape(nrt, nks, 32)  # even element low
            e = scl[:, :, l, :].reshape(nrt, nks).astype(np.int64) - 127
            vals[:, :, l % 32, 32 * (l // 32):32 * (l // 32) + 32] = v * np.ldexp(1.0, e)[:, :, None]
        return vals

    A, B = tiles(a_packed, M), tiles(bt_packed, N)
    C = np.zeros((A.shape[0] * 32, B.shape[0] * 32))
    for ks in range(K // 64):
        C += np.einsum("irk,jck->irjc", A[:, ks], B[:, ks]).reshape(A.shape[0] * 32, B.shape[0] * 32)
    return C[:M, :N]


# ---- NVFP4 in MFMA operand order ------------------------------------------------
#
# Also the implementation's own arrangement (section 7 of the format page
# leaves it open).  Codes are arranged as for MXFP4 above; the E4M3 block
# scales (16 values each) follow all codes: for row tile rt and group q of
# eight K steps, 1024 bytes, byte 16 l + 2 i + b holding the scale of row
# 32 rt + l % 32 and block 4 (8 q + i) + 2 (l // 32) + b; padding rows hold 0.

def nv_packed_bytes(rows: int, K: int) -> int:
    nrt = (rows + 31) // 32
    return nrt * 32 * (K // 2) + nrt * 32 * (K // 16)


def nv_pack_operand(codes: np.ndarray, scales: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Row-major NVFP4 operand (codes [rows, K/2], E4M3 scales [rows, K/16])
    to the packed NVFP4 layout, byte by byte in the order the layout lists."""
    nrt, nks = (rows + 31) // 32, K // 64
    c = np.zeros((nrt * 32, K // 2), np.uint8)
    c[:rows] = np.asarray(codes, np.uint8).reshape(rows, K // 2)
    s = np.zeros((nrt * 32, K // 16), np.uint8)
    s[:rows] = np.asarray(scales, np.uint8).reshape(rows, K // 16)
    out_c = np.zeros((nrt, nks, 64, 16), np.uint8)
    out_s = np.zeros((nrt, nks // 8, 64, 16), np.uint8)
    for l in range(64):
        row = np.arange(nrt)[:, None] * 32 + l % 32
        blk = 2 * np.arange(nks)[None, :] + l // 32           # 32-value block of this lane
        for b in range(16):
            out_c[:, :, l, b] = c[row, 16 * blk + b]
        for i in range(8):
            step = 8 * np.arange(nks // 8)[None, :] + i
            for b in range(2):
                out_s[:, :, l, 2 * i + b] = s[row, 4 * step + 2 * (l // 32) + b]
    return np.concatenate([out_c.reshape(-1), out_s.reshape(-1)])


def nv_gemm_from_packed(a_packed: np.ndarray, sg_a, bt_packed: np.ndarray, sg_b, M: int,
                        N: int, K: int) -> np.ndarray:
    """C = A @ B in binary64 from two packed NVFP4 operands, read the way the
    fp16 MFMA (v_mfma_f32_32x32x16_f16) consumes them: in sub-step u (0..3)
    of a 64-value step, lane l supplies row l % 32 and the eight values in
    bytes 4 u .. 4 u + 3 of its 16, times the E4M3 byte 2 i + (u >= 2) of
    its scale word, into K slots 8 (l // 32) .. + 7; both operands use the
    same slots, so the step adds all 64 products.  Written from the consumer's
    side, independently of nv_pack_operand."""
    ev = np.array([e2m1_value(c) for c in range(16)])
    mag = np.array([e4m3_value(c) if c < 127 else np.nan for c in range(128)])
    sv = np.concatenate([mag, -mag])

    def tiles(packed, rows):
        nrt, nks = (rows + 31) // 32, K // 64
        codes = np.asarray(packed[:nrt * nks * 1024], np.uint8).reshape(nrt, nks, 64, 16)
        scl = np.asarray(packed[nrt * nks * 1024:], np.uint8).reshape(nrt, nks // 8, 64, 16)
        vals = np.zeros((nrt, nks, 4, 32, 16))                  # [tile, step, u, row, slot]
        for l in range(64):
            sc = scl[:, :, l, :].reshape(nrt, nks, 2)            # [tile, step, b]
            for u in range(4):
                w = codes[:, :, l, 4 * u:4 * u + 4]
                v = np.stack([ev[w & 15], ev[w >> 4]], axis=-1).reshape(nrt, nks, 8)
                slot = 8 * (l // 32)
                vals[:, :, u, l % 32, slot:slot + 8] = v * sv[sc[:, :, u // 2]][:, :, None]
        return vals

    A, B = tiles(a_packed, M), tiles(bt_packed, N)
    C = np.zeros((A.shape[0] * 32, B.shape[0] * 32))
    for ks in range(K // 64):
        for u in range(4):
            C += np.einsum("irk,jck->irjc", A[:, ks, u], B[:, ks, u]).reshape(C.shape)
    return C[:M, :N] * float(np.float32(sg_a)) * float(np.float32(sg_b))
