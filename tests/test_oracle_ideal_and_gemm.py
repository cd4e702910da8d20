"""Pins for the ideal-scale teaching mode (the pages' printed examples) and
for the block-scaled GEMM reference."""
import numpy as np
import torch
import pytest

import oracle
import oracle.gemm as og
import workloads
from tests._golden import keyed, rows


def test_math_summary_worked_examples():
    g = keyed("math_summary_examples.txt")
    x, alpha, qv, xh = map(float, g["ex1"][0])
    c = oracle.ideal_code(x, alpha)
    assert oracle.e2m1_value(c) == qv
    assert oracle.e2m1_value(c) * alpha == pytest.approx(xh)
    vals = [float(v) for v in g["ex2"][0]]
    assert [oracle.e2m1_value(c) * vals[0] for c in range(8)] == vals[1:]
    xs = np.asarray([float(v) for v in g["ex3_x"][0]], np.float32)
    y = oracle.ideal_roundtrip(xs, 6)
    assert [oracle.e2m1_value(oracle.ideal_code(v, np.float32(xs.max() / 6))) for v in xs] == \
        [float(v) for v in g["ex3_q"][0]]
    assert np.float32(np.abs(xs).max()) / np.float32(6) == pytest.approx(float(g["ex3_alpha"][0][0]))
    assert y == pytest.approx([float(v) for v in g["ex3_xhat"][0]], abs=1e-6)
    xs = np.asarray([float(v) for v in g["ex4_x"][0]], np.float32)
    y = oracle.ideal_roundtrip(xs, 4)
    assert [oracle.e2m1_value(oracle.ideal_code(v, np.float32(20.0) / np.float32(6.0))) for v in xs] == \
        [float(v) for v in g["ex4_q"][0]]


def test_block_size_mae_matches_glossary():
    x = workloads.tiny_roundtrip().numpy().reshape(-1)
    for block, mae in rows("block_size_mae.txt"):
        y = oracle.ideal_roundtrip(x, int(block))
        got = float(np.mean(np.abs(y.astype(np.float64) - x.astype(np.float64))))
        assert got == pytest.approx(float(mae), abs=5e-5), block


def test_storage_bytes_match_page():
    for r in rows("storage_bytes.txt"):
        if r[0] == "padded":        # the row-padded layout, pinned with its encoders
            continue
        n, block, gb, want = r
        assert oracle.storage_bytes(int(n), int(block), int(gb)) == int(want)


def test_group_dot_product_example():
    g = keyed("group_dot.txt")
    bx = [float(v) for v in g["group_scales_x"][0]]
    bw = [float(v) for v in g["group_scales_w"][0]]
    # payloads with group dots 16 and -32 (16 * 1*1 and 16 * 2*(-1))
    px = np.asarray([1.0] * 16 + [2.0] * 16)
    pw = np.asarray([1.0] * 16 + [-1.0] * 16)
    dots = [float(np.dot(px[:16], pw[:16])), float(np.dot(px[16:], pw[16:]))]
    assert dots == [float(v) for v in g["group_dots"][0]]
    assert og.block_scaled_dot(px, np.asarray(bx), pw, np.asarray(bw), 16) == float(g["correct"][0][0])
    assert bx[0] * bw[0] * sum(dots) == float(g["wrong"][0][0])


def test_gemm_reference_equals_group_formula_and_integer_case():
    a, bt = workloads.gemm_operands(M=8, N=12, K=128)
    ap, asc, _ = oracle.mx_quantize(a.numpy())
    bp, bsc, _ = oracle.mx_quantize(bt.numpy())
    C = og.gemm_f64(ap, asc, bp, bsc, 8, 12, 128)
    A_codes = oracle.unpack(ap).reshape(8, 128)
    B_codes = oracle.unpack(bp).reshape(12, 128)
    val = np.vectorize(oracle.e2m1_value)
    pa, pb = val(A_codes), val(B_codes)
    sa = 2.0 ** (asc.reshape(8, 4).astype(np.float64) - 127)
    sb = 2.0 ** (bsc.reshape(12, 4).astype(np.float64) - 127)
    for m in range(8):
        for n in range(12):
            want = og.block_scaled_dot(pa[m], sa[m], pb[n], sb[n], 32)
            assert C[m, n] == pytest.approx(want, rel=1e-14, abs=1e-300)
    # a small integer-valued product is exact
    ai = np.full((2, 64), 2.0, np.float32)
    bi = np.full((3, 64), 3.0, np.float32)
    p1, s1, _ = oracle.mx_quantize(ai)
    p2, s2, _ = oracle.mx_quantize(bi)
    assert np.all(og.gemm_f64(p1, s1, p2, s2, 2, 3, 64) == 64 * 6.0)


# ---- NVFP4 x NVFP4 GEMM reference --------------------------------------------

def _e4m3_code(v: float) -> int:
    return [c for c in range(127) if oracle.e4m3_value(c) == v][0]


def test_nv_gemm_reproduces_the_pages_group_dot():
    g = keyed("group_dot.txt")
    bx = [float(v) for v in g["group_scales_x"][0]]
    bw = [float(v) for v in g["group_scales_w"][0]]
    # payloads 1 | 2 against 1 | -1 (codes 2, 4, 2, 10), global scales 1
    ca = np.array([2] * 16 + [4] * 16, np.uint8)
    cb = np.array([2] * 16 + [10] * 16, np.uint8)
    sa = np.array([_e4m3_code(v) for v in bx], np.uint8)
    sb = np.array([_e4m3_code(v) for v in bw], np.uint8)
    C = og.nv_gemm_f64(oracle.pack(ca), sa, 1.0, oracle.pack(cb), sb, 1.0, 1, 1, 32)
    assert C[0, 0] == float(g["correct"][0][0])


def test_nv_gemm_equals_the_group_formula():
    g = torch.Generator().manual_seed(51)
    a = (torch.randn(6, 64, generator=g) * 3).numpy()
    b = (torch.randn(5, 64, generator=g) * 0.1).numpy()
    ap, asc, sga, f1 = oracle.nv_quantize(a.reshape(-1))
    bp, bsc, sgb, f2 = oracle.nv_quantize(b.reshape(-1))
    assert f1 == 0 and f2 == 0
    C = og.nv_gemm_f64(ap, asc, sga, bp, bsc, sgb, 6, 5, 64)
    val = np.vectorize(oracle.e2m1_value)
    pa = val(oracle.unpack(ap).reshape(6, 64))
    pb = val(oracle.unpack(bp).reshape(5, 64))
    sa = np.vectorize(oracle.e4m3_value)(asc.reshape(6, 4))
    sb = np.vectorize(oracle.e4m3_value)(bsc.reshape(5, 4))
    for m in range(6):
        for n in range(5):
            want = float(sga) * float(sgb) * og.block_scaled_dot(pa[m], sa[m], pb[n], sb[n], 16)
            assert C[m, n] == pytest.approx(want, rel=1e-13, abs=1e-300)
    # and the operands dequantize to the NVFP4 values up to the fp32 rounding
    # of s_g * s_b that the elementwise dequantizer applies
    y = oracle.dequantize(oracle.NV, ap, asc, sga).reshape(6, 64)
    Ad = og.nv_dequant_matrix_exact(ap, asc, sga, 6, 64)
    assert np.allclose(y, Ad, rtol=2 ** -22, atol=0)


def test_nv_gemm_integer_case_is_exact():
    # codes 4 (2.0) and 5 (3.0) at block scale 1 (0x38), tensor scales 1 and 2
    ap = oracle.pack(np.full(2 * 64, 4, np.uint8))
    bp = oracle.pack(np.full(3 * 64, 5, np.uint8))
    one = _e4m3_code(1.0)
    asc = np.full(2 * 4, one, np.uint8)
    bsc = np.full(3 * 4, one, np.uint8)
    assert np.all(og.nv_gemm_f64(ap, asc, 1.0, bp, bsc, 2.0, 2, 3, 64) == 64 * 6.0 * 2.0)
