"""Seeded sweep over the GEMM family on generated shapes, each path with the
shapes it takes: fp4_gemm_mxfp4 (whichever of its kernels the shape and the
alignment select), split over K, on packed operands, NVFP4 x NVFP4 (row-major
and packed), and the W4A4 linear in one launch, two launches and on a packed
weight.  Each result
is within the relative Frobenius bound of the oracle's binary64 product, and
its bf16 output equals the RNE of its fp32 output."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import oracle.gemm as og
import workloads
from tests._gpu import announce, dev, oracle_view

pytestmark = pytest.mark.gpu

REL_FROB = 1e-5


def _shape(i, kmult, kmax, nmult=1):
    rng = np.random.default_rng(500 + i)
    M = int(rng.integers(1, 300))
    N = nmult * int(rng.integers(1, 700 // nmult))
    K = kmult * int(rng.integers(1, kmax // kmult + 1))
    return M, N, K


def _mx(M, N, K, seed):
    a, bt = workloads.gemm_operands(M, N, K, seed_a=seed, seed_b=seed + 1)
    ap, asc, f1 = oracle.mx_quantize(a.numpy())
    bp, bsc, f2 = oracle.mx_quantize(bt.numpy())
    assert f1 == 0 and f2 == 0
    return a, ap, asc, bp, bsc


def _close(c32, c16, ref, what):
    err = np.linalg.norm(c32.cpu().numpy().astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err <= REL_FROB, f"{what}: relative Frobenius error {err:.3e}"
    assert torch.equal(c16.cpu().view(torch.int16), c32.cpu().to(torch.bfloat16).view(torch.int16)), what


def _t(x, *shape):
    return dev(torch.from_numpy(np.ascontiguousarray(x).reshape(*shape)))


@pytest.mark.parametrize("i", range(8))
def test_mxfp4_gemm_entry_points(i):
    M, N, K = _shape(i, 32, 6144)
    _, ap, asc, bp, bsc = _mx(M, N, K, 40 + i)
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    ops = (_t(ap, M, K // 2), _t(asc, M, K // 32), _t(bp, N, K // 2), _t(bsc, N, K // 32))
    what = f"sweep {i}: gemm_mxfp4 {M}x{N}x{K}"
    announce(what)
    _close(fp4.gemm_mxfp4(*ops, torch.float32), fp4.gemm_mxfp4(*ops, torch.bfloat16), ref, what)
    if K % 512 == 0 and N % 4 == 0:
        what = f"sweep {i}: gemm_mxfp4_splitk {M}x{N}x{K}"
        announce(what)
        _close(fp4.gemm_mxfp4_splitk(*ops, torch.float32), fp4.gemm_mxfp4_splitk(*ops, torch.bfloat16),
               ref, what)


@pytest.mark.parametrize("i", range(6))
def test_mxfp4_gemm_packed_and_splitk(i):
    M, N, K = _shape(100 + i, 2048, 16384, nmult=4)
    _, ap, asc, bp, bsc = _mx(M, N, K, 60 + i)
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    pa = _t(og.pack_operand(ap, asc, M, K), -1)
    pb = _t(og.pack_operand(bp, bsc, N, K), -1)
    what = f"sweep {i}: gemm_mxfp4_packed {M}x{N}x{K}"
    announce(what)
    _close(fp4.gemm_mxfp4_packed(pa, pb, M, N, K, torch.float32),
           fp4.gemm_mxfp4_packed(pa, pb, M, N, K, torch.bfloat16), ref, what)
    ops = (_t(ap, M, K // 2), _t(asc, M, K // 32), _t(bp, N, K // 2), _t(bsc, N, K // 32))
    what = f"sweep {i}: gemm_mxfp4_splitk {M}x{N}x{K}"
    announce(what)
    _close(fp4.gemm_mxfp4_splitk(*ops, torch.float32), fp4.gemm_mxfp4_splitk(*ops, torch.bfloat16),
           ref, what)


@pytest.mark.parametrize("i", range(6))
def test_nvfp4_gemm(i):
    M, N, K = _shape(200 + i, 16, 4096)
    a, bt = workloads.gemm_operands(M, N, K, seed_a=80 + i, seed_b=81 + i)
    ap, asc, sga, f1 = oracle.nv_quantize(a.numpy().reshape(-1))
    bp, bsc, sgb, f2 = oracle.nv_quantize(bt.numpy().reshape(-1))
    assert f1 == 0 and f2 == 0
    ref = og.nv_gemm_f64(ap, asc, sga, bp, bsc, sgb, M, N, K)
    sa, sb = dev(torch.tensor([float(sga)])), dev(torch.tensor([float(sgb)]))
    ops = (_t(ap, M, K // 2), _t(asc, M, K // 16), sa, _t(bp, N, K // 2), _t(bsc, N, K // 16), sb)
    what = f"sweep {i}: gemm_nvfp4 {M}x{N}x{K}"
    announce(what)
    _close(fp4.gemm_nvfp4(*ops, torch.float32), fp4.gemm_nvfp4(*ops, torch.bfloat16), ref, what)


@pytest.mark.parametrize("i", range(6))
def test_nvfp4_gemm_packed(i):
    M, N, K = _shape(250 + i, 2048, 16384)
    a, bt = workloads.gemm_operands(M, N, K, seed_a=70 + i, seed_b=71 + i)
    ap, asc, sga, f1 = oracle.nv_quantize(a.numpy().reshape(-1))
    bp, bsc, sgb, f2 = oracle.nv_quantize(bt.numpy().reshape(-1))
    assert f1 == 0 and f2 == 0
    ref = og.nv_gemm_f64(ap, asc, sga, bp, bsc, sgb, M, N, K)
    what = f"sweep {i}: pack_nvfp4_operand {M}x{K}, {N}x{K}"
    announce(what)
    pa = fp4.pack_nvfp4_operand(_t(ap, M, K // 2), _t(asc, M, K // 16))
    pb = fp4.pack_nvfp4_operand(_t(bp, N, K // 2), _t(bsc, N, K // 16))
    torch.cuda.synchronize()
    assert np.array_equal(pa.cpu().numpy(), og.nv_pack_operand(ap, asc, M, K)), what
    assert np.array_equal(pb.cpu().numpy(), og.nv_pack_operand(bp, bsc, N, K)), what
    sa, sb = dev(torch.tensor([float(sga)])), dev(torch.tensor([float(sgb)]))
    what = f"sweep {i}: gemm_nvfp4_packed {M}x{N}x{K}"
    announce(what)
    _close(fp4.gemm_nvfp4_packed(pa, sa, pb, sb, M, N, K, torch.float32),
           fp4.gemm_nvfp4_packed(pa, sa, pb, sb, M, N, K, torch.bfloat16), ref, what)


@pytest.mark.parametrize("i", range(6))
def test_linear_modes(i):
    M, N, K = _shape(300 + i, 2048, 8192, nmult=1)
    a, ap, asc, bp, bsc = _mx(M, N, K, 90 + i)
    x = a.to(torch.bfloat16 if i % 2 else torch.float32)
    xp, xs, f = oracle.mx_quantize(oracle_view(x))
    assert f == 0
    ref = og.gemm_f64(xp, xs, bp, bsc, M, N, K)
    bt_d, bs_d = _t(bp, N, K // 2), _t(bsc, N, K // 32)
    for one in (True, False):
        what = f"sweep {i}: linear_mxfp4 one_launch={one} {M}x{N}x{K} {x.dtype}"
        announce(what)
        c32, _ = fp4.linear_mxfp4(dev(x), bt_d, bs_d, torch.float32, one_launch=one)
        c16, _ = fp4.linear_mxfp4(dev(x), bt_d, bs_d, torch.bfloat16, one_launch=one)
        _close(c32, c16, ref, what)
    what = f"sweep {i}: linear_mxfp4_packed {M}x{N}x{K} {x.dtype}"
    announce(what)
    pb = _t(og.pack_operand(bp, bsc, N, K), -1)
    c32, _ = fp4.linear_mxfp4_packed(dev(x), pb, N, torch.float32)
    c16, _ = fp4.linear_mxfp4_packed(dev(x), pb, N, torch.bfloat16)
    _close(c32, c16, ref, what)
