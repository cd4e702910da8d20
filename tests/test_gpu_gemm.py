"""GPU parity: MXFP4 x MXFP4 block-scaled GEMM against the oracle's binary64
product of the dequantized operands.

Tolerance: the summation order inside the scaled MFMA and across K steps is
the hardware's, so parity is a bound, not bit equality.  With fp32
accumulation over K = 8192 the expected relative error is about
sqrt(K / 32) * 2^-24 ~ 1e-6; the bound is a relative Frobenius error of 1e-5
on the fp32 output.  The bf16 output must equal the round-to-nearest-even of
the fp32 output element by element (it is the same accumulation, rounded
once).  Integer-valued products are exact and must match bit for bit."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import oracle.gemm as og
import workloads
from tests._gpu import announce, dev

pytestmark = pytest.mark.gpu

REL_FROB = 1e-5


def _operands(M, N, K, seed=0):
    a, bt = workloads.gemm_operands(M, N, K, seed_a=seed, seed_b=seed + 1)
    ap, asc, f1 = oracle.mx_quantize(a.numpy())
    bp, bsc, f2 = oracle.mx_quantize(bt.numpy())
    assert f1 == 0 and f2 == 0
    return ap, asc, bp, bsc


def _run(ap, asc, bp, bsc, M, N, K, out_dtype):
    return fp4.gemm_mxfp4(dev(torch.from_numpy(ap.reshape(M, K // 2))),
                          dev(torch.from_numpy(asc.reshape(M, K // 32))),
                          dev(torch.from_numpy(bp.reshape(N, K // 2))),
                          dev(torch.from_numpy(bsc.reshape(N, K // 32))), out_dtype)


def _check(M, N, K, seed=0):
    ap, asc, bp, bsc = _operands(M, N, K, seed)
    announce(f"gemm mxfp4 {M}x{N}x{K} fp32 out")
    c32 = _run(ap, asc, bp, bsc, M, N, K, torch.float32)
    announce(f"gemm mxfp4 {M}x{N}x{K} bf16 out")
    c16 = _run(ap, asc, bp, bsc, M, N, K, torch.bfloat16)
    torch.cuda.synchronize()
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    got = c32.cpu().numpy().astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"{M}x{N}x{K}: relative Frobenius error {err:.3e}"
    want16 = c32.cpu().to(torch.bfloat16)
    assert torch.equal(c16.cpu().view(torch.int16), want16.view(torch.int16))
    return err


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (32, 32, 64), (70, 50, 96), (128, 96, 32),
                                   (256, 64, 8192), (1, 33, 4128), (200, 72, 1536), (130, 96, 768),
                                   (96, 40, 8704)])
def test_gemm_small_and_ragged(M, N, K):
    _check(M, N, K)


def test_gemm_integer_valued_is_exact():
    # every product and partial sum is a small integer: exact in fp32
    M, N, K = 64, 64, 256
    a = np.ones((M, K), np.float32) * np.arange(1, M + 1, dtype=np.float32)[:, None] % 4
    b = np.ones((N, K), np.float32) * (np.arange(N, dtype=np.float32)[:, None] % 3 - 1)
    ap, asc, _ = oracle.mx_quantize(a)
    bp, bsc, _ = oracle.mx_quantize(b)
    announce("gemm integer-valued 64x64x256")
    c = _run(ap, asc, bp, bsc, M, N, K, torch.float32).cpu().numpy()
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    assert np.array_equal(c.astype(np.float64), ref)


def test_gemm_full_size_128x8192x8192():
    err = _check(128, 8192, 8192)
    print(f"relative Frobenius error {err:.3e}")


def test_gemm_deterministic():
    ap, asc, bp, bsc = _operands(128, 1024, 2048, seed=4)
    announce("gemm determinism 128x1024x2048")
    c1 = _run(ap, asc, bp, bsc, 128, 1024, 2048, torch.float32)
    c2 = _run(ap, asc, bp, bsc, 128, 1024, 2048, torch.float32)
    assert torch.equal(c1, c2)
