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
from tests._gpu import announce, assert_bytes_equal, dev, host_u8, oracle_view

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
                                   (96, 40, 8704), (64, 96, 256), (33, 64, 20736)])
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


def test_gemm_full_size_128x8192x16384():
    # K past 8192 takes the same LDS-staged kernel (the scales stream with
    # the codes, so K has no upper limit)
    err = _check(128, 8192, 16384)
    print(f"relative Frobenius error {err:.3e}")


def test_gemm_deterministic():
    ap, asc, bp, bsc = _operands(128, 1024, 2048, seed=4)
    announce("gemm determinism 128x1024x2048")
    c1 = _run(ap, asc, bp, bsc, 128, 1024, 2048, torch.float32)
    c2 = _run(ap, asc, bp, bsc, 128, 1024, 2048, torch.float32)
    assert torch.equal(c1, c2)


# ---- split over K: fp32 partials per K range, fixed-order reduction ------------

def _run_splitk(ap, asc, bp, bsc, M, N, K, out_dtype, workspace=None):
    return fp4.gemm_mxfp4_splitk(dev(torch.from_numpy(ap.reshape(M, K // 2))),
                                 dev(torch.from_numpy(asc.reshape(M, K // 32))),
                                 dev(torch.from_numpy(bp.reshape(N, K // 2))),
                                 dev(torch.from_numpy(bsc.reshape(N, K // 32))), out_dtype,
                                 workspace=workspace)


def _check_splitk(M, N, K, seed=0, workspace=None):
    ap, asc, bp, bsc = _operands(M, N, K, seed)
    parts = fp4.gemm_splitk_workspace_bytes(M, N, K) // (4 * M * N)
    announce(f"gemm mxfp4 split-K ({parts} ranges) {M}x{N}x{K} fp32 out")
    c32 = _run_splitk(ap, asc, bp, bsc, M, N, K, torch.float32, workspace)
    announce(f"gemm mxfp4 split-K {M}x{N}x{K} bf16 out")
    c16 = _run_splitk(ap, asc, bp, bsc, M, N, K, torch.bfloat16, workspace)
    torch.cuda.synchronize()
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    got = c32.cpu().numpy().astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"split-K {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    # bf16 is the same fixed-order fp32 sum, rounded once
    want16 = c32.cpu().to(torch.bfloat16)
    assert torch.equal(c16.cpu().view(torch.int16), want16.view(torch.int16))
    return err


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 8, 512), (70, 52, 2560), (200, 72, 3072),
                                   (256, 132, 4096), (33, 516, 1024), (130, 100, 16384)])
def test_gemm_splitk_small_and_ragged(M, N, K):
    _check_splitk(M, N, K)


def test_gemm_splitk_full_size_128x8192x8192():
    err = _check_splitk(128, 8192, 8192)
    print(f"relative Frobenius error {err:.3e}")


def test_gemm_splitk_integer_valued_is_exact():
    # small-integer products and sums: every partial and their sum are exact
    M, N, K = 64, 64, 4096
    a = np.ones((M, K), np.float32) * np.arange(1, M + 1, dtype=np.float32)[:, None] % 4
    b = np.ones((N, K), np.float32) * (np.arange(N, dtype=np.float32)[:, None] % 3 - 1)
    ap, asc, _ = oracle.mx_quantize(a)
    bp, bsc, _ = oracle.mx_quantize(b)
    announce("gemm split-K integer-valued 64x64x4096")
    c = _run_splitk(ap, asc, bp, bsc, M, N, K, torch.float32).cpu().numpy()
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    assert np.array_equal(c.astype(np.float64), ref)


def test_gemm_splitk_deterministic_and_workspace_reuse():
    ws = torch.empty(fp4.gemm_splitk_workspace_bytes(128, 8192, 8192), dtype=torch.uint8,
                     device="cuda")
    ap, asc, bp, bsc = _operands(128, 1024, 8192, seed=4)
    announce("gemm split-K determinism 128x1024x8192")
    c1 = _run_splitk(ap, asc, bp, bsc, 128, 1024, 8192, torch.float32, ws)
    # a smaller call in between leaves other partials in the same workspace
    _check_splitk(70, 52, 2560, seed=5, workspace=ws)
    c2 = _run_splitk(ap, asc, bp, bsc, 128, 1024, 8192, torch.float32, ws)
    assert torch.equal(c1, c2)
    # the unsplit kernel sums in another order: both within the bound
    c0 = _run(ap, asc, bp, bsc, 128, 1024, 8192, torch.float32)
    rel = (torch.linalg.norm((c1 - c0).double()) / torch.linalg.norm(c0.double())).item()
    assert rel <= 2 * REL_FROB


# ---- W4A4 linear: activation quantize + GEMM in one call -----------------------

def _check_linear(M, N, K, x_dtype=torch.float32, seed=0, workspace=None):
    a, bt = workloads.gemm_operands(M, N, K, seed_a=seed, seed_b=seed + 1)
    x = a.to(x_dtype)
    bp, bsc, f2 = oracle.mx_quantize(bt.numpy())
    assert f2 == 0
    ap, asc, f1 = oracle.mx_quantize(oracle_view(x))
    assert f1 == 0
    bt_d = dev(torch.from_numpy(bp.reshape(N, K // 2)))
    bs_d = dev(torch.from_numpy(bsc.reshape(N, K // 32)))
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    ws = workspace if workspace is not None else fp4.new_workspace(M, K, "cuda")
    announce(f"linear mxfp4 {M}x{N}x{K} x {x_dtype} fp32 out")
    c32, (ac, asd) = fp4.linear_mxfp4(dev(x), bt_d, bs_d, torch.float32, workspace=ws)
    announce(f"linear mxfp4 {M}x{N}x{K} x {x_dtype} bf16 out")
    c16, _ = fp4.linear_mxfp4(dev(x), bt_d, bs_d, torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    assert_bytes_equal(host_u8(asd), asc, f"linear {M}x{N}x{K}: A scales")
    assert_bytes_equal(host_u8(ac), ap, f"linear {M}x{N}x{K}: A codes")
    got = c32.cpu().numpy().astype(np.float64)
    err = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err <= REL_FROB, f"linear {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    want16 = c32.cpu().to(torch.bfloat16)
    assert torch.equal(c16.cpu().view(torch.int16), want16.view(torch.int16))
    # the same as the separate entry points, bit for bit, and as two launches
    c_sep = _run(ap, asc, bp, bsc, M, N, K, torch.float32)
    assert torch.equal(c32.cpu(), c_sep.cpu())
    announce(f"linear mxfp4 {M}x{N}x{K} two launches")
    c2, (ac2, as2) = fp4.linear_mxfp4(dev(x), bt_d, bs_d, torch.float32, workspace=ws,
                                      one_launch=False)
    assert torch.equal(c2.cpu(), c32.cpu())
    assert torch.equal(ac2.cpu(), ac.cpu()) and torch.equal(as2.cpu(), asd.cpu())
    return err


@pytest.mark.parametrize("M,N,K,dt", [(128, 8192, 8192, torch.float32),    # one launch, full size
                                      (128, 8192, 8192, torch.bfloat16),
                                      (128, 256, 512, torch.bfloat16),      # one launch, small grid
                                      (70, 50, 1024, torch.float32),        # ragged M and N
                                      (96, 40, 96, torch.float32),          # K % 512 != 0: two launches
                                      (128, 16384, 1024, torch.bfloat16)])  # grid above the CU count
def test_linear_matches_quantize_then_gemm(M, N, K, dt):
    _check_linear(M, N, K, dt)


def test_linear_workspace_shared_with_nvfp4_and_reused():
    ws = fp4.new_workspace(128, 8192, "cuda")
    for seed in range(3):
        _check_linear(128, 1024, 2048, torch.bfloat16, seed=seed, workspace=ws)
        x = workloads.nvfp4_weight(512, 4096, seed=seed).cuda()
        announce(f"nvfp4 quantize on the shared workspace, seed {seed}")
        codes, scales, sg = fp4.quantize_nvfp4(x, workspace=ws)
        p, s, sgo, f = oracle.nv_quantize(oracle_view(x.cpu()))
        assert_bytes_equal(host_u8(scales), s, "nvfp4 scales after linear")


def test_linear_flags_nonfinite_activations():
    M, N, K = 128, 256, 512
    a, bt = workloads.gemm_operands(M, N, K)
    bp, bsc, _ = oracle.mx_quantize(bt.numpy())
    x = a.clone()
    x[5, 7] = float("inf")
    with pytest.raises(ValueError):
        fp4.linear_mxfp4(dev(x), dev(torch.from_numpy(bp.reshape(N, K // 2))),
                         dev(torch.from_numpy(bsc.reshape(N, K // 32))))


# ---- NVFP4 x NVFP4 ---------------------------------------------------------------

def _nv_operands(M, N, K, seed=0):
    a, bt = workloads.gemm_operands(M, N, K, seed_a=seed, seed_b=seed + 1)
    ap, asc, sga, f1 = oracle.nv_quantize(a.numpy().reshape(-1))
    bp, bsc, sgb, f2 = oracle.nv_quantize(bt.numpy().reshape(-1))
    assert f1 == 0 and f2 == 0
    return ap, asc, sga, bp, bsc, sgb


def _run_nv(ap, asc, sga, bp, bsc, sgb, M, N, K, out_dtype):
    t = lambda v: dev(torch.tensor([float(v)], dtype=torch.float32))
    return fp4.gemm_nvfp4(dev(torch.from_numpy(ap.reshape(M, K // 2))),
                          dev(torch.from_numpy(asc.reshape(M, K // 16))), t(sga),
                          dev(torch.from_numpy(bp.reshape(N, K // 2))),
                          dev(torch.from_numpy(bsc.reshape(N, K // 16))), t(sgb), out_dtype)


def _check_nv(ops, M, N, K, what):
    ap, asc, sga, bp, bsc, sgb = ops
    announce(f"gemm nvfp4 {what} {M}x{N}x{K} fp32 out")
    c32 = _run_nv(ap, asc, sga, bp, bsc, sgb, M, N, K, torch.float32)
    announce(f"gemm nvfp4 {what} {M}x{N}x{K} bf16 out")
    c16 = _run_nv(ap, asc, sga, bp, bsc, sgb, M, N, K, torch.bfloat16)
    torch.cuda.synchronize()
    ref = og.nv_gemm_f64(ap, asc, sga, bp, bsc, sgb, M, N, K)
    got = c32.cpu().numpy().astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"nvfp4 {what} {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    assert torch.equal(c16.cpu().view(torch.int16), c32.cpu().to(torch.bfloat16).view(torch.int16))
    return err


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (70, 50, 256), (1, 33, 4096), (200, 72, 1536),
                                   (96, 40, 272), (64, 64, 8448), (3, 5, 16)])
def test_gemm_nvfp4_small_and_ragged(M, N, K):
    _check_nv(_nv_operands(M, N, K), M, N, K, "random")


def test_gemm_nvfp4_full_size_128x8192x8192():
    err = _check_nv(_nv_operands(128, 8192, 8192), 128, 8192, 8192, "full size")
    print(f"relative Frobenius error {err:.3e}")


def test_gemm_nvfp4_every_code_under_every_scale():
    # A: row r takes block scale code (r % 126) + 1 on every block and the
    # sixteen FP4 codes in each block; B: a fixed random NVFP4 operand
    M, N, K = 126, 64, 512
    codes = np.tile(np.arange(16, dtype=np.uint8), M * K // 16)
    ap = oracle.pack(codes)
    asc = np.repeat((np.arange(M) % 126 + 1).astype(np.uint8), K // 16)
    _, _, _, bp, bsc, sgb = _nv_operands(8, N, K, seed=7)
    for sga in (1.0, 2.0 ** -20, 3.0):
        _check_nv((ap, asc, np.float32(sga), bp, bsc, sgb), M, N, K, f"every code, s_gA={sga}")


def test_gemm_nvfp4_integer_case_is_exact():
    M, N, K = 64, 48, 256
    ap = oracle.pack(np.full(M * K, 4, np.uint8))          # 2.0
    bp = oracle.pack(np.full(N * K, 5, np.uint8))          # 3.0
    asc = np.full(M * K // 16, 0x38, np.uint8)             # scale 1
    bsc = np.full(N * K // 16, 0x38, np.uint8)
    c = _run_nv(ap, asc, 1.0, bp, bsc, 2.0, M, N, K, torch.float32).cpu().numpy()
    assert np.all(c == K * 6.0 * 2.0)


def test_gemm_nvfp4_deterministic():
    ops = _nv_operands(128, 1024, 2048, seed=4)
    c1 = _run_nv(*ops, 128, 1024, 2048, torch.float32)
    c2 = _run_nv(*ops, 128, 1024, 2048, torch.float32)
    assert torch.equal(c1, c2)


# ---- packed operands (MFMA operand order) ---------------------------------------

def _packed_case(M, N, K, seed=0):
    ap, asc, bp, bsc = _operands(M, N, K, seed)
    announce(f"pack mxfp4 operands {M}x{K} and {N}x{K}")
    pa = fp4.pack_mxfp4_operand(dev(torch.from_numpy(ap.reshape(M, K // 2))),
                                dev(torch.from_numpy(asc.reshape(M, K // 32))))
    pb = fp4.pack_mxfp4_operand(dev(torch.from_numpy(bp.reshape(N, K // 2))),
                                dev(torch.from_numpy(bsc.reshape(N, K // 32))))
    torch.cuda.synchronize()
    assert_bytes_equal(host_u8(pa), og.pack_operand(ap, asc, M, K), f"packed A {M}x{K}")
    if N * K <= 2048 * 8192:
        assert_bytes_equal(host_u8(pb), og.pack_operand(bp, bsc, N, K), f"packed Bt {N}x{K}")
    return ap, asc, bp, bsc, pa, pb


def _check_packed(M, N, K, seed=0):
    ap, asc, bp, bsc, pa, pb = _packed_case(M, N, K, seed)
    announce(f"gemm mxfp4 packed {M}x{N}x{K} fp32 and bf16 out")
    c32 = fp4.gemm_mxfp4_packed(pa, pb, M, N, K, torch.float32)
    c16 = fp4.gemm_mxfp4_packed(pa, pb, M, N, K, torch.bfloat16)
    torch.cuda.synchronize()
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    err = np.linalg.norm(c32.cpu().numpy().astype(np.float64) - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"packed {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    want16 = c32.cpu().to(torch.bfloat16)
    assert torch.equal(c16.cpu().view(torch.int16), want16.view(torch.int16))
    return err


@pytest.mark.parametrize("M,N,K", [(128, 256, 2048), (1, 32, 2048), (70, 100, 2048),
                                   (130, 64, 6144), (256, 512, 4096), (33, 40, 16384),
                                   (96, 33, 10240)])
def test_gemm_packed_small_and_ragged(M, N, K):
    _check_packed(M, N, K)


def test_gemm_packed_full_size_128x8192x8192():
    err = _check_packed(128, 8192, 8192)
    print(f"relative Frobenius error {err:.3e}")


def test_gemm_packed_integer_valued_is_exact_and_deterministic():
    M, N, K = 64, 96, 2048
    a = np.ones((M, K), np.float32) * np.arange(1, M + 1, dtype=np.float32)[:, None] % 4
    b = np.ones((N, K), np.float32) * (np.arange(N, dtype=np.float32)[:, None] % 3 - 1)
    ap, asc, _ = oracle.mx_quantize(a)
    bp, bsc, _ = oracle.mx_quantize(b)
    announce("gemm packed integer-valued 64x96x2048")
    pa = dev(torch.from_numpy(og.pack_operand(ap, asc, M, K)))
    pb = dev(torch.from_numpy(og.pack_operand(bp, bsc, N, K)))
    c1 = fp4.gemm_mxfp4_packed(pa, pb, M, N, K, torch.float32)
    c2 = fp4.gemm_mxfp4_packed(pa, pb, M, N, K, torch.float32)
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    assert np.array_equal(c1.cpu().numpy().astype(np.float64), ref)
    assert torch.equal(c1, c2)


# ---- NVFP4 on packed operands ---------------------------------------------------

def _nv_pack_dev(p, sc, rows, K, what):
    packed = fp4.pack_nvfp4_operand(dev(torch.from_numpy(p.reshape(rows, K // 2))),
                                    dev(torch.from_numpy(sc.reshape(rows, K // 16))))
    torch.cuda.synchronize()
    if rows * K <= 2048 * 8192:
        assert_bytes_equal(host_u8(packed), og.nv_pack_operand(p, sc, rows, K), what)
    return packed


def _check_nv_packed(ops, M, N, K, what):
    ap, asc, sga, bp, bsc, sgb = ops
    announce(f"pack nvfp4 operands {M}x{K} and {N}x{K} ({what})")
    pa = _nv_pack_dev(ap, asc, M, K, f"nv packed A {M}x{K}")
    pb = _nv_pack_dev(bp, bsc, N, K, f"nv packed Bt {N}x{K}")
    t = lambda v: dev(torch.tensor([float(v)], dtype=torch.float32))
    announce(f"gemm nvfp4 packed {what} {M}x{N}x{K} fp32 and bf16 out")
    c32 = fp4.gemm_nvfp4_packed(pa, t(sga), pb, t(sgb), M, N, K, torch.float32)
    c16 = fp4.gemm_nvfp4_packed(pa, t(sga), pb, t(sgb), M, N, K, torch.bfloat16)
    torch.cuda.synchronize()
    ref = og.nv_gemm_f64(ap, asc, sga, bp, bsc, sgb, M, N, K)
    got = c32.cpu().numpy().astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"nvfp4 packed {what} {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    assert torch.equal(c16.cpu().view(torch.int16), c32.cpu().to(torch.bfloat16).view(torch.int16))
    return c32, err


@pytest.mark.parametrize("M,N,K", [(128, 256, 2048), (1, 32, 2048), (70, 100, 2048),
                                   (130, 64, 6144), (256, 96, 8192), (33, 40, 16384)])
def test_gemm_nvfp4_packed_small_and_ragged(M, N, K):
    _check_nv_packed(_nv_operands(M, N, K), M, N, K, "random")


def test_gemm_nvfp4_packed_full_size_128x8192x8192():
    _, err = _check_nv_packed(_nv_operands(128, 8192, 8192), 128, 8192, 8192, "full size")
    print(f"relative Frobenius error {err:.3e}")


def test_gemm_nvfp4_packed_every_code_under_every_scale_of_both_signs():
    # A: row r takes E4M3 byte (r % 126) + 1, with the sign bit on odd rows,
    # on every block and the sixteen FP4 codes in each block
    M, N, K = 252, 64, 2048
    ap = oracle.pack(np.tile(np.arange(16, dtype=np.uint8), M * K // 16))
    r = np.arange(M)
    asc = np.repeat(((r % 126 + 1) | ((r % 2) << 7)).astype(np.uint8), K // 16)
    _, _, _, bp, bsc, sgb = _nv_operands(8, N, K, seed=7)
    for sga in (1.0, 2.0 ** -20):
        _check_nv_packed((ap, asc, np.float32(sga), bp, bsc, sgb), M, N, K,
                         f"every code, s_gA={sga}")


def test_gemm_nvfp4_packed_integer_case_is_exact_and_deterministic():
    M, N, K = 64, 48, 2048
    ap = oracle.pack(np.full(M * K, 4, np.uint8))          # 2.0
    bp = oracle.pack(np.full(N * K, 5, np.uint8))          # 3.0
    asc = np.full(M * K // 16, 0x38, np.uint8)             # scale 1
    bsc = np.full(N * K // 16, 0x40, np.uint8)             # scale 2
    c1, _ = _check_nv_packed((ap, asc, np.float32(1.0), bp, bsc, np.float32(0.5)), M, N, K,
                             "integer")
    assert np.all(c1.cpu().numpy() == K * 6.0)
    ops = _nv_operands(128, 1024, 4096, seed=4)
    ca, _ = _check_nv_packed(ops, 128, 1024, 4096, "repeat 1")
    cb, _ = _check_nv_packed(ops, 128, 1024, 4096, "repeat 2")
    assert torch.equal(ca, cb)


# ---- NVFP4 quantize into the packed layout, and the packed NVFP4 linear ---------

@pytest.mark.parametrize("rows,cols,dt", [(1, 512, torch.float32), (70, 2048, torch.bfloat16),
                                          (128, 8192, torch.bfloat16), (33, 1536, torch.float32)])
def test_quantize_nvfp4_packed_matches_oracle(rows, cols, dt):
    g = torch.Generator().manual_seed(3 * rows + cols)
    x = (torch.randn(rows, cols, generator=g) * torch.rand(rows, cols, generator=g) ** 3).to(dt)
    announce(f"quantize nvfp4 packed {rows}x{cols} {dt}")
    got, sg = fp4.quantize_nvfp4_packed(dev(x))
    torch.cuda.synchronize()
    p, sc, sg_ref, flags = oracle.nv_quantize(oracle_view(x).reshape(-1))
    assert flags == 0
    assert np.float32(sg.item()) == np.float32(sg_ref)
    assert_bytes_equal(host_u8(got), og.nv_pack_operand(p, sc, rows, cols),
                       f"nv packed quantize {rows}x{cols}")


def test_quantize_nvfp4_packed_flags_nonfinite():
    x = torch.zeros(32, 512)
    x[5, 100] = float("inf")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    announce("quantize nvfp4 packed, one inf")
    fp4.quantize_nvfp4_packed(dev(x), check=False, status=st)
    assert int(st.item()) & fp4.FLAG_NONFINITE


@pytest.mark.parametrize("M,N,K,dt", [(128, 8192, 8192, torch.bfloat16), (70, 100, 2048, torch.float32),
                                      (33, 40, 16384, torch.bfloat16)])
def test_linear_nvfp4_packed_matches_oracle(M, N, K, dt):
    a, bt = workloads.gemm_operands(M, N, K, seed_a=11, seed_b=12)
    x = a.to(dt)
    xp, xs, xg, f1 = oracle.nv_quantize(oracle_view(x).reshape(-1))
    bp, bsc, bg, f2 = oracle.nv_quantize(bt.numpy().reshape(-1))
    assert f1 == 0 and f2 == 0
    pb = _nv_pack_dev(bp, bsc, N, K, f"nv packed Bt {N}x{K}")
    t = lambda v: dev(torch.tensor([float(v)], dtype=torch.float32))
    announce(f"linear nvfp4 packed {M}x{N}x{K} {dt}")
    c32, (apk, ag) = fp4.linear_nvfp4_packed(dev(x), pb, t(bg), N, torch.float32)
    c16, _ = fp4.linear_nvfp4_packed(dev(x), pb, t(bg), N, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.float32(ag.item()) == np.float32(xg)
    assert_bytes_equal(host_u8(apk), og.nv_pack_operand(xp, xs, M, K), f"linear nv packed A {M}x{K}")
    ref = og.nv_gemm_f64(xp, xs, xg, bp, bsc, bg, M, N, K)
    err = np.linalg.norm(c32.cpu().numpy().astype(np.float64) - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"linear nvfp4 packed {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    assert torch.equal(c16.cpu().view(torch.int16), c32.cpu().to(torch.bfloat16).view(torch.int16))


# ---- quantize straight into the packed layout, and the packed W4A4 linear ------

@pytest.mark.parametrize("rows,cols,dt", [(1, 512, torch.float32), (70, 2048, torch.bfloat16),
                                          (128, 8192, torch.bfloat16), (33, 1536, torch.float32)])
def test_quantize_mxfp4_packed_matches_oracle(rows, cols, dt):
    g = torch.Generator().manual_seed(rows + cols)
    x = (torch.randn(rows, cols, generator=g) * torch.rand(rows, cols, generator=g) ** 3).to(dt)
    announce(f"quantize mxfp4 packed {rows}x{cols} {dt}")
    got = fp4.quantize_mxfp4_packed(dev(x))
    torch.cuda.synchronize()
    p, s, flags = oracle.mx_quantize(oracle_view(x))
    assert flags == 0
    assert_bytes_equal(host_u8(got), og.pack_operand(p, s, rows, cols), f"packed quantize {rows}x{cols}")


def test_quantize_mxfp4_packed_flags_nonfinite():
    x = torch.zeros(32, 512)
    x[3, 100] = float("inf")
    announce("quantize mxfp4 packed non-finite")
    with pytest.raises(ValueError):
        fp4.quantize_mxfp4_packed(dev(x))


@pytest.mark.parametrize("M,N,K,dt", [(128, 8192, 8192, torch.bfloat16), (70, 100, 2048, torch.float32),
                                      (200, 96, 4096, torch.bfloat16)])
def test_linear_packed_matches_oracle(M, N, K, dt):
    a, bt = workloads.gemm_operands(M, N, K, seed_a=2, seed_b=3)
    x = a.to(dt)
    bp, bsc, f2 = oracle.mx_quantize(bt.numpy())
    ap, asc, f1 = oracle.mx_quantize(oracle_view(x))
    assert f1 == 0 and f2 == 0
    bt_packed = dev(torch.from_numpy(og.pack_operand(bp, bsc, N, K)))
    announce(f"linear mxfp4 packed {M}x{N}x{K} {dt}")
    c32, a_packed = fp4.linear_mxfp4_packed(dev(x), bt_packed, N, torch.float32)
    c16, _ = fp4.linear_mxfp4_packed(dev(x), bt_packed, N, torch.bfloat16)
    torch.cuda.synchronize()
    assert_bytes_equal(host_u8(a_packed), og.pack_operand(ap, asc, M, K), f"linear {M}x{N}x{K}: packed A")
    ref = og.gemm_f64(ap, asc, bp, bsc, M, N, K)
    err = np.linalg.norm(c32.cpu().numpy().astype(np.float64) - ref) / np.linalg.norm(ref)
    assert err <= REL_FROB, f"linear packed {M}x{N}x{K}: relative Frobenius error {err:.3e}"
    assert torch.equal(c16.cpu().view(torch.int16), c32.cpu().to(torch.bfloat16).view(torch.int16))
    # the same bits as the packed GEMM on the same packed operands
    c2 = fp4.gemm_mxfp4_packed(a_packed, bt_packed, M, N, K, torch.float32)
    assert torch.equal(c2, c32)


def test_packed_binding_rejects_bad_scales_and_global_scales():
    # checked in Python before any launch: the C calls take no size for the
    # scale buffers, and the tensor scales are read on the device
    rows, K = 64, 512
    codes = torch.zeros(rows, K // 2, dtype=torch.uint8, device="cuda")
    good_nv = torch.zeros(rows, K // 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fp4.pack_nvfp4_operand(codes, good_nv[:, :-1].contiguous())      # short
    with pytest.raises(TypeError):
        fp4.pack_nvfp4_operand(codes, good_nv.float())                    # dtype
    with pytest.raises(ValueError):
        fp4.pack_nvfp4_operand(codes, good_nv.cpu())                      # host memory
    with pytest.raises(ValueError):
        fp4.pack_mxfp4_operand(codes, torch.zeros(rows, K // 16, dtype=torch.uint8, device="cuda"))
    ap = fp4.pack_nvfp4_operand(codes, good_nv)
    sg = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fp4.gemm_nvfp4_packed(ap, sg.cpu(), ap, sg, rows, rows, K)
    with pytest.raises(TypeError):
        fp4.gemm_nvfp4_packed(ap, sg, ap, sg.double(), rows, rows, K)
    with pytest.raises(ValueError):
        fp4.gemm_nvfp4_packed(ap, sg[:0], ap, sg, rows, rows, K)
    x = torch.zeros(rows, K, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        fp4.linear_nvfp4_packed(x, ap, sg.half(), rows)
    torch.cuda.synchronize()
