"""GPU parity: dequantization (bit-exact, fp32 and bf16 outputs) and the
MSE-optimal NVFP4 scale search (bit-exact codes and scale bytes)."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import (announce, assert_bytes_equal, assert_float_bits_equal, dev, f32_bits,
                        host_u8, oracle_view)

pytestmark = pytest.mark.gpu


def _dq_check(fmt, packed: np.ndarray, scales: np.ndarray, s_g: float, rows: int, what: str):
    cols = packed.size * 2 // rows
    codes_d = dev(torch.from_numpy(packed.reshape(rows, cols // 2)))
    scales_d = dev(torch.from_numpy(scales))
    sg_d = dev(torch.tensor([s_g], dtype=torch.float32))
    for out_dtype, bf in ((torch.float32, False), (torch.bfloat16, True)):
        announce(f"dequantize fmt={fmt} {what} {rows}x{cols} -> {out_dtype}")
        y = fp4.dequantize(fmt, codes_d, scales_d, sg_d if fmt == fp4.NVFP4 else None, out_dtype)
        torch.cuda.synchronize()
        want = oracle.dequantize(fmt, packed, scales, s_g, out_bf16=bf)
        got = y.cpu()
        got = workloads.bf16_bits(got).reshape(-1) if bf else got.numpy().reshape(-1)
        assert_float_bits_equal(got, want, f"{what} -> {out_dtype}")


def test_dequant_roundtrips_of_the_workloads():
    x = workloads.tiny_roundtrip()
    p, s, f = oracle.mx_quantize(oracle_view(x))
    _dq_check(fp4.MXFP4, p, s, 1.0, 1, "tiny MX")
    p, s, sg, f = oracle.nv_quantize(oracle_view(x))
    _dq_check(fp4.NVFP4, p, s, float(sg), 1, "tiny NV")
    w = workloads.nvfp4_weight()
    p, s, sg, f = oracle.nv_quantize(oracle_view(w))
    _dq_check(fp4.NVFP4, p, s, float(sg), 8192, "weight 8192x8192 NV")


def test_dequant_every_code_and_scale_byte():
    # every code in every nibble position against every scale byte
    codes = np.tile(np.arange(256, dtype=np.uint8), 256 * 2)  # 256 scale rows
    # MX: block = 16 packed bytes; 256 * 2 * 256 bytes = 8192 blocks
    nblk_mx = codes.size // 16
    s_mx = (np.arange(nblk_mx) % 253).astype(np.uint8)         # finite products (e <= 125)
    s_mx[::97] = 255                                           # NaN scale
    _dq_check(fp4.MXFP4, codes, s_mx, 1.0, 64, "all codes x E8M0")
    nblk_nv = codes.size // 8
    s_nv = (np.arange(nblk_nv) % 256).astype(np.uint8)         # includes negatives and NaNs
    for sg in (1.0, 0.0123, 3.1e-38, 1e-44, 2.5e30):
        _dq_check(fp4.NVFP4, codes, s_nv, sg, 64, f"all codes x E4M3, s_g={sg}")


def _search_check(x: torch.Tensor, what: str, ncand=64, c_lo=0.5, c_hi=1.0, sample=None):
    announce(f"scale search {what} {tuple(x.shape)} n={ncand} c=[{c_lo},{c_hi}]")
    codes, scales, sg = fp4.scale_search(dev(x), ncand, c_lo, c_hi)
    torch.cuda.synchronize()
    xo = oracle_view(x)
    s_g, f1 = oracle.nv_global_scale(xo)
    assert f1 == 0
    assert f32_bits(sg.cpu().numpy())[0] == f32_bits([s_g])[0]
    gc, gs = host_u8(codes), host_u8(scales)
    if sample is None:
        p, s, f2 = oracle.scale_search_with_scale(xo, s_g, ncand, c_lo, c_hi)
        assert f2 == 0
        assert_bytes_equal(gs, s, f"{what}: scales")
        assert_bytes_equal(gc, p, f"{what}: codes")
    else:
        blocks = np.asarray(sample)
        xb = xo.reshape(-1, 16)[blocks].reshape(-1)
        p, s, f2 = oracle.scale_search_with_scale(xb, s_g, ncand, c_lo, c_hi)
        assert f2 == 0
        assert_bytes_equal(gs[blocks], s, f"{what}: sampled scales")
        assert_bytes_equal(gc.reshape(-1, 8)[blocks].reshape(-1), p, f"{what}: sampled codes")


def test_search_counterexample_and_wide_range():
    x = torch.tensor([2688.0] * 16 + [0.4] * 15 + [3.6] + [3.75] + [0.0] * 15).reshape(1, 48)
    _search_check(x, "page counterexample")
    _search_check(x, "page counterexample wide", c_hi=1.5)
    _search_check(x.to(torch.bfloat16), "page counterexample bf16")


def test_search_small_laplace_full_compare():
    x = workloads.scale_search_input(64, 1024, seed=3)
    _search_check(x, "laplace 64x1024")
    _search_check(x, "laplace 64x1024 n=33 c=[0.75,1.25]", ncand=33, c_lo=0.75, c_hi=1.25)
    g = torch.Generator().manual_seed(9)
    y = torch.randn(32, 512, generator=g) * torch.rand(32, 512, generator=g) ** 3 * 1e-3
    _search_check(y, "heavy-tailed fp32 32x512")
    _search_check((y * 2.0 ** -120).to(torch.float32), "tiny magnitudes 2^-120")


def test_search_full_size_sampled():
    x = workloads.scale_search_input()
    nblocks = x.numel() // 16
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([np.arange(0, 1792),                       # first two rows
                                       rng.integers(0, nblocks, 20000),
                                       np.arange(nblocks - 896, nblocks)]))     # last row
    _search_check(x, "laplace 4096x14336 (sampled blocks)", sample=sample)
