"""GPU parity: dequantization (bit-exact, fp32 and bf16 outputs) and the
MSE-optimal NVFP4 scale search (bit-exact codes and scale bytes)."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import (announce, assert_bytes_equal, assert_float_bits_equal, dev, f32_bits,
                        host_u8, oracle_split, oracle_view)

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
    p, s, f = oracle.mx_quantize(oracle_view(w))
    assert f == 0
    _dq_check(fp4.MXFP4, p, s, 1.0, 8192, "weight 8192x8192 MX")


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


def _search_check(x: torch.Tensor, what: str, ncand=64, c_lo=0.5, c_hi=1.0):
    announce(f"scale search {what} {tuple(x.shape)} n={ncand} c=[{c_lo},{c_hi}]")
    codes, scales, sg = fp4.scale_search(dev(x), ncand, c_lo, c_hi)
    torch.cuda.synchronize()
    xo = oracle_view(x)
    s_g, f1 = oracle.nv_global_scale(xo)
    assert f1 == 0
    assert f32_bits(sg.cpu().numpy())[0] == f32_bits([s_g])[0]
    res = oracle_split(lambda part: oracle.scale_search_with_scale(part, s_g, ncand, c_lo, c_hi),
                       xo, 16)
    assert all(r[2] == 0 for r in res)
    assert_bytes_equal(host_u8(scales), np.concatenate([r[1] for r in res]), f"{what}: scales")
    assert_bytes_equal(host_u8(codes), np.concatenate([r[0] for r in res]), f"{what}: codes")


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
    # bf16 with s_g below the normal range: the generic walk (exact divides)
    _search_check((y * 2.0 ** -120).to(torch.bfloat16), "tiny magnitudes bf16 2^-120")
    # bf16, a ragged last tile (222 chunks): blocks still queued when a
    # wave's tiles run out are drained in partial passes
    _search_check(workloads.scale_search_input(3, 592, seed=4), "laplace bf16 3x592")
    _search_check(workloads.scale_search_input(3, 592, seed=4), "laplace bf16 3x592 wide", c_hi=1.5)


def test_search_scale_underflow_flag_bf16():
    # a block whose amax is far below the tensor amax has no candidate code
    # (every one rounds to code 0): the oracle and the kernel both flag it
    x = torch.tensor([1.0] * 16 + [2.0 ** -24] * 16 + [0.5, -0.25] * 8).reshape(1, 48)
    x = x.to(torch.bfloat16)
    p, s, sg, f = oracle.scale_search(oracle_view(x))
    assert f == fp4.FLAG_SCALE_UNDERFLOW
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    announce("scale search bf16 with a scale underflow")
    codes, scales, s_g = fp4.scale_search(dev(x), check=False, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == f
    # the underflowing block gets code 0 and zero codes, the others their search
    assert_bytes_equal(host_u8(scales), s, "search scales with an underflow")
    assert_bytes_equal(host_u8(codes), p, "search codes with an underflow")


def test_search_ragged_shapes_of_the_one_wave_amax_pass():
    # bf16 inputs of 8 to 64 chunks per lane on all CUs take the tensor-amax
    # pass of one workgroup per CU; 2049 x 4112 (1,053,186 chunks: on 256
    # CUs 129 workgroups of 16 chunks per lane, the last grid row partly past
    # the end) with the largest magnitude planted in the tensor's last chunk,
    # then in its first: s_g, codes and scale bytes every block against the
    # oracle
    x = workloads.scale_search_input(2049, 4112, seed=5)
    y = x.clone()
    y[-1, -3] = 0.75
    _search_check(y, "laplace 2049x4112, amax in the last chunk")
    y = x.clone()
    y[0, 1] = -0.75
    _search_check(y, "laplace 2049x4112, amax in the first chunk")


def test_search_full_size_every_block():
    # the 4096 x 14336 Laplace(0, 0.01) search input, 64 candidates in
    # [0.5, 1]: every one of its 3.67M blocks against the oracle (the oracle
    # split over host threads)
    _search_check(workloads.scale_search_input(), "laplace 4096x14336 (every block)")
