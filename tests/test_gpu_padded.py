"""GPU parity for the row-padded layout ("NVFP4 / MXFP4 format" page, section
8): quantize of rows zero-padded to whole blocks, and the cropping decode,
bit-exact against the oracle, on ragged shapes (down to a single value) in
fp32 and bf16."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
from tests._gpu import (announce, assert_bytes_equal, assert_float_bits_equal, dev, f32_bits,
                        host_u8, oracle_view)
import workloads

pytestmark = pytest.mark.gpu

SHAPES = [(2, 17), (1, 1), (3, 31), (5, 33), (7, 100), (129, 4097), (64, 7173)]


def _input(rows, cols, seed, dtype, heavy=True):
    # heavy tails for MXFP4; for NVFP4 plain Gaussian values, since a tail
    # block of a few tiny values would underflow its E4M3 scale (an error by
    # the format's contract, tested on its own below)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * 4
    if heavy:
        x = x * torch.rand(rows, cols, generator=g) ** 3
    if rows > 2:
        x[1] = 0.0                       # a zero row
        x[2, ::3] = -0.0
    return x.to(dtype)


def _check(fmt, x, what):
    rows, cols = x.shape
    announce(f"quantize padded fmt={fmt} {what} {rows}x{cols} {x.dtype}")
    codes, scales, s_g = fp4.quantize_padded(fmt, dev(x))
    torch.cuda.synchronize()
    xo = oracle_view(x)
    if fmt == fp4.MXFP4:
        p, s, f = oracle.mx_quantize_padded(xo, rows, cols)
        sg = 1.0
    else:
        p, s, sg, f = oracle.nv_quantize_padded(xo, rows, cols)
        assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0]
    assert f == 0
    assert_bytes_equal(host_u8(scales), s, f"{what}: padded scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: padded codes")
    # the cropping decode, from the oracle's bytes
    for out_dtype, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = fp4.dequantize_padded(fmt, dev(torch.from_numpy(p.reshape(rows, -1))),
                                  dev(torch.from_numpy(s.reshape(rows, -1))), cols,
                                  dev(torch.tensor([float(sg)], dtype=torch.float32))
                                  if fmt == fp4.NVFP4 else None, out_dtype)
        torch.cuda.synchronize()
        want = oracle.dequantize_padded(fmt, p, s, rows, cols, sg, out_bf16=bf)
        got = workloads.bf16_bits(y.cpu()).reshape(-1) if bf else y.cpu().numpy().reshape(-1)
        assert_float_bits_equal(got, want, f"{what}: padded decode -> {out_dtype}")


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
def test_padded_roundtrip_matches_oracle(fmt, rows, cols):
    for dtype in (torch.float32, torch.bfloat16):
        _check(fmt, _input(rows, cols, rows * 1000 + cols, dtype, heavy=fmt == 0), "random")


def test_padded_equals_block_aligned_entry_points_on_complete_rows():
    x = _input(48, 1024, 5, torch.bfloat16, heavy=False)
    c1, s1, _ = fp4.quantize_padded(fp4.MXFP4, dev(x))
    c2, s2 = fp4.quantize_mxfp4(dev(x))
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    c1, s1, g1 = fp4.quantize_padded(fp4.NVFP4, dev(x))
    c2, s2, g2 = fp4.quantize_nvfp4(dev(x))
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(g1, g2)


def test_padded_page_example_bytes():
    x = (torch.arange(34, dtype=torch.float32) / 7 - 2).reshape(2, 17)
    codes, scales, s_g = fp4.quantize_padded(fp4.NVFP4, dev(x))
    assert codes.numel() + scales.numel() + 4 == 40 == fp4.padded_storage_bytes(fp4.NVFP4, 2, 17)
    _check(fp4.NVFP4, x, "page 2x17")


def test_padded_underflow_flag_matches_oracle():
    # a row whose padded last block holds one value far below the tensor
    # amax: its block scale rounds to code 0 in the oracle and on the GPU
    x = torch.ones(3, 17)
    x[1, 16] = 1e-7
    p, s, sg, f = oracle.nv_quantize_padded(x.numpy(), 3, 17)
    assert f & 2
    with pytest.raises(ValueError):
        fp4.quantize_padded(fp4.NVFP4, dev(x))
    x[1, 16] = 1e-3
    _check(fp4.NVFP4, x, "tail block above the underflow")


def test_padded_flags_nonfinite():
    x = torch.ones(3, 20)
    x[2, 19] = float("nan")
    for fmt in (fp4.MXFP4, fp4.NVFP4):
        with pytest.raises(ValueError):
            fp4.quantize_padded(fmt, dev(x))
