"""Seeded randomized parity sweep: every quantizer entry point bit-exact
against the oracle on 30 generated tensors.  Shapes vary over 1..199 rows
and 32..3040 columns, in both dtypes.  The values are normal, heavy-tailed,
sparse with exact zeros, fp32-subnormal, or with a different power-of-two
scale per row (2^-6 .. 2^6, or 2^-60 .. 2^60 so that NVFP4 blocks
underflow).  The
dequantizers run on the results.  Status flags must equal the oracle's;
bytes are compared whenever no flag is set (outputs are unspecified
otherwise)."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import oracle.gemm as og
import workloads
from tests._gpu import (announce, assert_bytes_equal, assert_float_bits_equal, dev, f32_bits,
                        host_u8, oracle_view)

pytestmark = pytest.mark.gpu

KINDS = ["normal", "heavy-tailed", "sparse", "subnormal", "row scales"]


def _case(i):
    rng = np.random.default_rng(1000 + i)
    rows = int(rng.integers(1, 200))
    cols = 32 * int(rng.integers(1, 96))
    kind = KINDS[i % len(KINDS)]
    g = torch.Generator().manual_seed(2000 + i)
    x = torch.randn(rows, cols, generator=g)
    if kind == "heavy-tailed":
        x = x / torch.sqrt(torch.rand(rows, cols, generator=g) + 1e-3)
    elif kind == "sparse":
        x = x * (torch.rand(rows, cols, generator=g) < 0.2)
    elif kind == "subnormal":
        x = x * 1e-39
    elif kind == "row scales":
        span = 60 if i % 10 == 4 else 6   # the wide span makes some NVFP4 blocks underflow
        x = x * torch.exp2(torch.randint(-span, span + 1, (rows, 1), generator=g).float())
    e = int(rng.integers(-20, 21)) if kind != "subnormal" else 0
    x = (x * 2.0 ** e).float()
    dt = torch.bfloat16 if i % 2 else torch.float32
    return x.to(dt), f"case {i}: {rows}x{cols} {kind} x 2^{e} {dt}"


def _status():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _dequant_check(fmt, p, s, sg, rows, what):
    cols = p.size * 2 // rows
    for out_dtype, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = fp4.dequantize(fmt, dev(torch.from_numpy(p.reshape(rows, cols // 2))),
                           dev(torch.from_numpy(s.reshape(rows, -1))),
                           dev(torch.tensor([sg], dtype=torch.float32)) if fmt == fp4.NVFP4 else None,
                           out_dtype)
        want = oracle.dequantize(fmt, p, s, sg, out_bf16=bf)
        got = workloads.bf16_bits(y.cpu()).reshape(-1) if bf else y.cpu().numpy().reshape(-1)
        assert_float_bits_equal(got, want, f"{what}: dequantize -> {out_dtype}")


@pytest.mark.parametrize("i", range(30))
def test_sweep(i):
    x, what = _case(i)
    rows, cols = x.shape
    xd, xo = dev(x), oracle_view(x)

    announce(f"{what}: mxfp4 quantize, rules, dequantize")
    p, s, f = oracle.mx_quantize(xo)
    assert f == 0
    codes, scales = fp4.quantize_mxfp4(xd)
    assert_bytes_equal(host_u8(scales), s, f"{what}: MX scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: MX codes")
    _dequant_check(fp4.MXFP4, p, s, 1.0, rows, f"{what} MX")
    for rule in ("ceil", "mse"):
        pr, sr, _ = oracle.mx_quantize_rule(xo, rule)
        cr, scr = fp4.quantize_mxfp4_rule(xd, rule)
        assert_bytes_equal(host_u8(scr), sr, f"{what}: MX {rule} scales")
        assert_bytes_equal(host_u8(cr), pr, f"{what}: MX {rule} codes")
    if cols % 512 == 0:
        got = fp4.quantize_mxfp4_packed(xd)
        assert_bytes_equal(host_u8(got), og.pack_operand(p, s, rows, cols), f"{what}: MX packed")

    announce(f"{what}: nvfp4 quantize, dequantize, scale search")
    p, s, sg, f = oracle.nv_quantize(xo)
    st = _status()
    codes, scales, s_g = fp4.quantize_nvfp4(xd, check=False, status=st)
    assert int(st.item()) == f, f"{what}: NV flags {int(st.item())} vs oracle {f}"
    if f == 0:
        assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: s_g"
        assert_bytes_equal(host_u8(scales), s, f"{what}: NV scales")
        assert_bytes_equal(host_u8(codes), p, f"{what}: NV codes")
        _dequant_check(fp4.NVFP4, p, s, float(sg), rows, f"{what} NV")
    if cols % 512 == 0:
        st = _status()
        got, s_g = fp4.quantize_nvfp4_packed(xd, check=False, status=st)
        assert int(st.item()) == f, f"{what}: NV packed flags {int(st.item())} vs oracle {f}"
        if f == 0:
            assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: packed s_g"
            assert_bytes_equal(host_u8(got), og.nv_pack_operand(p, s, rows, cols), f"{what}: NV packed")
    p, s, sg, f = oracle.scale_search(xo)
    st = _status()
    codes, scales, s_g = fp4.scale_search(xd, check=False, status=st)
    assert int(st.item()) == f, f"{what}: search flags {int(st.item())} vs oracle {f}"
    if f == 0:
        assert_bytes_equal(host_u8(scales), s, f"{what}: search scales")
        assert_bytes_equal(host_u8(codes), p, f"{what}: search codes")

    announce(f"{what}: stochastic rounding")
    seed = 0x9E3779B97F4A7C15 * (i + 1) % 2**64
    p, s, f = oracle.mx_quantize_sr(xo, seed)
    codes, scales = fp4.quantize_sr(fp4.MXFP4, xd, seed)
    assert_bytes_equal(host_u8(scales), s, f"{what}: MX SR scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: MX SR codes")
    p, s, sg, f = oracle.nv_quantize_sr(xo, seed)
    st = _status()
    codes, scales, s_g = fp4.quantize_sr(fp4.NVFP4, xd, seed, check=False, status=st)
    assert int(st.item()) == f, f"{what}: NV SR flags {int(st.item())} vs oracle {f}"
    if f == 0:
        assert_bytes_equal(host_u8(scales), s, f"{what}: NV SR scales")
        assert_bytes_equal(host_u8(codes), p, f"{what}: NV SR codes")


@pytest.mark.parametrize("i", range(12))
def test_sweep_padded(i):
    """The row-padded layout on generated shapes whose rows are not whole
    blocks (any column count), both formats, with the cropping decode."""
    rng = np.random.default_rng(3000 + i)
    rows, cols = int(rng.integers(1, 120)), int(rng.integers(1, 3000))
    g = torch.Generator().manual_seed(4000 + i)
    x = torch.randn(rows, cols, generator=g) / torch.sqrt(torch.rand(rows, cols, generator=g) + 1e-3)
    x = x.to(torch.bfloat16 if i % 2 else torch.float32)
    what = f"padded case {i}: {rows}x{cols} {x.dtype}"
    xo = oracle_view(x)
    for fmt in (fp4.MXFP4, fp4.NVFP4):
        announce(f"{what} fmt={fmt}")
        codes, scales, s_g = fp4.quantize_padded(fmt, dev(x))
        if fmt == fp4.MXFP4:
            p, s, f = oracle.mx_quantize_padded(xo, rows, cols)
            sg = 1.0
        else:
            p, s, sg, f = oracle.nv_quantize_padded(xo, rows, cols)
            assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: s_g"
        assert f == 0
        assert_bytes_equal(host_u8(scales), s, f"{what}: padded scales fmt={fmt}")
        assert_bytes_equal(host_u8(codes), p, f"{what}: padded codes fmt={fmt}")
        for out_dtype, bf in ((torch.float32, False), (torch.bfloat16, True)):
            y = fp4.dequantize_padded(fmt, codes, scales, cols,
                                      s_g if fmt == fp4.NVFP4 else None, out_dtype)
            want = oracle.dequantize_padded(fmt, p, s, rows, cols, sg, out_bf16=bf)
            got = workloads.bf16_bits(y.cpu()).reshape(-1) if bf else y.cpu().numpy().reshape(-1)
            assert_float_bits_equal(got, want, f"{what}: padded decode fmt={fmt} -> {out_dtype}")


@pytest.mark.parametrize("i", range(10))
def test_sweep_packed_layouts(i):
    """The generated tensors, their rows repeated out to a multiple of 512
    columns, through both quantizers that write the packed layouts."""
    x, what = _case(i)
    rows, cols = x.shape
    k = max(1, cols // 512)
    x = x.repeat(1, -(-512 * k // cols))[:, :512 * k].contiguous()
    cols = x.shape[1]
    what = f"{what}, repeated to {rows}x{cols}"
    xd, xo = dev(x), oracle_view(x)
    announce(f"{what}: quantize into the packed layouts")
    p, s, f = oracle.mx_quantize(xo)
    assert f == 0
    got = fp4.quantize_mxfp4_packed(xd)
    assert_bytes_equal(host_u8(got), og.pack_operand(p, s, rows, cols), f"{what}: MX packed")
    p, s, sg, f = oracle.nv_quantize(xo)
    st = _status()
    got, s_g = fp4.quantize_nvfp4_packed(xd, check=False, status=st)
    assert int(st.item()) == f, f"{what}: NV packed flags {int(st.item())} vs oracle {f}"
    if f == 0:
        assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: packed s_g"
        assert_bytes_equal(host_u8(got), og.nv_pack_operand(p, s, rows, cols), f"{what}: NV packed")
