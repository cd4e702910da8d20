"""Pins for the oracle's NVFP4 two-level encoder and NV dequantization."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import _exact
from tests._golden import keyed

G = keyed("nv_scale_examples.txt")


def _f32(vals):
    return np.asarray(vals, np.float32)


def _mse(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.mean((x - y) ** 2))


def test_tensor_scale_fixed_by_a_2688_block():
    s_g, flags = oracle.nv_global_scale(_f32([2688.0] * 16))
    assert flags == 0 and s_g == float(G["tensor_scale_from_2688"][0][0])


def test_pattern_block_scale_codes_bytes_and_reconstruction():
    pattern = [float(v) for v in G["pattern"][0]]
    x = _f32([2688.0] * 16 + pattern * 2)
    packed, scales, s_g, flags = oracle.nv_quantize(x)
    assert flags == 0 and s_g == 1.0
    assert scales[0] == 0x7E                                       # tensor-max block: 448
    assert oracle.e4m3_value(int(scales[1])) == float(G["pattern_e4m3_scale"][0][0])
    codes = oracle.unpack(packed)[16:]
    assert list(codes) == list(range(8)) * 2
    assert packed[8:].tobytes().hex(" ") == "10 32 54 76 10 32 54 76"
    y = oracle.dequantize(oracle.NV, packed, scales, s_g)[16:24]
    assert list(y) == [float(v) for v in G["pattern_recon"][0]]


@pytest.mark.parametrize("row", G["pattern_mse"])
def test_pattern_mse_at_fixed_scales(row):
    scale, want = float(row[0]), float(row[1])
    pattern = _f32([float(v) for v in G["pattern"][0]] * 2)
    mse = oracle.block_loss(pattern, scale) / 16.0
    # the page's values are for decimal inputs; fp32 inputs move them by < 1e-6
    assert mse == pytest.approx(want, rel=1e-6, abs=1e-12)


def test_counterexample_maxbased_and_better_scale():
    v, n, big = G["counter"][0]
    block = _f32([float(v)] * int(n) + [float(big)])
    x = np.concatenate([_f32([2688.0] * 16), block])
    packed, scales, s_g, _ = oracle.nv_quantize(x)
    sc, num, den = G["counter_maxbased"][0]
    assert oracle.e4m3_value(int(scales[1])) == float(sc)
    y = oracle.dequantize(oracle.NV, packed, scales, s_g)[16:]
    assert _mse(block, y) == pytest.approx(int(num) / int(den), rel=1e-6)
    sc2, num2, den2 = G["counter_better"][0]
    assert oracle.e4m3_value(oracle.e4m3_nearest(float(sc2), 1.0)) == float(sc2)
    assert oracle.block_loss(block, float(sc2)) / 16 == pytest.approx(int(num2) / int(den2), rel=1e-6)


def test_zero_tensor_and_zero_block():
    x = np.zeros(32, np.float32)
    x[5] = -0.0
    packed, scales, s_g, flags = oracle.nv_quantize(x)
    assert flags == 0 and s_g == 1.0 and list(scales) == [0x38, 0x38]
    codes = oracle.unpack(packed)
    assert codes[5] == 8 and codes.sum() == 8
    x = _f32([2688.0] * 16 + [0.0] * 16)
    packed, scales, s_g, flags = oracle.nv_quantize(x)
    assert flags == 0 and scales[1] == 0x38
    assert np.all(oracle.dequantize(oracle.NV, packed, scales, s_g)[16:] == 0.0)


def test_contract_violations():
    with pytest.raises(ValueError):
        oracle.nv_quantize_with_scale(_f32([1.0] * 17), 1.0)
    assert oracle.nv_quantize(_f32([np.nan] * 16))[3] & oracle.FLAG_NONFINITE
    # the page's [1e-50]*16 is below fp32 range; an fp32 subnormal tensor
    # makes the tensor scale A/2688 underflow to zero the same way
    assert oracle.nv_quantize(_f32([1e-42] * 16))[3] & oracle.FLAG_SCALE_UNDERFLOW
    # nonzero block whose E4M3 scale rounds to zero
    assert oracle.nv_quantize(_f32([2688.0] * 16 + [1e-10] * 16))[3] & oracle.FLAG_SCALE_UNDERFLOW


def test_tensor_scale_is_correctly_rounded_quotient():
    rng = np.random.default_rng(21)
    for A in list(rng.uniform(1e-30, 1e30, 200)) + [2.0 ** -120, 3e-38, 1e-41]:
        x = _f32([A] + [0.0] * 15)
        s_g, _ = oracle.nv_global_scale(x)
        assert s_g == _exact.rn32(Fraction(float(x[0])) / 2688), A


def test_max_block_scale_code_is_448():
    t = torch.randn(32, 256, generator=torch.Generator().manual_seed(8)).numpy()
    packed, scales, s_g, flags = oracle.nv_quantize(t)
    amax = np.abs(t).reshape(-1, 16).max(axis=1)
    assert flags == 0
    assert np.all(scales[amax == amax.max()] == 0x7E)


def test_matches_exact_definition_on_random_and_adversarial_blocks():
    rng = np.random.default_rng(13)
    blocks = [rng.normal(0, 1, 16) * 10.0 ** rng.integers(-3, 3) for _ in range(60)]
    blocks.append([0.3, 0.6, 0.9, 1.2, 1.8, 2.4, 3.6, -0.0, 1e-30, -1e-30] + [0.0] * 6)
    blocks.append([4.1] * 16)
    x = np.concatenate([np.asarray(b, np.float32) for b in blocks])
    s_g_want = _exact.nv_tensor_scale(x)
    packed, scales, s_g, flags = oracle.nv_quantize(x)
    assert flags == 0 and s_g == s_g_want
    codes = oracle.unpack(packed)
    for i, b in enumerate(blocks):
        sc, cb = _exact.nv_block(np.asarray(b, np.float32), s_g)
        assert scales[i] == sc, i
        assert list(codes[16 * i: 16 * i + 16]) == cb, i


def test_subnormal_tensor_scale_still_exact():
    # tensor amax ~1e-40: s_g is an fp32 subnormal with few significant bits
    rng = np.random.default_rng(17)
    x = (rng.uniform(-1, 1, 64) * 1e-36).astype(np.float32)
    x[0] = np.float32(3e-36)
    packed, scales, s_g, flags = oracle.nv_quantize(x)
    assert s_g < np.finfo(np.float32).tiny
    if flags:
        return
    codes = oracle.unpack(packed)
    for i in range(4):
        sc, cb = _exact.nv_block(x[16 * i: 16 * i + 16], s_g)
        assert scales[i] == sc and list(codes[16 * i:16 * i + 16]) == cb


def test_dequant_values():
    rng = np.random.default_rng(19)
    p = rng.integers(0, 256, 32, dtype=np.uint8)
    s = rng.integers(1, 127, 4, dtype=np.uint8)
    s_g = np.float32(0.0123)
    y = oracle.dequantize(oracle.NV, p, s, s_g)
    codes = oracle.unpack(p)
    for i in range(64):
        alpha = _exact.rn32(Fraction(float(s_g)) * _exact.E4M3_POS[int(s[i // 16])])
        want = _exact.rn32(Fraction(float(oracle.e2m1_value(int(codes[i])))) * Fraction(float(alpha)))
        assert y[i] == want
    yb = oracle.dequantize(oracle.NV, p, s, s_g, out_bf16=True)
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, tb)
    assert np.isnan(oracle.dequantize(oracle.NV, p[:8], np.array([0x7F], np.uint8), s_g)).all()


def test_bf16_rounding_matches_torch_on_many_patterns():
    rng = np.random.default_rng(23)
    bits = rng.integers(0, 0x7F800000, 200000, dtype=np.uint32)
    bits = np.concatenate([bits, (bits & 0xFFFF0000) | 0x8000, bits | 0x80000000])
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    idx = np.concatenate([np.arange(0, 2000), np.arange(200000, 202000), np.arange(400000, 402000)])
    got = np.array([oracle.f32_to_bf16_bits(v) for v in f[idx]], np.uint16)
    assert np.array_equal(got, want[idx])
