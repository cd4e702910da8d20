"""Pins for the oracle's MXFP4 encoder (OCP floor rule) and MX dequantization."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from tests import _exact
from tests._golden import keyed


def _block_with(values, fill=0.0):
    b = np.full(32, fill, np.float32)
    b[: len(values)] = values
    return b


def test_amax_7_gives_scale_1_and_saturates_to_6():
    amax, scale, recon = map(float, keyed("mx_examples.txt")["floor_rule"][0])
    packed, scales, flags = oracle.mx_quantize(_block_with([amax]))
    assert flags == 0
    assert 2.0 ** (int(scales[0]) - 127) == scale
    y = oracle.dequantize(oracle.MX, packed, scales)
    assert y[0] == recon


def test_transpose_counterexample():
    base, big, want_qt, want_tq = map(float, keyed("mx_examples.txt")["transpose"][0])
    w = np.full((32, 32), base, np.float32)
    w[0, 0] = big
    p, s, _ = oracle.mx_quantize(w)
    q_then_t = oracle.dequantize(oracle.MX, p, s).reshape(32, 32).T
    p2, s2, _ = oracle.mx_quantize(np.ascontiguousarray(w.T))
    t_then_q = oracle.dequantize(oracle.MX, p2, s2).reshape(32, 32)
    assert q_then_t[0, 1] == want_qt
    assert t_then_q[0, 1] == want_tq


def test_codebook_at_scale_0_125():
    row = keyed("mx_examples.txt")["codebook"][0]
    s = float(row[0])
    vals = [float(v) for v in row[1:]]
    assert [oracle.e2m1_value(c) * s for c in range(8)] == vals


def test_exponent_is_exact_floor_log2_minus_2():
    rng = np.random.default_rng(5)
    amaxes = list(rng.uniform(1e-3, 1e3, 200).astype(np.float32))
    amaxes += [np.float32(2.0 ** k) for k in range(-149, 128)]
    amaxes += [np.nextafter(np.float32(2.0 ** k), np.float32(0)) for k in range(-140, 128)]
    for a in amaxes:
        want = max(_exact.floor_log2(Fraction(float(a))) - 2, -127)
        assert oracle.mx_exponent(float(a)) == want, a


def test_zero_block_and_signed_zero():
    x = np.zeros(32, np.float32)
    x[3] = -0.0
    p, s, flags = oracle.mx_quantize(x)
    assert flags == 0 and s[0] == 127
    codes = oracle.unpack(p)
    assert codes[3] == 8 and codes.sum() == 8


def test_tiny_block_clamps_at_minus_127():
    x = np.full(32, 2.0 ** -140, np.float32)
    p, s, flags = oracle.mx_quantize(x)
    assert s[0] == 0   # 2^-127
    # 2^-140 / 2^-127 = 2^-13 rounds to zero
    assert np.all(oracle.unpack(p) == 0)


def test_matches_exact_definition_on_random_and_adversarial_blocks():
    rng = np.random.default_rng(9)
    blocks = [rng.normal(0, 1, 32) * 10.0 ** rng.integers(-30, 30) for _ in range(40)]
    # ties at every midpoint for a block scale of 1 (amax 4 -> e = 0)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0, -0.25, -0.75, -5.0, 7.0, -7.9]
    blocks.append(_block_with(mids + [4.0]))
    blocks.append(_block_with([2.0 ** -130, -2.0 ** -133, 2.0 ** -127, 1e-40]))
    x = np.concatenate([np.asarray(b, np.float32) for b in blocks])
    p, s, flags = oracle.mx_quantize(x)
    assert flags == 0
    codes = oracle.unpack(p)
    for i, b in enumerate(blocks):
        sb, cb = _exact.mx_block(np.asarray(b, np.float32))
        assert s[i] == sb
        assert list(codes[32 * i: 32 * i + 32]) == cb


def test_block_max_maps_to_top_codes_and_roundtrip_is_idempotent():
    x = torch.randn(64, 256, generator=torch.Generator().manual_seed(2)).numpy()
    p, s, _ = oracle.mx_quantize(x)
    codes = oracle.unpack(p).reshape(-1, 32)
    assert np.all((codes & 7).max(axis=1) >= 6)
    y = oracle.dequantize(oracle.MX, p, s)
    p2, s2, _ = oracle.mx_quantize(y)
    assert np.array_equal(p, p2) and np.array_equal(s, s2)


def test_nonfinite_flagged():
    x = np.zeros(64, np.float32)
    x[40] = np.inf
    assert oracle.mx_quantize(x)[2] & oracle.FLAG_NONFINITE


def test_bf16_input_equals_widened_fp32_input():
    t = torch.randn(8, 64, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    from workloads import bf16_bits
    a = oracle.mx_quantize(bf16_bits(t))
    b = oracle.mx_quantize(t.float().numpy())
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_dequant_is_exact_and_bf16_matches_torch_rounding():
    rng = np.random.default_rng(10)
    p = rng.integers(0, 256, 64, dtype=np.uint8)
    s = rng.integers(0, 253, 4, dtype=np.uint8)   # e <= 125: every product is finite
    y = oracle.dequantize(oracle.MX, p, s)
    codes = oracle.unpack(p)
    for i in range(128):
        want = Fraction(float(oracle.e2m1_value(int(codes[i])))) * Fraction(2) ** (int(s[i // 32]) - 127)
        assert Fraction(float(y[i])) == want
    yb = oracle.dequantize(oracle.MX, p, s, out_bf16=True)
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, tb)
    assert np.isnan(oracle.dequantize(oracle.MX, p[:16], np.array([255], np.uint8))).all()
