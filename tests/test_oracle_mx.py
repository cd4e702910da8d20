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


# ---- encoder variants ("NVFP4 / MXFP4 format" page, section 5) ---------------

def test_ceil_rule_amax_7_gives_scale_2():
    amax, scale, reach = map(float, keyed("mx_examples.txt")["ceil_rule"][0])
    packed, scales, flags = oracle.mx_quantize_rule(_block_with([amax]), "ceil")
    assert flags == 0
    assert 2.0 ** (int(scales[0]) - 127) == scale
    assert 6 * scale == reach
    # 7 / 2 = 3.5 is the midpoint of 3 and 4: the even code (4) reconstructs 8
    y = oracle.dequantize(oracle.MX, packed, scales)
    assert y[0] == 8.0


def _ceil_exponent_exact(amax: float) -> int:
    """Smallest e with 6 * 2^e >= amax, by exact rationals, clamped at -127."""
    a = Fraction(amax)
    e = 0
    while Fraction(6) * Fraction(2) ** e < a:
        e += 1
    while Fraction(6) * Fraction(2) ** (e - 1) >= a:
        e -= 1
    return max(e, -127)


def test_ceil_rule_exponent_is_the_smallest_power_covering_amax_over_6():
    rng = np.random.default_rng(21)
    cases = [6.0, 6.0 * (1 + 2 ** -23), 1.5, 1.5 * (1 + 2 ** -23), 3.0, 12.0, 4.0, 2.0 ** -126,
             1e-45, 3e38, 0.75 * 2.0 ** -120]
    cases += list((rng.uniform(1, 2, 300) * 2.0 ** rng.integers(-140, 120, 300)).astype(np.float32))
    for a in cases:
        a = float(np.float32(a))
        assert oracle.mx_exponent_ceil(a) == _ceil_exponent_exact(a), a


def test_ceil_rule_never_saturates_and_lands_the_max_in_3_to_6():
    g = torch.Generator().manual_seed(22)
    x = (torch.randn(64, 32, generator=g) * 2.0 ** torch.randint(-20, 20, (64, 1), generator=g))
    x = x.numpy().astype(np.float32)
    packed, scales, flags = oracle.mx_quantize_rule(x.reshape(-1), "ceil")
    assert flags == 0
    codes = oracle.unpack(packed).reshape(64, 32)
    for b in range(64):
        e = int(scales[b]) - 127
        q = x[b].astype(np.float64) / 2.0 ** e
        assert np.abs(q).max() <= 6.0 and np.abs(q).max() > 3.0
        # the block maximum's magnitude code is 5, 6 or 7 (3, 4 or 6)
        i = int(np.argmax(np.abs(x[b])))
        assert (codes[b, i] & 7) in (5, 6, 7)
    # and it never picks a smaller exponent than the floor rule
    _, s_floor, _ = oracle.mx_quantize(x.reshape(-1))
    assert np.all(scales.astype(int) >= s_floor.astype(int))
    assert np.all(scales.astype(int) - s_floor.astype(int) <= 1)


def _exact_sse32(block, e) -> Fraction:
    """Exact sum of squared errors of a 32-block at scale 2^e."""
    tot = Fraction(0)
    s = Fraction(2) ** e
    for v in block:
        c = _exact.e2m1_code_of_f32(_exact.rn32(Fraction(float(v)) / s))
        tot += (Fraction(float(v)) - Fraction(float(oracle.e2m1_value(c))) * s) ** 2
    return tot


def test_mse_rule_hand_worked_blocks():
    # [7.5, 0 x 31]: OCP e = 0 saturates 7.5 to 6 (loss 2.25); e = 1 sends
    # 3.75 to 4, i.e. 8 (loss 0.25); e = -1 saturates at 3 (loss 20.25)
    b = _block_with([7.5])
    _, s, f = oracle.mx_quantize_rule(b, "mse")
    assert f == 0 and int(s[0]) - 127 == 1
    assert [float(_exact_sse32(b, e)) for e in (-1, 0, 1)] == [20.25, 2.25, 0.25]
    # [4, 0.2 x 31]: at e = 0 every 0.2 rounds to 0 (loss 31 * 0.04); at
    # e = -1 they become 0.25 each (0.4 -> 0.5) and 4 saturates to 3
    b = _block_with([4.0], fill=0.2)
    _, s, _ = oracle.mx_quantize_rule(b, "mse")
    assert int(s[0]) - 127 == -1
    l = [_exact_sse32(b, e) for e in (-1, 0, 1)]
    assert l[0] < l[1] and l[0] < l[2]
    # [7, 0 x 31]: e = 0 (7 -> 6) and e = 1 (3.5 -> 4, i.e. 8) both lose 1:
    # the OCP exponent stays
    b = _block_with([7.0])
    _, s, _ = oracle.mx_quantize_rule(b, "mse")
    assert int(s[0]) - 127 == 0
    assert _exact_sse32(b, 0) == _exact_sse32(b, 1) == 1


def test_mse_rule_loss_is_the_fp32_pairwise_sum_within_its_error_bound():
    g = torch.Generator().manual_seed(23)
    x = (torch.randn(20, 32, generator=g) * 3).numpy().astype(np.float32)
    for b in x:
        for e in (-1, 0, 1, 2):
            exact = _exact_sse32(b, e)
            got = Fraction(oracle.mx_block_loss32(b, e))
            # 32 squared terms and 31 additions, each one rounding of 2^-24
            assert abs(got - exact) <= exact * Fraction(70, 2 ** 24) + Fraction(1, 2 ** 140)


def test_mse_rule_never_worse_than_ocp_and_stays_within_one_exponent():
    g = torch.Generator().manual_seed(24)
    x = torch.randn(256, 32, generator=g) * torch.rand(256, 32, generator=g) ** 3
    x = x.numpy().astype(np.float32)
    _, s_mse, f = oracle.mx_quantize_rule(x.reshape(-1), "mse")
    _, s_ocp, _ = oracle.mx_quantize(x.reshape(-1))
    assert f == 0
    d = s_mse.astype(int) - s_ocp.astype(int)
    assert set(np.unique(d)) <= {-1, 0, 1} and (d != 0).any()
    for b in range(256):
        e0, e = int(s_ocp[b]) - 127, int(s_mse[b]) - 127
        L = {k: oracle.mx_block_loss32(x[b], k) for k in (e0 - 1, e0, e0 + 1)}
        assert L[e] == min(L.values())
        assert e == e0 or L[e] < L[e0]
    # the rule "ocp" reproduces the floor-rule encoder exactly
    p1, s1, _ = oracle.mx_quantize_rule(x.reshape(-1), "ocp")
    p2, s2, _ = oracle.mx_quantize(x.reshape(-1))
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
