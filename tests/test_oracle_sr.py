"""Pins of the oracle's stochastic rounding (Ultralytics glossary "FP4",
section "Inferenza e addestramento FP4": NVFP4 pretraining rounds gradients
stochastically; the pages name the technique and give no rule).

The reading pinned here: q (the deterministic encoder's fp32 quotient) rounds
to one of its two neighbouring E2M1 magnitudes lo <= |q| < hi, up with
probability (|q| - lo) / (hi - lo) at 24-bit resolution; |q| >= 6 saturates;
grid values never move; the sign bit is kept.  The 24 random bits of element
i come from SplitMix64 on a counter, pinned to the generator's published
known-answer outputs.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import E2M1_MAG
from tests._golden import rows
from tests._sr_cases import (SEED_ZERO_BITS_AT_16, mean_within_bounds, neighbour_values, neighbours,
                             threshold_blocks, tiny_quotient_cases, tiny_quotient_tensor)

M64 = 2**64 - 1
TWO24 = 2**24


def _golden_outputs():
    out = {}
    for state, k, v in rows("splitmix64.txt"):
        out[(int(state), int(k))] = int(v)
    return out


def test_generator_matches_published_known_answers():
    """Element 2k and 2k+1 of seed s draw from the (k+1)-th output of
    SplitMix64 started at state s: low half then high half, top 24 bits."""
    gold = _golden_outputs()
    assert gold, "fixture empty"
    for (state, k), v in gold.items():
        lo32, hi32 = v & 0xFFFFFFFF, v >> 32
        assert oracle.sr_bits(state, 2 * (k - 1)) == lo32 >> 8, (state, k)
        assert oracle.sr_bits(state, 2 * (k - 1) + 1) == hi32 >> 8, (state, k)


def test_generator_bits_are_24_bit_and_roughly_uniform():
    r = np.array([oracle.sr_bits(7, i) for i in range(20000)], dtype=np.int64)
    assert r.min() >= 0 and r.max() < TWO24
    # mean of U[0, 2^24) over 20000 draws: sd of the mean ~ 2^24 / sqrt(12 * 20000)
    sd = TWO24 / math.sqrt(12 * r.size)
    assert abs(r.mean() - (TWO24 - 1) / 2) < 5 * sd
    # the top bit is a fair coin, the low bit too
    for bit in (23, 0):
        ones = int(((r >> bit) & 1).sum())
        assert abs(ones - r.size / 2) < 5 * math.sqrt(r.size / 4)
    # neighbouring elements are not equal
    assert np.mean(r[1:] == r[:-1]) < 1e-3


def _f32(v) -> float:
    return float(np.float32(v))


def _threshold(q: float) -> int:
    """Number of r in [0, 2^24) that round |q| up, found by bisection on the
    oracle (the decision is monotone in r)."""
    lo_code = oracle.e2m1_round_sr(q, TWO24 - 1)
    if oracle.e2m1_round_sr(q, 0) == lo_code:
        return 0
    a, b = 0, TWO24 - 1  # rounds up at a, down at b
    while b - a > 1:
        mid = (a + b) // 2
        if oracle.e2m1_round_sr(q, mid) == lo_code:
            b = mid
        else:
            a = mid
    return b


def _sample_quotients(seed=0):
    rng = np.random.default_rng(seed)
    qs = []
    for k in range(7):  # random points in every grid interval
        lo, hi = float(E2M1_MAG[k]), float(E2M1_MAG[k + 1])
        qs += [_f32(v) for v in rng.uniform(lo, hi, 40)]
        gap = hi - lo
        # points a few 2^-24 steps of the gap past lo and short of hi
        qs += [_f32(lo + gap * j / TWO24) for j in (1, 2, 3, 5)]
        qs += [_f32(np.nextafter(np.float32(hi), np.float32(0)))]
        qs += [_f32(lo + gap / 2), _f32(lo + gap / 4), _f32(lo + 3 * gap / 4)]
    # tiny and subnormal quotients: only r = 0 rounds them up
    qs += [2.0**-25, 2.0**-26, 2.0**-100, 2.0**-126, 2.0**-149, 3 * 2.0**-149, 1e-30]
    return [q for q in qs if 0.0 < q < 6.0]


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_round_up_probability_is_the_distance_ratio(sign):
    """P(up) = (|q| - lo) / (hi - lo): exactly ceil(2^24 (|q| - lo) / gap) of
    the 2^24 draws round up (the draws r with r gap 2^-24 < |q| - lo), the
    others down, and the two results are the neighbours' codes."""
    for m in _sample_quotients():
        q = sign * m
        fm = Fraction(m)
        lo, hi, k = neighbours(fm)
        d = fm - lo
        expect = 0 if d == 0 else math.ceil(d / (hi - lo) * TWO24)
        assert _threshold(q) == expect, q
        s = 8 if sign < 0 else 0
        if expect > 0:
            assert oracle.e2m1_round_sr(q, 0) == s | (k + 1), q
            assert oracle.e2m1_round_sr(q, expect - 1) == s | (k + 1), q
        if expect < TWO24:
            assert oracle.e2m1_round_sr(q, expect) == s | k, q
            assert oracle.e2m1_round_sr(q, TWO24 - 1) == s | k, q


def test_rounding_is_unbiased_at_24_bit_resolution():
    """For |q| a multiple of gap 2^-24 the mean over all 2^24 draws is q
    exactly; for any q it is within gap 2^-24 above it."""
    for m in _sample_quotients(1):
        fm = Fraction(m)
        lo, hi, _ = neighbours(fm)
        gap = hi - lo
        up = _threshold(m)
        mean = lo + gap * Fraction(up, TWO24)
        assert fm <= mean < fm + gap / TWO24, m
        if (fm - lo) / gap * TWO24 == int((fm - lo) / gap * TWO24):
            assert mean == fm, m


def test_grid_values_never_move_and_large_values_saturate():
    rs = [0, 1, 12345, TWO24 // 2, TWO24 - 1]
    for k, v in enumerate(E2M1_MAG):
        for s in (0, 8):
            q = -float(v) if s else float(v)
            if k == 0 and s:
                q = -0.0
            for r in rs:
                assert oracle.e2m1_round_sr(q, r) == s | k, (q, r)
    for m in (6.0, _f32(6.0000005), 7.5, 1e30, float(np.finfo(np.float32).max), math.inf):
        for r in rs:
            assert oracle.e2m1_round_sr(m, r) == 7
            assert oracle.e2m1_round_sr(-m, r) == 15


def test_result_is_a_neighbour_of_the_nearest_even_result():
    """The stochastic code is the floor or the ceiling neighbour, and the
    deterministic nearest-even code is one of the two."""
    rng = np.random.default_rng(3)
    for q in rng.uniform(-7, 7, 400).astype(np.float32):
        c = oracle.e2m1_round_sr(float(q), int(rng.integers(TWO24)))
        d = oracle.e2m1_round(float(q))
        m = Fraction(abs(float(q)))
        if m >= 6:
            assert c == d
            continue
        lo, hi, k = neighbours(m)
        assert c & 7 in (k, k + 1) and d & 7 in (k, k + 1)
        assert c & 8 == d & 8 == (8 if q < 0 else 0)


def _neighbour_values(x: np.ndarray, scale: np.ndarray):
    """The two E2M1 neighbours of RN32(x / scale), times scale."""
    q = (x.astype(np.float32) / scale.astype(np.float32)).astype(np.float32)
    return neighbour_values(q, scale)


def _mx_scale_values(scales: np.ndarray) -> np.ndarray:
    return np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32)


def test_mx_tensor_keeps_the_deterministic_scales_and_picks_a_neighbour():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(32 * 64) * 3).astype(np.float32)
    x[::97] *= 40
    p_det, s_det, f_det = oracle.mx_quantize(x)
    p, s, f = oracle.mx_quantize_sr(x, seed=11)
    assert f == f_det == 0
    assert np.array_equal(s, s_det)
    y = oracle.dequantize(oracle.MX, p, s).astype(np.float64)
    lo, hi = _neighbour_values(x, _mx_scale_values(s))
    assert np.all((y == lo) | (y == hi))
    # deterministic in the seed, and another seed changes some codes
    assert np.array_equal(p, oracle.mx_quantize_sr(x, seed=11)[0])
    assert not np.array_equal(p, oracle.mx_quantize_sr(x, seed=12)[0])


def test_nv_tensor_keeps_the_deterministic_scales_and_picks_a_neighbour():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(16 * 128)).astype(np.float32)
    x[::61] *= 25
    p_det, s_det, sg_det, f_det = oracle.nv_quantize(x)
    p, s, sg, f = oracle.nv_quantize_sr(x, seed=99)
    assert f == f_det == 0
    assert sg == sg_det and np.array_equal(s, s_det)
    alpha = np.repeat(np.array([np.float32(np.float64(sg) * oracle.e4m3_value(int(c)))
                                for c in s], np.float64), 16)
    y = oracle.dequantize(oracle.NV, p, s, sg).astype(np.float64)
    lo, hi = _neighbour_values(x, alpha)
    # the dequantized value is RN32(code value * alpha); so are the bounds
    lo32, hi32 = lo.astype(np.float32).astype(np.float64), hi.astype(np.float32).astype(np.float64)
    assert np.all((y == lo32) | (y == hi32))


def test_draws_follow_the_element_index_not_the_block():
    """Element i draws the same bits wherever it sits: quantizing a prefix
    of whole blocks with the same seed gives the prefix of the codes."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal(32 * 40).astype(np.float32)
    full = oracle.mx_quantize_sr(x, seed=3)[0]
    head = oracle.mx_quantize_sr(x[: 32 * 13], seed=3)[0]
    assert np.array_equal(full[: head.size], head)


def test_mean_over_seeds_recovers_the_input():
    """End to end unbiasedness: averaged over many seeds, the dequantized
    tensor is consistent with expectation x (per element and summed), while
    nearest rounding on the same data is several times further off."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal(256).astype(np.float32)
    x[5] = 0.0
    x[9] = -0.0
    nseed = 2000
    acc = np.zeros(x.size)
    for sd in range(nseed):
        p, s, _ = oracle.mx_quantize_sr(x, seed=1000 + sd)
        acc += oracle.dequantize(oracle.MX, p, s).astype(np.float64)
    mean = acc / nseed
    s_det = oracle.mx_quantize(x)[1]
    lo, hi = _neighbour_values(x, _mx_scale_values(s_det))
    assert mean_within_bounds(x.astype(np.float64), lo, hi, mean, nseed)
    det = oracle.dequantize(oracle.MX, *oracle.mx_quantize(x)[:2]).astype(np.float64)
    assert np.abs(det - x).mean() > 5 * np.abs(mean - x).mean()
    # a planted bias of a tenth of a step is caught
    assert not mean_within_bounds(x.astype(np.float64), lo, hi, mean + 0.1 * np.abs(hi - lo),
                                  nseed)


@pytest.mark.parametrize("block,lead", [(32, 0), (16, 16)])
@pytest.mark.parametrize("seed", [3, 2**63 + 11])
def test_quotients_one_step_either_side_of_each_threshold(block, lead, seed):
    """Quotients placed at each element's own threshold round down, one fp32
    step above it round up: the decisions built from exact fractions."""
    x, want = threshold_blocks(block, 48, seed, offset=lead)
    if lead:  # NVFP4: a leading 2688 block fixes s_g = 1
        x = np.concatenate([np.full(lead, 2688.0, np.float32), x])
        p, s, sg, f = oracle.nv_quantize_sr(x, seed)
        assert float(sg) == 1.0
    else:
        p, s, f = oracle.mx_quantize_sr(x, seed)
    assert f == 0
    assert np.array_equal(oracle.unpack(p)[lead:], want)


def test_bf16_input_equals_widened_fp32_input():
    rng = np.random.default_rng(10)
    x = rng.standard_normal(32 * 8).astype(np.float32)
    bits = np.array([struct.unpack("<I", struct.pack("<f", v))[0] >> 16 for v in x], np.uint16)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    a = oracle.mx_quantize_sr(bits, seed=4)
    b = oracle.mx_quantize_sr(widened, seed=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.nv_quantize_sr(bits, seed=4)
    d = oracle.nv_quantize_sr(widened, seed=4)
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1]) and c[2] == d[2]


def test_nonfinite_flagged():
    x = np.ones(64, np.float32)
    x[3] = np.nan
    assert oracle.mx_quantize_sr(x, 1)[2] & oracle.FLAG_NONFINITE
    assert oracle.nv_quantize_sr(x, 1)[3] & oracle.FLAG_NONFINITE


def test_tiny_quotients_round_up_only_when_nonzero():
    """With zero random bits every nonzero quotient rounds up to 0.5 and a
    zero one stays: quotients far below 2^-25 decide only by being zero,
    which RN32(x / alpha) is exactly when |x / alpha| <= 2^-150 (the tie at
    2^-150 goes to the even value 0)."""
    assert oracle.sr_bits(SEED_ZERO_BITS_AT_16, 16) == 0
    for value, nv_code, mx_code in tiny_quotient_cases():
        xn = tiny_quotient_tensor(16, value)
        p, s, sg, f = oracle.nv_quantize_sr(xn, SEED_ZERO_BITS_AT_16)
        assert f == 0 and float(sg) == 1.0 and int(s[1]) == 0x40   # alpha = 2
        assert oracle.unpack(p)[16] == nv_code, value
        xm = tiny_quotient_tensor(32, value)
        p, s, f = oracle.mx_quantize_sr(xm, SEED_ZERO_BITS_AT_16)
        assert f == 0 and int(s[0]) == 127
        assert oracle.unpack(p)[16] == mx_code, value
