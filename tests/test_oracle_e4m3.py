"""Pins for the oracle's E4M3FN decode and nearest-code scale encoder."""
import math
from fractions import Fraction

import numpy as np

import oracle
from tests import _exact
from tests._golden import keyed


def test_value_table_shape_and_named_codes():
    vals = [oracle.e4m3_value(c) for c in range(127)]
    assert vals == sorted(vals) and len(set(vals)) == 127
    assert oracle.e4m3_value(0x7E) == 448.0          # max finite (format page s.2)
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x32) == 0.625
    assert oracle.e4m3_value(0x36) == 0.875
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert oracle.e4m3_value(0xB8) == -1.0


def test_ranges_match_precision_page_table():
    r = keyed("format_ranges.txt")
    mx, mn_norm, mn_pos = map(float, r["e4m3"][0])
    assert oracle.e4m3_value(0x7E) == mx
    assert oracle.e4m3_value(0x08) == mn_norm
    assert oracle.e4m3_value(0x01) == mn_pos
    mx, mn_norm, mn_pos = map(float, r["e2m1"][0])
    assert oracle.e2m1_value(7) == mx and oracle.e2m1_value(2) == mn_norm and oracle.e2m1_value(1) == mn_pos


def test_page_scale_examples():
    assert oracle.e4m3_value(oracle.e4m3_nearest(0.6, 1.0)) == 0.625   # format page s.4
    assert oracle.e4m3_nearest(0.875, 1.0) == 0x36
    assert oracle.e4m3_nearest(448.0, 1.0) == 0x7E
    assert oracle.e4m3_nearest(1e30, 1.0) == 0x7E                      # saturation
    # 2688 / (6 * a) with a = 1: the tensor-max block saturates at 448
    assert oracle.e4m3_nearest(2688.0, 6.0) == 0x7E


def test_ties_go_to_even_code():
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    assert oracle.e4m3_nearest(1.0625, 1.0) == 0x38
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): 0x3A
    assert oracle.e4m3_nearest(1.1875, 1.0) == 0x3A
    # subnormal midpoints: 2^-10 -> 0, 3*2^-10 -> code 2
    assert oracle.e4m3_nearest(2.0 ** -10, 1.0) == 0
    assert oracle.e4m3_nearest(3 * 2.0 ** -10, 1.0) == 2
    # 432 between 416 (0x7D) and 448 (0x7E): even 0x7E
    assert oracle.e4m3_nearest(432.0, 1.0) == 0x7E


def test_nearest_matches_exact_brute_force():
    rng = np.random.default_rng(11)
    cases = []
    for _ in range(300):
        s_g = np.float32(rng.uniform(1e-6, 10.0))
        A_g = np.float32(rng.uniform(0, 2688.0) * float(s_g))
        cases.append((float(A_g), float(s_g)))
    # adversarial: numerators placed exactly on or one fp32 ulp around midpoints
    for c in range(0, 126, 5):
        mid = (_exact.E4M3_POS[c] + _exact.E4M3_POS[c + 1]) / 2
        for s_g in (np.float32(1.0), np.float32(0.3), np.float32(1.7e-5)):
            a = _exact.rn32(mid * 6 * Fraction(float(s_g)))
            for v in (np.nextafter(a, np.float32(0)), a, np.nextafter(a, np.float32(1e9))):
                cases.append((float(v), float(s_g)))
    for A_g, s_g in cases:
        want = _exact.e4m3_nearest(Fraction(A_g) / (6 * Fraction(s_g)))
        assert oracle.e4m3_nearest(A_g, 6.0 * s_g) == want, (A_g, s_g)
