"""Pins for the oracle's E2M1 decode / RoundE2M1 / nibble packing.

Values come from the pages (golden fixtures) and from an independent closed
form of round-to-nearest with ties to the even code.
"""
import math
import struct

import numpy as np
import pytest

import oracle
from tests import _exact
from tests._golden import rows


def test_decode_table_matches_page():
    for code, value in rows("e2m1_table.txt"):
        v = oracle.e2m1_value(int(code))
        assert v == float(value)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(value))


def test_decode_8_is_negative_zero():
    assert oracle.e2m1_value(8) == 0.0
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0


def test_encode_of_decode_is_identity():
    for c in range(16):
        assert oracle.e2m1_round(oracle.e2m1_value(c)) == c


def test_midpoints_and_saturation_match_page():
    for x, want in rows("e2m1_midpoints.txt"):
        c = oracle.e2m1_round(float(x))
        assert oracle.e2m1_value(c) == float(want), x
        # the negated midpoint keeps the sign bit and the same magnitude code
        cn = oracle.e2m1_round(-float(x))
        assert cn == (c ^ 8)


def test_largest_finite_saturates_and_nonfinite_rejected():
    fmax = np.finfo(np.float32).max
    assert oracle.e2m1_value(oracle.e2m1_round(fmax)) == 6.0
    assert oracle.e2m1_value(oracle.e2m1_round(-fmax)) == -6.0
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert oracle.e2m1_round(bad) == -1


def test_sign_of_zero_is_kept():
    assert oracle.e2m1_round(-0.0) == 8
    assert oracle.e2m1_round(0.0) == 0
    assert oracle.e2m1_round(-0.1) == 8      # rounds to zero, keeps the sign bit
    assert oracle.e2m1_round(-1e-45) == 8


def _ladder(q: np.ndarray) -> np.ndarray:
    """Closed form of nearest-E2M1 with ties to the even code: count the
    decision thresholds passed.  A midpoint between an even code below and
    an odd code above stays below (strict >); between an odd code below and
    an even code above it moves up (>=)."""
    m = np.minimum(np.abs(q.astype(np.float64)), 6.0)
    k = ((m > 0.25).astype(np.int32) + (m >= 0.75) + (m > 1.25) + (m >= 1.75)
         + (m > 2.5) + (m >= 3.5) + (m > 5.0))
    return (np.signbit(q).astype(np.int32) << 3) | k


def _neighbourhood(center: float, span: int) -> np.ndarray:
    b = np.frombuffer(struct.pack("<f", center), np.uint32)[0]
    bits = np.arange(int(b) - span, int(b) + span + 1, dtype=np.int64)
    bits = bits[(bits >= 0) & (bits < 0x7F800000)].astype(np.uint32)
    f = bits.view(np.float32)
    return np.concatenate([f, -f])


def test_round_matches_closed_form_on_all_bf16_and_near_every_decision_point():
    allbf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf)]
    parts = [allbf]
    for p in (0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0):
        parts.append(_neighbourhood(p, 1 << 14))
    rng = np.random.default_rng(1234)
    rnd = rng.integers(0, 0x7F800000, size=1 << 21, dtype=np.uint32).view(np.float32)
    parts += [rnd, -rnd]
    q = np.concatenate(parts).astype(np.float32)
    got = oracle.e2m1_round_array(q)
    assert np.array_equal(got.astype(np.int32), _ladder(q))


def test_round_matches_exact_brute_force_sample():
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.uniform(-7, 7, 300), rng.normal(0, 1e-3, 50)]).astype(np.float32)
    for v in vals:
        assert oracle.e2m1_round(v) == _exact.e2m1_code_of_f32(v)


def test_pack_codes_0_15_matches_page():
    want = bytes.fromhex("".join(rows("pack_codes.txt")[0]))
    assert oracle.pack(np.arange(16, dtype=np.uint8)).tobytes() == want


def test_pack_unpack_roundtrip_and_odd_length_rejected():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, 1000, dtype=np.uint8)
    assert np.array_equal(oracle.unpack(oracle.pack(codes)), codes)
    with pytest.raises(ValueError):
        oracle.pack(np.array([1, 2, 3], np.uint8))
