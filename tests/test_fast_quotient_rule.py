"""The quotient shortcuts of the one-pass NVFP4 kernel, checked by brute force.

The method divides each element by its block's alpha with a correctly
rounded fp32 division and rounds the quotient to E2M1.  For bf16 input the
kernel uses cheaper forms where they provably give the same result:

1. q0 = RN32(x * RN32(1 / a)) unless the block's divisor a is flagged:
   flagged when, for some E2M1 decision point m ("NVFP4 / MXFP4 format" page,
   section 1: the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), m * a lies
   within 2^-22 (relative) of a number with at most 8 significant bits.  The
   claim: for an unflagged a, every finite bf16 x gets the same E2M1 code from
   q0 as from RN32(x / a).  The rule is restated here from its definition
   (binary64 distance to the nearest 8-bit-significand value); the E2M1 code
   is the closed-form ladder of the midpoints, ties to the even code.
2. For a divisor with at most 16 significant bits, fma(x, yh, RN32(x yl))
   with yh = RD32(1/a), yl = RN32(1/a - yh) >= 0 equals RN32(x / a) bit for
   bit (checked in exact rational arithmetic).

No GPU.
"""
import numpy as np

MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_magnitude_code(q: np.ndarray) -> np.ndarray:
    m = np.abs(q.astype(np.float64))
    return ((m > 0.25).astype(np.int8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5)
            + (m >= 3.5) + (m > 5.0))


def e2m1_code(q: np.ndarray) -> np.ndarray:
    return e2m1_magnitude_code(q) | (np.signbit(q).astype(np.int8) << 3)


def flagged(a: np.float32) -> bool:
    """Restated rule: distance, in units of 2^(e-52), from m*a to the nearest
    value with 8 significant bits is at most 2^31 for some midpoint m."""
    p = MIDS * np.float64(a)
    b = p.view(np.uint64)
    low = b & np.uint64((1 << 45) - 1)
    dist = np.minimum(low, np.uint64(1 << 45) - low)
    return bool((dist <= np.uint64(1 << 31)).any())


def all_bf16_finite() -> np.ndarray:
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    return x[np.isfinite(x)]


def codes_both_ways(x: np.ndarray, a: np.float32):
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        y = np.float32(1.0) / a
        q_div = (x / a).astype(np.float32)
        q_mul = (x * y).astype(np.float32)
    return e2m1_code(q_div), e2m1_code(q_mul)


def relevant(x: np.ndarray, a: np.float32) -> np.ndarray:
    # in a block whose scale is a, |x| / a stays below ~6.5 (the block amax
    # rounds to the scale within one E4M3 step)
    return x[np.abs(x.astype(np.float64)) <= 8.0 * np.float64(a)]


def test_rule_is_sound_on_random_divisors():
    rng = np.random.default_rng(11)
    xs = all_bf16_finite()
    # divisors over the normal range the kernels use (alpha' >= 2^-90)
    sig = rng.integers(1 << 23, 1 << 24, size=400).astype(np.float64)
    exp = rng.integers(-90, 100, size=400)
    divisors = (sig * 2.0 ** (exp - 23)).astype(np.float32)
    checked = 0
    for a in divisors:
        if flagged(a):
            continue
        x = relevant(xs, a)
        cd, cm = codes_both_ways(x, a)
        bad = np.nonzero(cd != cm)[0]
        assert bad.size == 0, f"a={a!r}: x={x[bad[0]]!r} codes {cd[bad[0]]} vs {cm[bad[0]]}"
        # the scaled form used for tiny alphas: (x 2^64) / (a 2^64), same quotient
        checked += 1
    assert checked > 350


def test_rule_flags_every_divisor_where_the_product_errs():
    """Divisors built so that a midpoint multiple is (nearly) a bf16 value:
    whenever the two ways disagree, the rule must have flagged the divisor."""
    rng = np.random.default_rng(12)
    xs = all_bf16_finite()
    found_disagreement = 0
    for trial in range(600):
        m = MIDS[trial % 7]
        # X with 8 significant bits, a = X / m nudged by a few ulps
        X = np.float64(rng.integers(128, 256)) * 2.0 ** int(rng.integers(-30, 30))
        a0 = np.float32(X / m)
        a = np.nextafter(a0, np.float32(np.inf)) if trial % 3 == 1 else (
            np.nextafter(a0, np.float32(0)) if trial % 3 == 2 else a0)
        x = relevant(xs, a)
        cd, cm = codes_both_ways(x, a)
        if (cd != cm).any():
            found_disagreement += 1
            assert flagged(a), f"unflagged divisor {a!r} where the product errs"
    # the construction does produce divisors on which the product errs
    assert found_disagreement > 0


def test_scaled_operands_keep_the_quotient():
    # x / a == (x 2^64) / (a 2^64) in fp32 for tiny a and bf16-range x
    rng = np.random.default_rng(13)
    for _ in range(200):
        a = np.float32(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-149, -90)))
        if a == 0:
            continue
        x = np.float32(a * rng.uniform(0, 7))
        s = np.float32(2.0 ** 64)
        with np.errstate(under="ignore"):
            assert np.float32(x / a) == np.float32((x * s) / (a * s))


# ---- the two-operation quotient for short divisors ------------------------------
#
# When the tensor scale has at most 12 significant bits every block divisor a
# has at most 16, and the one-pass kernel computes the quotient as
# fma(x, yh, RN32(x * yl)) with yh = RD32(1/a) and yl = RN32(1/a - yh) >= 0.
# The claim: that is exactly RN32(x / a) (bit for bit, -0 included) for every
# bf16 x.  Checked in exact rational arithmetic.

from fractions import Fraction  # noqa: E402

from tests._exact import rn32  # noqa: E402


def _two_float_reciprocal(a: np.float32):
    r = 1.0 / np.float64(a)                 # binary64 reciprocal, as the kernel's table build
    yh = np.float32(r)
    if np.float64(yh) > r:
        yh = np.nextafter(yh, np.float32(0))
    yl = np.float32(r - np.float64(yh))
    return yh, yl


def _two_op_quotient(x: np.float32, yh: np.float32, yl: np.float32) -> np.float32:
    p = rn32(Fraction(float(x)) * Fraction(float(yl)))
    if p == 0 and np.signbit(x):
        p = np.float32(-0.0)                 # RN32 of a zero product keeps the sign rule
    s = Fraction(float(x)) * Fraction(float(yh)) + Fraction(float(p))
    if s == 0:
        # exact zero sum: -0 only when both addends are -0 (round to nearest)
        neg = np.signbit(x) and np.signbit(p)
        return np.float32(-0.0) if neg else np.float32(0.0)
    return rn32(s)


def test_two_operation_quotient_is_correctly_rounded_for_short_divisors():
    rng = np.random.default_rng(14)
    xs = all_bf16_finite()
    checked = n_ties = 0
    for trial in range(60):
        # divisor with at most 16 significant bits, as s_g (<= 12) times E4M3
        # (<= 4); every other s_g has at most 4 bits (as A = 21 k 2^e gives),
        # so that exact ties x = m a occur
        bits = 12 if trial % 2 == 0 else 4
        sg = np.float32(int(rng.integers(1 << (bits - 1), 1 << bits)) * 2.0 ** int(rng.integers(-40, 0)))
        code = int(rng.integers(8, 127))
        e, f = code >> 3, code & 7
        a = np.float32(sg * np.float32((8 + f) / 8 * 2.0 ** (e - 7)))
        yh, yl = _two_float_reciprocal(a)
        assert yl >= 0
        x = relevant(xs, a)
        x = x[(np.abs(x.astype(np.float64)) >= 0.2 * np.float64(a)) | (x == 0)]
        # every exact tie x = m a that bf16 can hold, plus a sample of the rest
        ties = []
        for m in MIDS:
            t = np.float32(m * np.float64(a))
            if (t.view(np.uint32) & 0xFFFF) == 0 and np.float64(t) == m * np.float64(a):
                ties.append(t)          # m a is itself a bf16 value
        n_ties += len(ties)
        sample = np.concatenate([np.array(ties, np.float32), -np.array(ties, np.float32),
                                 x[:: max(1, x.size // 400)]])
        for xv in sample:
            want = rn32(Fraction(float(xv)) / Fraction(float(a)))
            if want == 0 and np.signbit(xv):
                want = np.float32(-0.0)
            got = _two_op_quotient(xv, yh, yl)
            assert got.view(np.uint32) == want.view(np.uint32), (a, xv, got, want)
            checked += 1
    assert checked > 10000 and n_ties > 20
