"""Test-side cases for stochastic rounding, shared by the oracle pins and the
GPU parity tests.  Nothing here rounds stochastically: expected decisions
are built from exact fractions and the element's random bits."""
from fractions import Fraction

import numpy as np

import oracle
from tests._exact import E2M1_MAG

TWO24 = 2**24


def neighbours(m: Fraction):
    """(lo, hi, code_lo) with lo <= m < hi consecutive E2M1 magnitudes."""
    for k in range(7):
        if E2M1_MAG[k] <= m < E2M1_MAG[k + 1]:
            return E2M1_MAG[k], E2M1_MAG[k + 1], k
    raise AssertionError(m)


def neighbour_values(q: np.ndarray, scale: np.ndarray):
    """Per element of the fp32 quotients q: the E2M1 neighbours below and
    above |q| (both 6 past the top), with q's sign, times scale."""
    lo = np.empty(q.size)
    hi = np.empty(q.size)
    for i, v in enumerate(np.asarray(q, np.float32)):
        m = Fraction(abs(float(v)))
        if m >= 6:
            lo[i] = hi[i] = 6.0
        else:
            a, b, _ = neighbours(m)
            lo[i], hi[i] = float(a), float(b)
    sgn = np.where(np.signbit(q), -1.0, 1.0)
    return sgn * lo * scale, sgn * hi * scale


def threshold_blocks(block: int, nblocks: int, seed: int, offset: int = 0):
    """fp32 blocks whose first element pins the scale to 1 (MXFP4: 7.5, an
    exponent-0 block; NVFP4: 6, block code 0x38 under s_g = 1) and whose other
    elements, with the scale 1, are quotients just at (rounds down) or one
    fp32 step above (rounds up) the threshold lo + r (hi - lo) 2^-24 of their
    own random bits r (element j of the result has flat index offset + j).
    Returns (values, expected codes)."""
    vals = [float(v) for v in E2M1_MAG]
    x = np.zeros(block * nblocks, np.float32)
    want = np.zeros(block * nblocks, np.uint8)
    for b in range(nblocks):
        sign = -1.0 if b % 3 == 1 else 1.0
        i0 = b * block
        x[i0] = sign * (7.5 if block == 32 else 6.0)
        want[i0] = (8 if sign < 0 else 0) | 7
        for j in range(1, block):
            i = i0 + j
            k = (b + j) % 7
            lo, hi = Fraction(vals[k]), Fraction(vals[k + 1])
            r = oracle.sr_bits(seed, offset + i)
            t = lo + (hi - lo) * Fraction(r, TWO24)          # exact in binary64
            down = np.float32(float(t))
            if Fraction(float(down)) > t:
                down = np.nextafter(down, np.float32(0))
            up = np.nextafter(down, np.float32(np.inf))
            go_up = (i // 7) % 2 == 1
            q = up if go_up else down
            if Fraction(float(q)) >= hi:                      # only when r is near 2^24
                q, go_up = down, False
            x[i] = np.float32(sign * float(q))
            want[i] = (8 if np.signbit(x[i]) else 0) | (k + 1 if go_up else k)
    return x, want


# Failure probability allowed to each statistical check below.
STAT_DELTA = 1e-9


def bernstein_halfwidth(var: np.ndarray, bound: np.ndarray, delta: float = STAT_DELTA):
    """Half-width t of Bernstein's inequality for a sum of independent,
    zero-mean terms each bounded by `bound` in magnitude, with total variance
    `var`: P(|sum| >= t) <= 2 exp(-t^2 / (2 (var + bound t / 3))) = delta.
    Unlike a k-sigma rule it holds for every distribution of the terms, in
    particular for the skewed two-point draws of a rounding probability near 0
    or 1."""
    L = np.log(2.0 / delta)
    a = bound * L / 3.0
    return a + np.sqrt(a * a + 2.0 * L * var)


def mean_within_bounds(x: np.ndarray, lo: np.ndarray, hi: np.ndarray, mean: np.ndarray, n: int):
    """Whether the mean of n independent two-point draws (lo or hi, up with
    probability p = (x - lo) / (hi - lo)) is consistent with its expectation
    x (x clamped to the saturation value where lo = hi): every element, and
    the sum over elements, within Bernstein's bound at failure probability
    STAT_DELTA.  Per element the mean is a sum of n terms bounded by
    (hi - lo) / n with variance (hi - lo)^2 p (1 - p) / n."""
    x = np.where(lo == hi, lo, x)  # saturated: the draw is always +-6 scale
    gap = np.abs(hi - lo)
    p = np.where(gap > 0, np.abs(x - lo) / np.where(gap > 0, gap, 1), 0.0)
    var = gap * gap * p * (1 - p) / n
    dev = mean - x
    ok_each = bool(np.all(np.abs(dev) <= bernstein_halfwidth(var, gap / n) + 1e-12))
    ok_sum = bool(abs(dev.sum()) <= bernstein_halfwidth(var.sum(), gap.max() / n) + 1e-12)
    return ok_each and ok_sum


# A seed whose 24 random bits are zero at element 16 (found by search; the
# tests check it): with r = 0 every nonzero quotient rounds up, so quotients
# far below 2^-25 decide only by whether they are zero.
SEED_ZERO_BITS_AT_16 = 1269119


def tiny_quotient_cases():
    """(value at element 16, expected NVFP4 code there, expected MXFP4 code)
    for the tensors built by tiny_quotient_tensor: NVFP4 alpha = 2 (a 2688
    block fixes s_g = 1, the test block holds 12), MXFP4 scale 1 (the block
    holds 4).  RN32(x / alpha) is zero exactly when |x / alpha| <= 2^-150."""
    return [
        (2.0**-148, 1, 1),    # NV q = 2^-149: nonzero, up.  MX q = 2^-148: up
        (-(2.0**-148), 9, 9),
        (2.0**-149, 0, 1),    # NV q = 2^-150, the tie, rounds to 0: stays 0.  MX q = 2^-149: up
        (1e-35, 1, 1),        # normal fp32, quotient below 2^-100: up
        (0.0, 0, 0),
        (-0.0, 8, 8),
    ]


def tiny_quotient_tensor(fmt_block: int, value: float) -> np.ndarray:
    if fmt_block == 16:
        x = np.zeros(32, np.float32)
        x[:16] = 2688.0
        x[17] = 12.0
    else:
        x = np.zeros(32, np.float32)
        x[0] = 4.0
    x[16] = np.float32(value)
    return x
