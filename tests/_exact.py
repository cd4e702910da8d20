"""Exact-arithmetic brute force used to pin the oracle (tests only).

Everything here works on fractions.Fraction, independent of the oracle's C
code and of any floating-point division: rounding to binary32 is done by
locating the value between consecutive representable numbers, and nearest
E2M1 / E4M3 values are found by comparing exact distances over the whole
code table (ties to the even code, as the format page prescribes).
"""
from fractions import Fraction

import numpy as np

E2M1_MAG = [Fraction(v) for v in ("0", "1/2", "1", "3/2", "2", "3", "4", "6")]


def e4m3_pos_values():
    vals = []
    for c in range(127):
        e, f = c >> 3, c & 7
        if e == 0:
            vals.append(Fraction(f, 512))
        else:
            vals.append(Fraction(8 + f, 8) * Fraction(2) ** (e - 7))
    return vals


E4M3_POS = e4m3_pos_values()


def floor_log2(a: Fraction) -> int:
    assert a > 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rn32(r: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32, ties to even."""
    if r == 0:
        return np.float32(0.0)
    neg = r < 0
    a = -r if neg else r
    e = floor_log2(a)
    ulp = Fraction(2) ** max(e - 23, -149)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * ulp
    f = np.float32(float(v))
    assert Fraction(float(f)) == v, "value not representable"
    return np.float32(-f) if neg else f


def e2m1_code_of_f32(q: np.float32) -> int:
    """Nearest E2M1 code to an fp32 value; sign from the sign bit."""
    sign = 8 if np.signbit(q) else 0
    m = min(abs(Fraction(float(q))), Fraction(6))
    best = min(range(8), key=lambda c: (abs(E2M1_MAG[c] - m), c & 1))
    return sign | best


def e4m3_nearest(t: Fraction) -> int:
    t = min(t, E4M3_POS[126])
    return min(range(127), key=lambda c: (abs(E4M3_POS[c] - t), c & 1))


def nv_tensor_scale(xs) -> np.float32:
    A = max(abs(Fraction(float(v))) for v in xs)
    if A == 0:
        return np.float32(1.0)
    return rn32(A / 2688)


def nv_block(xs, s_g: np.float32):
    """(scale code, element codes) of one 16-block by the exact definition."""
    A_g = max(abs(Fraction(float(v))) for v in xs)
    sg = Fraction(float(s_g))
    code = 0x38 if A_g == 0 else e4m3_nearest(A_g / (6 * sg))
    alpha = rn32(sg * E4M3_POS[code])
    codes = []
    for v in xs:
        fv = np.float32(v)
        q = rn32(Fraction(float(fv)) / Fraction(float(alpha)))
        if q == 0 and np.signbit(fv):
            q = np.float32(-0.0)
        codes.append(e2m1_code_of_f32(q))
    return code, codes


def mx_block(xs):
    """(scale byte, element codes) of one 32-block by the exact definition."""
    A_g = max(abs(Fraction(float(v))) for v in xs)
    e = 0 if A_g == 0 else max(floor_log2(A_g) - 2, -127)
    s = Fraction(2) ** e
    codes = []
    for v in xs:
        fv = np.float32(v)
        q = rn32(Fraction(float(fv)) / s)
        if q == 0 and np.signbit(fv):
            q = np.float32(-0.0)
        codes.append(e2m1_code_of_f32(q))
    return e + 127, codes
