"""The reciprocal-correction table of the one-pass NVFP4 kernel
(csrc/fp4_recip_table.h) is what its generator's rule gives, and the rule is
sound on exhaustive checks: for sampled (M, k) the chosen reciprocal's product
gives every bf16 value of the decision-point neighbourhoods the E2M1 code of
the correctly rounded quotient (exact rational arithmetic)."""
import importlib.util
import os
import random
from fractions import Fraction as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_block_amax_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_recip_table", os.path.join(CSRC, "gen_recip_table.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_committed_header_matches_the_generator():
    g = _gen()
    with open(os.path.join(CSRC, "fp4_recip_table.h")) as f:
        assert f.read() == g.render(g.table())


def test_chosen_reciprocal_is_exact_on_every_nearby_bf16_value():
    # independent of the hazard shortcut: every bf16 value within 2^-12 of
    # each decision point m alpha (hundreds per point), both the chosen
    # candidate's product and the correctly rounded quotient, compared
    g = _gen()
    t = g.table()
    rng = random.Random(5)
    cases = [(M, k) for M in range(128) for k in range(8) if t[M][k] != 3]
    for M, k in rng.sample(cases, 24) + [(12, 0), (40, 6), (82, 3)]:
        s = g.rn(F(128 + M, 128) / 2688, 24)
        a = g.rn(s * F(8 + k, 8), 24)
        y0 = g.rn(1 / a, 24)
        choice = t[M][k]
        y = {0: y0, 1: y0 - (g.ulp24(y0 / 2) if y0 == F(2) ** g.binade(y0) else g.ulp24(y0)),
             2: y0 + g.ulp24(y0)}[choice]
        for m in g.MIDS:
            c = m * a
            e = g.binade(c)
            step = F(2) ** (e - 7)  # bf16 spacing near c
            base = (c // step) * step
            for j in range(-40, 41):
                x = base + j * step
                if x <= 0:
                    continue
                assert g.e2m1(g.rn(x * y, 24)) == g.e2m1(g.rn(x / a, 24)), (M, k, m, x)


def test_two_operation_codes_are_exact_ties():
    # the five entries no reciprocal fits hold an alpha with few significant
    # bits, where some bf16 value is exactly m alpha
    g = _gen()
    t = g.table()
    fours = [(M, k) for M in range(128) for k in range(8) if t[M][k] == 3]
    assert 0 < len(fours) <= 16
    for M, k in fours:
        s = g.rn(F(128 + M, 128) / 2688, 24)
        a = g.rn(s * F(8 + k, 8), 24)
        assert any(g.rn(m * a, 8) == m * a for m in g.MIDS), (M, k)
        n = a.numerator
        while n % 2 == 0:
            n //= 2
        assert n.bit_length() <= 16, (M, k)  # what the two-operation quotient needs
