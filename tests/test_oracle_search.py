"""Pins for the oracle's MSE-optimal NVFP4 block-scale search."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import _exact
from tests._golden import keyed

G = keyed("nv_scale_examples.txt")


def _exact_mse(block, alpha) -> Fraction:
    """Exact mean squared error of a block reconstructed at fp32 scale alpha."""
    tot = Fraction(0)
    a = Fraction(float(alpha))
    for v in block:
        q = _exact.rn32(Fraction(float(v)) / a)
        c = _exact.e2m1_code_of_f32(q)
        xh = _exact.rn32(Fraction(float(oracle.e2m1_value(c))) * a)
        tot += (Fraction(float(v)) - Fraction(float(xh))) ** 2
    return tot / len(block)


def test_candidates_are_linspace_rounded_once():
    cs = [oracle.candidate_c(k) for k in range(64)]
    assert cs[0] == 0.5 and cs[63] == 1.0
    for k, c in enumerate(cs):
        assert c == _exact.rn32(Fraction(63 + k, 126))


def test_counterexample_search_picks_maxbased_and_brute_force_finds_better():
    v, n, big = G["counter"][0]
    block = np.asarray([float(v)] * int(n) + [float(big)], np.float32)
    x = np.concatenate([np.full(16, 2688.0, np.float32), block])
    packed, scales, s_g, flags = oracle.scale_search(x)
    assert flags == 0 and s_g == 1.0
    # candidates alpha = (3.6/6) c, c in [0.5, 1]: every E4M3 code from 0.3125
    # to 0.625; the loss falls monotonically, so the max-based 0.625 wins
    winner = oracle.e4m3_value(int(scales[1]))
    sc, num, den = G["counter_maxbased"][0]
    assert winner == float(sc)
    cands = [0.3125, 0.34375, 0.375, 0.40625, 0.4375, 0.46875, 0.5, 0.5625, 0.625]
    mses = [_exact_mse(block, c) for c in cands]
    assert all(mses[i] > mses[i + 1] for i in range(len(mses) - 1))
    assert mses[-1] == pytest.approx(int(num) / int(den), rel=1e-6)
    # brute force over every nonzero E4M3 code finds the page's better scale
    best = min(range(1, 127), key=lambda c: (_exact_mse(block, oracle.e4m3_value(c)), c))
    sc2, num2, den2 = G["counter_better"][0]
    assert oracle.e4m3_value(best) == float(sc2)
    assert float(_exact_mse(block, oracle.e4m3_value(best))) == pytest.approx(int(num2) / int(den2), rel=1e-6)


def test_search_with_wider_range_reaches_better_scale():
    v, n, big = G["counter"][0]
    block = np.asarray([float(v)] * int(n) + [float(big)], np.float32)
    x = np.concatenate([np.full(16, 2688.0, np.float32), block])
    packed, scales, s_g, flags = oracle.scale_search(x, ncand=64, c_lo=0.5, c_hi=1.5)
    assert oracle.e4m3_value(int(scales[1])) == 0.875


def _blocks(seed, nblocks=64):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(nblocks * 16, generator=g) * torch.rand(nblocks * 16, generator=g)
    return x.numpy().astype(np.float32)


def test_winner_never_worse_than_maxbased_and_is_a_candidate():
    x = _blocks(1)
    s_g, _ = oracle.nv_global_scale(x)
    p_s, sc_s, f_s, loss = oracle.scale_search_with_scale(x, s_g, want_loss=True)
    p_m, sc_m, f_m = oracle.nv_quantize_with_scale(x, s_g)
    assert f_s == 0 and f_m == 0
    for b in range(x.size // 16):
        xb = x[16 * b:16 * b + 16]
        L_max = oracle.block_loss(xb, float(np.float32(float(s_g) * oracle.e4m3_value(int(sc_m[b])))))
        assert loss[b] <= L_max
        amax = float(np.abs(xb).max())
        lo = oracle.e4m3_nearest(0.5 * amax, 6.0 * float(s_g))
        assert max(lo, 1) <= sc_s[b] <= sc_m[b]


def test_distinct_candidate_codes_form_a_contiguous_range():
    """The 64 encoded candidates of a block are exactly the E4M3 codes from
    E4M3(c_0 t) to E4M3(c_63 t) (t = A_g / (6 s_g)): the candidate grid is
    finer than the E4M3 grid everywhere, so no code in between is skipped."""
    rng = np.random.default_rng(31)
    s_g = np.float32(1.0)
    amaxes = np.concatenate([rng.uniform(1e-4, 2688, 300), 2.0 ** rng.uniform(-12, 12, 300)])
    # the grids the library accepts: step (c_hi - c_lo)/(n - 1) <= c_lo/24
    grids = [(64, 0.5, 1.0), (64, 0.5, 1.5), (33, 0.75, 1.25), (13, 0.5, 0.75)]
    for n, c_lo, c_hi in grids:
        assert (c_hi - c_lo) / (n - 1) <= c_lo / 24
        for amax in amaxes.astype(np.float32):
            cs = [float(oracle.candidate_c(k, n, c_lo, c_hi)) for k in range(n)]
            codes = {oracle.e4m3_nearest(c * float(amax), 6.0) for c in cs}
            lo = oracle.e4m3_nearest(cs[0] * float(amax), 6.0)
            hi = oracle.e4m3_nearest(cs[-1] * float(amax), 6.0)
            assert codes == set(range(lo, hi + 1)), (n, c_lo, c_hi, amax)


def test_zero_block_and_underflow():
    x = np.concatenate([np.full(16, 2688.0, np.float32), np.zeros(16, np.float32)])
    p, sc, s_g, flags = oracle.scale_search(x)
    assert flags == 0 and sc[1] == 0x38 and np.all(oracle.unpack(p)[16:] == 0)
    x = np.concatenate([np.full(16, 2688.0, np.float32), np.full(16, 1e-10, np.float32)])
    assert oracle.scale_search(x)[3] & oracle.FLAG_SCALE_UNDERFLOW


def test_loss_is_pairwise_fp32_sum():
    rng = np.random.default_rng(41)
    xb = rng.normal(0, 1, 16).astype(np.float32)
    alpha = np.float32(0.37)
    t = []
    for v in xb:
        q = np.float32(v / alpha)
        c = oracle.e2m1_round(q)
        xh = np.float32(np.float64(oracle.e2m1_value(c)) * np.float64(alpha))
        e = np.float32(v - xh)
        t.append(np.float32(e * e))
    while len(t) > 1:
        t = [np.float32(t[2 * i] + t[2 * i + 1]) for i in range(len(t) // 2)]
    assert oracle.block_loss(xb, float(alpha)) == t[0]


def test_equal_losses_go_to_the_smallest_candidate():
    # [3.75, 0 x 15] under a = 1: both 0.625 (3.75 = 6 * 0.625) and 0.9375
    # (3.75 = 4 * 0.9375) reconstruct it exactly; with c up to 1.5 both are
    # candidates, and the smaller one (smaller k, smaller code) wins
    block = np.zeros(16, np.float32)
    block[0] = 3.75
    x = np.concatenate([np.full(16, 2688.0, np.float32), block])
    p, sc, s_g, flags = oracle.scale_search(x, ncand=64, c_lo=0.5, c_hi=1.5)
    assert flags == 0 and oracle.e4m3_value(int(sc[1])) == 0.625
    assert oracle.block_loss(block, 0.9375) == 0.0 and oracle.block_loss(block, 0.625) == 0.0


# ---- brute force over every E4M3 code, and the wider range ------------------

def test_brute_force_search_finds_the_pages_better_scale():
    v, n, big = G["counter"][0]
    block = np.asarray([float(v)] * int(n) + [float(big)], np.float32)
    x = np.concatenate([np.full(16, 2688.0, np.float32), block])
    packed, scales, s_g, flags = oracle.scale_search_all(x)
    assert flags == 0 and s_g == 1.0
    sc2, num2, den2 = G["counter_better"][0]
    assert oracle.e4m3_value(int(scales[1])) == float(sc2)
    _, _, _, loss = oracle.scale_search_all_with_scale(block, 1.0, want_loss=True)
    assert float(loss[0]) / 16 == pytest.approx(int(num2) / int(den2), rel=1e-6)


def test_brute_force_winner_has_the_least_exact_loss():
    g = torch.Generator().manual_seed(31)
    x = (torch.randn(6 * 16, generator=g) * torch.rand(6 * 16, generator=g)).numpy().astype(np.float32)
    s_g = np.float32(0.01)
    _, scales, flags, loss = oracle.scale_search_all_with_scale(x, s_g, want_loss=True)
    assert flags == 0
    for b in range(6):
        blk = x[16 * b: 16 * b + 16]
        exact = {c: _exact_mse(blk, np.float32(s_g * np.float32(oracle.e4m3_value(c))))
                 for c in range(1, 127)}
        best = min(exact.values())
        w = int(scales[b])
        # the fp32 loss may reorder candidates whose exact losses differ by
        # less than its rounding error; none does by more
        assert exact[w] <= best * (1 + Fraction(80, 2 ** 24))


def test_brute_force_never_worse_than_the_range_searches():
    x = _blocks(32, 128)
    s_g = np.float32(np.abs(x).max() / 2688)
    _, s_all, f, l_all = oracle.scale_search_all_with_scale(x, s_g, want_loss=True)
    for lo, hi in [(0.5, 1.0), (0.5, 1.5)]:
        _, s_r, f_r, l_r = oracle.scale_search_with_scale(x, s_g, c_lo=lo, c_hi=hi, want_loss=True)
        assert f == 0 and f_r == 0
        assert np.all(l_all <= l_r)


def test_wider_range_maps_the_max_to_4_for_the_pages_block():
    gold = keyed("scale_choice_examples.txt")
    vals = [float(v) for v in gold["four_over_six"][0]]
    want_scale = float(gold["four_over_six_scale"][0][0])
    block = np.asarray(vals * 4, np.float32)
    packed, scales, flags, loss = oracle.scale_search_with_scale(block, 1.0, c_lo=0.5, c_hi=1.5,
                                                                 want_loss=True)
    assert flags == 0 and oracle.e4m3_value(int(scales[0])) == want_scale and loss[0] == 0.0
    y = oracle.dequantize(oracle.NV, packed, scales, 1.0)
    assert np.array_equal(y, block)
    # the default range c in [0.5, 1] cannot reach amax / 4
    _, s2, _, l2 = oracle.scale_search_with_scale(block, 1.0, want_loss=True)
    assert oracle.e4m3_value(int(s2[0])) < want_scale and l2[0] > 0.0
