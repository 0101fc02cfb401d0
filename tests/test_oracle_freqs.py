"""Pins of the oracle's frequency rules against closed forms, special cases and
printed values (CPU only)."""

import math

import numpy as np
import pytest

from oracle import freqs

# (head_dim, base, factor, original length) of the workloads
CONFIGS = [
    (64, 10000.0, 4.0, 64),
    (128, 10000.0, 4.0, 4096),
    (128, 500000.0, 8.0, 16384),
]


@pytest.mark.parametrize("d,base", [(64, 10000.0), (128, 10000.0), (128, 500000.0), (8, 16.0)])
def test_theta_closed_form(d, base):
    th = freqs.rope_theta(d, base)
    assert th.shape == (d // 2,)
    assert th[0] == 1.0
    # last pair: base^(-(d-2)/d), written through exp/log instead of pow
    assert th[-1] == pytest.approx(math.exp(-(d - 2) / d * math.log(base)), rel=1e-14)
    assert np.all(np.diff(th) < 0)
    # geometric series: constant ratio base^(-2/d)
    ratios = th[1:] / th[:-1]
    assert np.allclose(ratios, math.exp(-2.0 / d * math.log(base)), rtol=1e-13, atol=0)


def test_theta_tiny_exact_values():
    # base 16, d = 8: theta = 16^0, 16^-1/4, 16^-1/2, 16^-3/4 = 1, 1/2, 1/4, 1/8
    assert list(freqs.rope_theta(8, 16.0)) == [1.0, 0.5, 0.25, 0.125]


def _regions(d, base, s, L):
    th = freqs.rope_theta(d, base)
    tp = freqs.yarn_theta(d, base, s, L)
    region = []
    for a, b in zip(th, tp):
        if b == a:
            region.append("unscaled")
        elif b == a / s:
            region.append("pi")
        else:
            region.append("ramp")
    return region


@pytest.mark.parametrize("d,base,s,L", CONFIGS)
def test_yarn_region_boundaries_closed_form(d, base, s, L):
    """r_i = L theta_i / 2pi >= beta  <=>  i <= (d/2) ln(L / (2 pi beta)) / ln(base);
    r_i <= alpha <=> i >= (d/2) ln(L / (2 pi alpha)) / ln(base)."""
    alpha, beta = 1.0, 32.0
    i_hi = (d / 2) * math.log(L / (2 * math.pi * beta)) / math.log(base)
    i_lo = (d / 2) * math.log(L / (2 * math.pi * alpha)) / math.log(base)
    region = _regions(d, base, s, L)
    for i, reg in enumerate(region):
        if i <= i_hi:
            assert reg == "unscaled", (i, reg)
        elif i >= i_lo:
            assert reg == "pi", (i, reg)
        else:
            assert reg == "ramp", (i, reg)


def test_yarn_region_index_ranges_of_the_workloads():
    def spans(region):
        out = {}
        for i, r in enumerate(region):
            lo, hi = out.get(r, (i, i))
            out[r] = (min(lo, i), max(hi, i))
        return out
    assert spans(_regions(64, 10000.0, 4.0, 64)) == {"ramp": (0, 8), "pi": (9, 31)}
    assert spans(_regions(128, 10000.0, 4.0, 4096)) == {
        "unscaled": (0, 20), "ramp": (21, 45), "pi": (46, 63)}
    assert spans(_regions(128, 500000.0, 8.0, 16384)) == {
        "unscaled": (0, 21), "ramp": (22, 38), "pi": (39, 63)}


@pytest.mark.parametrize("d,base,s,L", CONFIGS)
def test_yarn_monotone_and_bracketed(d, base, s, L):
    th = freqs.rope_theta(d, base)
    tp = freqs.yarn_theta(d, base, s, L)
    assert np.all(np.diff(tp) < 0)
    assert np.all(tp <= th) and np.all(tp >= th / s)


def test_gamma_ramp_shape():
    a, b = 1.0, 32.0
    assert freqs.yarn_gamma(a, a, b) == 0.0
    assert freqs.yarn_gamma(b, a, b) == 1.0
    assert freqs.yarn_gamma(0.0, a, b) == 0.0
    assert freqs.yarn_gamma(1e9, a, b) == 1.0
    assert freqs.yarn_gamma((a + b) / 2, a, b) == 0.5
    # continuity at both ends and linearity inside
    eps = 1e-9
    assert freqs.yarn_gamma(a + eps, a, b) == pytest.approx(0.0, abs=1e-9)
    assert freqs.yarn_gamma(b - eps, a, b) == pytest.approx(1.0, abs=1e-9)
    xs = np.linspace(a, b, 17)
    gs = np.array([freqs.yarn_gamma(x, a, b) for x in xs])
    assert np.allclose(np.diff(gs), gs[1] - gs[0], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("d,base,L", [(64, 10000.0, 64), (128, 10000.0, 4096), (128, 500000.0, 16384)])
def test_s1_is_plain_rope_bitwise(d, base, L):
    assert np.array_equal(freqs.yarn_theta(d, base, 1.0, L), freqs.rope_theta(d, base))
    assert freqs.attention_temperature(1.0) == 1.0
    assert np.array_equal(freqs.to_fp32(freqs.yarn_theta(d, base, 1.0, L)),
                          freqs.rope_theta(d, base).astype(np.float32))


@pytest.mark.parametrize("d,base,s", [(64, 10000.0, 4.0), (128, 500000.0, 8.0), (128, 10000.0, 3.0)])
def test_pi_angles_are_positions_over_s(d, base, s):
    th = freqs.rope_theta(d, base)
    tp = freqs.pi_theta(d, base, s)
    for m in (0, 1, 7, 4095, 65537, 131072):
        a = m * tp
        b = (m / s) * th
        assert np.all(np.abs(a - b) <= np.spacing(np.abs(b)) + 0.0)


def test_large_ratio_limit_is_pi_and_small_ratio_limit_is_unscaled():
    # a tiny original length makes every pair turn less than once: pure PI
    d, base, s = 64, 10000.0, 4.0
    assert np.array_equal(freqs.yarn_theta(d, base, s, 1), freqs.rope_theta(d, base) / s)
    # a huge original length makes every pair turn more than beta times: unscaled
    assert np.array_equal(freqs.yarn_theta(d, base, s, 10 ** 12), freqs.rope_theta(d, base))


def test_temperature_values():
    ln4 = 1.3862943611198906
    ln8 = 2.0794415416798357
    assert freqs.attention_temperature(4.0) == pytest.approx(1.0 + 0.1 * ln4, rel=1e-15)
    assert freqs.attention_temperature(8.0) == pytest.approx(1.0 + 0.1 * ln8, rel=1e-15)
    assert freqs.attention_temperature(4.0) == pytest.approx(1.1386294361119891, rel=1e-15)
    assert freqs.attention_temperature(8.0) == pytest.approx(1.2079441541679836, rel=1e-15)
    assert freqs.temperature_for("pi", 8.0) == 1.0
    assert freqs.softmax_scale(64, freqs.attention_temperature(4.0)) == pytest.approx(1.1386294361119891 / 8.0)


def test_ntk_worked_example():
    # printed: base ~ 82,000 for s = 8, d = 128 (exact 82,684.6...)
    b = freqs.ntk_base(128, 10000.0, 8.0)
    assert b == pytest.approx(82684.6, rel=1e-5)
    assert abs(b - 82000.0) / 82000.0 < 0.01
    th = freqs.ntk_theta(128, 10000.0, 8.0)
    assert th[0] == 1.0 and th[-1] < freqs.rope_theta(128, 10000.0)[-1]


@pytest.mark.parametrize("d,base,s,L", CONFIGS + [(128, 10000.0, 8.0, 4096), (64, 10000.0, 2.0, 2048)])
@pytest.mark.parametrize("method", ["plain", "pi", "ntk", "yarn"])
def test_fp32_table_far_from_rounding_midpoints(d, base, s, L, method):
    th = freqs.theta_for(method, d, base, s, L)
    assert np.min(freqs.fp32_midpoint_distance(th)) > 2.0 ** -40


# ---- the interior of the YaRN ramp ------------------------------------------
# The pages print no worked YaRN frequency, so the ramp interior is pinned by
# constructions whose answer the mathematics fixes: an original length L that
# puts a pair's turn count r = L / lambda at a known point of [alpha, beta]
# ("Arch 03 -- Long Context", YaRN slide: linear ramp between the PI-scaled
# and the unscaled frequency; steps table: alpha = 1, beta = 32).

def _ulps(a, b):
    return abs(a - b) / np.spacing(abs(b))


@pytest.mark.parametrize("s", [2.0, 4.0, 8.0])
def test_yarn_ramp_midpoint_is_the_mean_of_pi_and_unscaled(s):
    """r = (alpha + beta) / 2 = 16.5 turns: gamma = 1/2, so theta' is the
    arithmetic mean of theta / s and theta.  Base 16, d 8 gives theta =
    1, 1/2, 1/4, 1/8 exactly; L = 16.5 * 2 pi / theta_i puts pair i there."""
    th = [1.0, 0.5, 0.25, 0.125]
    for i, t in enumerate(th):
        L = 16.5 * 2.0 * math.pi / t
        got = freqs.yarn_theta(8, 16.0, s, L)[i]
        want = (t + t / s) / 2.0
        assert _ulps(got, want) <= 2, (i, got, want)
    # s = 4, pair 0: (1 + 1/4) / 2 = 0.625 written out
    assert _ulps(freqs.yarn_theta(8, 16.0, 4.0, 33.0 * math.pi)[0], 0.625) <= 2


def test_yarn_ramp_quarter_and_three_quarter_points():
    """r = alpha + (beta - alpha)/4 = 8.75 gives gamma = 1/4: theta' =
    theta/s + (theta - theta/s)/4, i.e. 0.4375 for theta = 1, s = 4;
    r = alpha + 3 (beta - alpha)/4 = 24.25 gives gamma = 3/4: 0.8125."""
    assert _ulps(freqs.yarn_theta(8, 16.0, 4.0, 8.75 * 2.0 * math.pi)[0], 0.4375) <= 2
    assert _ulps(freqs.yarn_theta(8, 16.0, 4.0, 24.25 * 2.0 * math.pi)[0], 0.8125) <= 2
    # pair 2 (theta = 1/4) at the quarter point, s = 8: 1/32 + (1/4 - 1/32)/4
    got = freqs.yarn_theta(8, 16.0, 8.0, 8.75 * 2.0 * math.pi / 0.25)[2]
    assert _ulps(got, 0.0859375) <= 2


def test_yarn_ramp_is_linear_in_the_original_length():
    """Inside the ramp r is proportional to L, so theta'(L) is an affine
    function of L: the value at the midpoint of two lengths is the mean of the
    two values, and equal steps in L give equal steps in theta'.  A blend that
    is linear in log(theta) (geometric between theta/s and theta) fails this."""
    d, base, s = 128, 10000.0, 4.0
    lam = 2.0 * math.pi / freqs.rope_theta(d, base)
    i = 30
    # lengths that keep pair i strictly inside (alpha, beta)
    lo, hi = 2.0 * lam[i], 30.0 * lam[i]
    Ls = np.linspace(lo, hi, 9)
    vals = np.array([freqs.yarn_theta(d, base, s, L)[i] for L in Ls])
    steps = np.diff(vals)
    assert np.all(steps > 0)
    assert np.allclose(steps, steps[0], rtol=1e-9, atol=0)
    mid = freqs.yarn_theta(d, base, s, (lo + hi) / 2.0)[i]
    assert mid == pytest.approx((vals[0] + vals[-1]) / 2.0, rel=1e-14)
    # and the line runs from theta/s at r = alpha to theta at r = beta
    th = freqs.rope_theta(d, base)[i]
    slope = steps[0] / (Ls[1] - Ls[0])
    assert vals[0] + slope * (1.0 * lam[i] - lo) == pytest.approx(th / s, rel=1e-12)
    assert vals[0] + slope * (32.0 * lam[i] - lo) == pytest.approx(th, rel=1e-12)


# ---- Dynamic NTK --------------------------------------------------------------
def test_dynamic_ntk_factor_rule():
    # "s equal to the current sequence length / L_train"; no scaling below it
    assert freqs.dynamic_ntk_factor(0, 4096) == 1.0
    assert freqs.dynamic_ntk_factor(4096, 4096) == 1.0
    assert freqs.dynamic_ntk_factor(2000, 4096) == 1.0
    assert freqs.dynamic_ntk_factor(8192, 4096) == 2.0
    assert freqs.dynamic_ntk_factor(32768, 4096) == 8.0
    assert freqs.dynamic_ntk_factor(6144, 4096) == 1.5


def test_dynamic_ntk_below_training_length_is_plain_rope():
    for n in (1, 100, 4096):
        assert np.array_equal(freqs.dynamic_ntk_theta(128, 10000.0, n, 4096),
                              freqs.rope_theta(128, 10000.0))


def test_dynamic_ntk_at_eight_times_the_training_length_is_the_printed_base():
    # the NTK-aware slide's worked case: s = 8, d = 128, base 10000 -> ~82,000
    th = freqs.dynamic_ntk_theta(128, 10000.0, 8 * 4096, 4096)
    b = freqs.ntk_base(128, 10000.0, 8.0)
    assert abs(b - 82000.0) / 82000.0 < 0.01
    # theta_i = b^(-2i/d): i = 32 gives b^(-1/2)
    assert th[32] == pytest.approx(b ** -0.5, rel=1e-14)
    assert th[0] == 1.0


def test_dynamic_ntk_frequencies_fall_as_the_sequence_grows():
    prev = freqs.dynamic_ntk_theta(64, 10000.0, 1024, 1024)
    for n in (1500, 2048, 5000, 65536):
        cur = freqs.dynamic_ntk_theta(64, 10000.0, n, 1024)
        assert cur[0] == 1.0
        assert np.all(cur[1:] < prev[1:])
        prev = cur
