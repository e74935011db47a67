"""Pins of the ADN binned-sum oracle ([ADN] "SyclReproSum" README).

The oracle holds two formulations (the closed form and the float32 steps);
besides their agreement, each pin below rests on something other than the
oracle itself: exact integer arithmetic, the page's printed error term and
capacity, its special-value rules and its quick-start example.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import adn


def exact(x):
    return sum((Fraction(float(v)) for v in np.asarray(x, np.float32).ravel()), Fraction(0))


def bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def datasets(seed):
    return W.sum_mixed_sets(seed)


@pytest.mark.parametrize("fold", [2, 3, 4, 6, 13, 21])
def test_closed_form_equals_the_float32_steps(fold):
    # The float32 deposit algorithm (sticky bit, renormalisation, merges) and
    # the closed form of its result must agree bit for bit, in any order and
    # any split into partial accumulators.
    for seed in range(2):
        for name, x in datasets(seed):
            want = adn.adn_sum(x, fold)
            rng = np.random.default_rng(seed + 10)
            for parts, perm in ((1, False), (1, True), (5, True), (17, False)):
                xx = rng.permutation(x) if perm else x
                got = adn.adn_deposit_sum(xx, fold, parts=parts, seed=seed)
                assert bits(got) == bits(want), (name, fold, parts, perm, got, want)


def test_renormalisation_interval_and_capacity_constants():
    # "How It Works" step 2: every 2^(mantissa_bits - W - 2) deposits; with a
    # float carry counter exact below 2^23 per quarter this gives the printed
    # capacity (2^23 - 1) * 2^9.
    assert adn.RENORM_EVERY == 2 ** (24 - 13 - 2) == 512
    assert adn.MAX_COUNT == (2 ** 23 - 1) * 2 ** 9 == 4_294_966_784
    # a long run of deposits of the largest value a fold accepts stays exact
    a = adn.Accumulator(3)
    v = np.float32(np.nextafter(np.float32(2.0 ** 9), np.float32(0)))  # just below 2^(13*11-134)
    for _ in range(3 * 512 + 7):
        a.deposit(v)
    assert a.result() == oracle.round_f32(Fraction(float(v)) * (3 * 512 + 7))


def test_integer_data_is_exact():
    # Integers of magnitude <= 2^20: the last fold's unit is <= 1, so every
    # deposit is exact and the result is the correctly rounded exact sum.
    rng = np.random.default_rng(5)
    x = rng.integers(-(2 ** 20), 2 ** 20, 20000).astype(np.float32)
    s = exact(x)
    assert adn.adn_sum(x, 3) == oracle.round_f32(s)
    assert adn.adn_deposit_sum(x[:3000], 3, parts=4) == oracle.round_f32(exact(x[:3000]))


def test_quick_start_in_float():
    # [ADN] Quick Start: 5 pairs of +/-1e16 then 10000 ones sum to 10000.  In
    # float the 1e16 pairs set the top bin to the one holding 2^53; three
    # folds reach down to units of 2^23, so the ones round away (error term
    # of the "Template Parameters" table: N * 2^-26 * max|x| = 1.5e12); five
    # folds reach 2^-3 and give 10000 exactly.
    x = np.array([1e16, -1e16] * 5 + [1.0] * 10000, np.float32)
    assert adn.adn_sum(x, 3) == 0.0
    assert adn.adn_sum(x, 5) == 10000.0
    assert adn.adn_sum(x, 6) == 10000.0
    assert abs(float(adn.adn_sum(x, 3)) - 10000) <= x.size * 2.0 ** -26 * 1e16
    assert adn.adn_deposit_sum(x, 5, parts=3) == 10000.0


@pytest.mark.parametrize("fold", [2, 3, 4])
def test_error_within_the_printed_term(fold):
    # "Template Parameters": dominant binned error ~ N * 2^(-W(K-1)) * max|x|
    # (2^-26 at K = 3), absolute; plus the final rounding to float.
    rng = np.random.default_rng(7 + fold)
    for _ in range(5):
        n = 5000
        x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
        s = exact(x)
        got = Fraction(float(adn.adn_sum(x, fold)))
        bound = n * Fraction(2) ** (-13 * (fold - 1)) * Fraction(float(np.max(np.abs(x))))
        assert abs(got - s) <= bound + abs(s) * Fraction(2) ** -23


def test_specials_follow_the_page():
    # "How It Works": any NaN, or +Inf with -Inf, gives the quiet NaN
    # 0x7fc00000 whatever the payloads; a single-signed Inf stays.
    x = np.ones(10, np.float32)
    payload = np.array([0x7FA12345], np.uint32).view(np.float32)[0]   # a signalling NaN
    negnan = np.array([0xFFC00001], np.uint32).view(np.float32)[0]
    for extra in ([payload], [negnan], [np.inf, -np.inf], [np.nan, np.inf]):
        y = np.concatenate([x, np.array(extra, np.float32)])
        assert bits(adn.adn_sum(y)) == 0x7FC00000
        assert bits(adn.adn_deposit_sum(y, parts=2)) == 0x7FC00000
    assert adn.adn_sum(np.concatenate([x, [np.inf]]).astype(np.float32)) == np.inf
    assert adn.adn_sum(np.concatenate([x, [-np.inf]]).astype(np.float32)) == -np.inf
    assert bits(adn.adn_sum(np.zeros(0, np.float32))) == 0
    assert bits(adn.adn_sum(np.full(7, -0.0, np.float32))) == 0


def test_subnormal_rounding_and_absorption():
    # The finest unit is 2^-146: subnormal multiples of it are exact; smaller
    # parts round to nearest, ties away from zero ("subnormals deposit into
    # the bottom bins; values below the absorption threshold round away").
    t = np.float32(2.0 ** -149)
    assert adn.adn_sum(np.array([8 * t] * 5, np.float32)) == np.float32(40 * 2.0 ** -149)
    assert adn.adn_sum(np.array([3 * t] * 5, np.float32)) == 0.0         # 3/8 of a unit each
    assert adn.adn_sum(np.array([4 * t] * 5, np.float32)) == np.float32(40 * 2.0 ** -149)  # ties away
    assert adn.adn_sum(np.array([-4 * t] * 5, np.float32)) == np.float32(-40 * 2.0 ** -149)


def test_overflowing_total_and_largest_values():
    big = np.float32(3.0e38)
    assert adn.adn_sum(np.array([big, big], np.float32)) == np.inf
    assert adn.adn_sum(np.array([big, big, -big], np.float32)) == big
    x = np.array([big, -big, 1.5e30, 2.0 ** 113], np.float32)
    assert adn.adn_sum(x) == adn.adn_deposit_sum(x, parts=2)


def test_index_reading():
    # R2: top bin = smallest b with |x| < 2^(13b - 134), at least K-1.
    assert adn.bin_of(1.0) == math.ceil(135 / 13)
    assert adn.bin_of(float(np.float32(3.4e38))) == 21
    assert adn.bin_of(2.0 ** 113) == 20 and adn.bin_of(2.0 ** 113 * 0.75) == 19
    assert adn.bin_of(2.0 ** -149) == 0
    for b in range(22):
        hi = 2.0 ** (13 * b - 134)
        assert adn.bin_of(np.nextafter(hi, 0)) == b or b == 0
        assert adn.bin_of(hi) == b + 1 or b == 21
