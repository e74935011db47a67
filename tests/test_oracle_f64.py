"""Pins of the binary64 oracle (the float64 path of the method).

Pinned against exact rational arithmetic, closed forms and the identical-
values behaviour that the method page prints for float32 ([VAR] §3) and
lists as not measured for float64 ([VAR] §5, "float64 ([1e307]*3)").
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

U64 = Fraction(1, 2 ** 53)


def exact_var(xs, ddof=0):
    xs = [Fraction(float(v)) for v in xs]
    n = len(xs)
    mu = sum(xs, Fraction(0)) / n
    return sum(((v - mu) ** 2 for v in xs), Fraction(0)) / (n - ddof), mu


def test_two_sum_f64_is_exact():
    rng = np.random.default_rng(31)
    vals = np.concatenate([rng.standard_normal(200) * np.exp2(rng.integers(-1000, 1000, 200)),
                           np.array([1.0, 2.0 ** -60, -1e308, 1e308, 5e-324, 0.0, -0.0])])
    for _ in range(3000):
        a, b = rng.choice(vals, 2)
        s, e = oracle.two_sum_f64(a, b)
        if np.isfinite(s):
            assert Fraction(s) + Fraction(e) == Fraction(float(a)) + Fraction(float(b))
    assert oracle.two_sum_f64(1.0, 2.0 ** -60) == (1.0, 2.0 ** -60)


def test_tree_f64_integer_data_exact_and_bounded():
    rng = np.random.default_rng(32)
    x = rng.integers(-(2 ** 40), 2 ** 40, 100_000).astype(np.float64)
    assert oracle.tree_sum_f64(x) == float(sum(int(v) for v in x))
    for _ in range(10):
        n = int(rng.integers(2, 400))
        y = rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))
        s = sum((Fraction(float(v)) for v in y), Fraction(0))
        a = sum((Fraction(abs(float(v))) for v in y), Fraction(0))
        h = (n - 1).bit_length()
        got = Fraction(float(oracle.tree_sum_f64(y)))
        assert abs(got - s) <= U64 * abs(s) + 2 * h * h * U64 * U64 * a


@pytest.mark.parametrize("n", [3, 1000, 1024, 4096])
def test_arithmetic_progression_closed_form(n):
    # x_i = 1e8 + i: shift, centring and squares are exact in double, so only
    # the final division rounds: var = fl((n^2 - 1) / 12), mean exact
    x = (1e8 + np.arange(n, dtype=np.float64))[None, :]
    v, m = oracle.variance_f64(x, axis=1)
    assert v[0] == float(Fraction(n * n - 1, 12)) and m[0] == 1e8 + (n - 1) / 2


@pytest.mark.parametrize("c", [1.0, 1e10, 1e100, 1e300, 1e307, 1e308])
@pytest.mark.parametrize("ddof", [0, 1])
def test_identical_values_give_zero(c, ddof):
    # the shift makes every y zero ([VAR] §2 step 1), whatever the magnitude
    for n in (3, 1000):
        v, m = oracle.variance_f64(np.full((1, n), c), axis=1, ddof=ddof)
        assert v[0] == 0.0 and m[0] == c


def test_reference_formula_fails_like_float32_at_the_top_of_the_range():
    # [VAR] §3 prints NaN for the two-term reference on [1e38]*3 in float32;
    # the same mechanism in double: m = fl(3e307) * fl(1/3) is one ulp off,
    # d ~ 1e291, d^2 overflows, inf - inf.
    v, _ = oracle.variance_f64(np.full((1, 3), 1e307), axis=1, method=oracle.METHOD_REFERENCE)
    assert np.isnan(v[0])
    v, _ = oracle.variance_f64(np.full((1, 3), 1e307), axis=1)
    assert v[0] == 0.0
    vf, _ = oracle.variance(np.full((1, 3), np.float32(1e38)), axis=1, method=oracle.METHOD_REFERENCE)
    assert np.isnan(vf[0])


def test_page_datasets_in_double_against_exact():
    # D1..D4 cast to double: relative error to the exact rational variance
    # within 4 * 2^-53 on every seventh slice (the float32 bound scaled to
    # double)
    for name, a, ax, _ in W.datasets_d1_d4():
        x = a.astype(np.float64)
        v, m = oracle.variance_f64(x, axis=ax)
        slices = x.T if ax == 0 else x
        for k in range(0, slices.shape[0], 7):
            ev, emu = exact_var(slices[k])
            assert abs(Fraction(float(v[k])) - ev) <= 4 * U64 * ev, (name, k)
            # mean = x0 + m: its error scales with the data, not with the mean
            # (D3's mean is near 0 while its values are near 1)
            assert abs(Fraction(float(m[k])) - emu) <= 2 * U64 * Fraction(float(np.abs(slices[k]).max())), (name, k)
