"""Pins of the double-word-carry tree (the carry variant of the method's node).

The renormalised tree is the method's compensated node followed by TwoSum of
the node's (sum, carry) pair.  Its pins rest on exact arithmetic: exact sums
of the inputs (integer mantissa sums), a first-order error bound derived for
the node, and facts about specific seeded inputs where the renormalised and
the plain carry give different bits.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

U = Fraction(1, 2 ** 24)


def bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def test_c_matches_the_vectorised_form():
    rng = np.random.default_rng(21)
    for n in (1, 2, 3, 5, 64, 1000, 4097, 65536):
        for x in (rng.standard_normal(n).astype(np.float32), W.adversarial_values(n, seed=n),
                  W.sum_cancelling_pairs(n, 0.3, seed=n)):
            assert bits(oracle.tree_sum_dw(x)) == bits(oracle.np_tree_sum_dw(x)), n


def test_zero_padding_leaves_the_bits_unchanged():
    # renormalising a pair that TwoSum produced returns it unchanged
    rng = np.random.default_rng(22)
    for n in (3, 100, 1000):
        for x in (W.adversarial_values(n, seed=n + 1), W.sum_cancelling_pairs(n, 0.3, seed=n)):
            p = 1 << (n - 1).bit_length()
            want = bits(oracle.tree_sum_dw(x))
            for pad in (2 * p, 8 * p):
                assert bits(oracle.tree_sum_dw(x, pad_to=pad)) == want
    x = np.array([np.inf, 1.0, -3.0], np.float32)
    assert oracle.tree_sum_dw(x) == np.inf
    assert np.isnan(oracle.tree_sum_dw(np.array([np.inf, -np.inf, 1.0], np.float32)))


@pytest.mark.parametrize("seed", range(4))
def test_first_order_error_bound(seed):
    # One node adds at most u(|c_l| + |c_r|) + u|c_l + c_r + e| with |c| <=
    # u|s| after renormalisation and |e| <= u|s|: about 3u^2 (|s_l| + |s_r|).
    # Leaves add nothing.  Summed over the h - 1 upper levels, plus the final
    # rounding:  |result - S| <= u|S| + 3.01 u^2 (h - 1) sum|x|.
    rng = np.random.default_rng(seed)
    for _ in range(40):
        n = int(rng.integers(2, 300))
        x = W.adversarial_values(n, seed=int(rng.integers(1 << 30)))
        x = x[np.isfinite(x)]
        if x.size < 2:
            continue
        s = sum((Fraction(float(v)) for v in x), Fraction(0))
        a = sum((Fraction(abs(float(v))) for v in x), Fraction(0))
        h = (x.size - 1).bit_length()
        got = Fraction(float(oracle.tree_sum_dw(x)))
        bound = U * abs(s) + Fraction(301, 100) * U * U * (h - 1) * a + Fraction(2) ** -149
        assert abs(got - s) <= bound


@pytest.mark.parametrize("n,frac,seed", [(1 << 16, 0.3, 1), (1 << 18, 0.2, 2), (1 << 20, 0.1, 1),
                                         (1 << 20, 0.3, 1), (1 << 22, 0.05, 0)])
def test_cancelling_sets_where_the_carries_differ(n, frac, seed):
    # Large values as exactly cancelling pairs (the 10^8 workload's mix at a
    # higher density): the renormalised carry gives the correctly rounded
    # exact sum where the plain carry does not.  A dropped or misplaced
    # renormalisation reproduces the plain tree and fails.
    x = W.sum_cancelling_pairs(n, frac, seed=seed)
    want = oracle.round_f32(oracle.exact_sum(x))
    assert bits(oracle.tree_sum_dw(x)) == bits(want)
    assert bits(oracle.tree_sum(x)) != bits(want)


def test_full_workload_is_correctly_rounded():
    # the 10^8-value workload: plain carry 3735.1025 (3.9e-7), renormalised
    # carry the correctly rounded 3735.104
    x = W.sum_cancelling_pairs()
    want = oracle.round_f32(oracle.exact_sum(x))
    assert bits(oracle.tree_sum_dw(x)) == bits(want)
    assert abs(float(oracle.tree_sum(x)) - float(want)) / abs(float(want)) > 3e-7


def test_integer_data_exact():
    # |x| < 2^24 integers, n < 2^22: partial sums < 2^46, renormalised
    # carries < 2^21, every carry addition exact.
    rng = np.random.default_rng(23)
    x = rng.integers(-(1 << 24) + 1, 1 << 24, 1 << 20).astype(np.float32)
    assert oracle.tree_sum_dw(x) == oracle.round_f32(oracle.exact_sum(x))


def test_variance_with_renormalised_carries_has_the_same_errors():
    # On the method page's datasets the sums of the variance are well
    # conditioned: the renormalised carries change no error (as the page's
    # two-term step changes none).
    for name, a, ax, _ in W.datasets_d1_d4():
        v64 = oracle.var_f64(a, axis=ax)
        e0 = oracle.max_rel_err(oracle.variance(a, axis=ax)[0], v64)
        e9 = oracle.max_rel_err(oracle.variance(a, axis=ax, method=oracle.METHOD_KERNEL_DW)[0], v64)
        assert e0 == e9, name
