"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against a value the pages print, a closed form,
an exact (integer) computation, an invariant of the arithmetic or a brute
force on tiny inputs.  A plausible mistake in the oracle (a dropped carry, a
wrong sign in TwoSum, a wrong pairing, a missing shift, a division where the
reference multiplies by the reciprocal) fails at least one of them; the
comment on each test says which.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from conftest import read_kv, read_table

U = 2.0 ** -24          # unit roundoff of float32
TOL_VAR = 4 * U         # 4 * 2^-24 relative, for well-conditioned data


def F(v) -> Fraction:
    return Fraction(float(v))


def bits(v) -> int:
    return int(np.asarray(v, np.float32).view(np.uint32))


# ---------------------------------------------------------------- TwoSum

def _twosum_pairs(rng, n):
    a = W.adversarial_values(n, int(rng.integers(1 << 30)))
    b = W.adversarial_values(n, int(rng.integers(1 << 30)))
    # near-cancelling and equal-exponent pairs
    c = rng.normal(0, 1, n).astype(np.float32)
    d = (-c * np.float32(1 + 2 ** -20)).astype(np.float32)
    return np.concatenate([a, c]), np.concatenate([b, d])


def test_twosum_error_is_exact():
    # Invariant of the published TwoSum: s + e == a + b exactly, with
    # s = fl(a + b).  A wrong operand or sign in the error formula fails.
    rng = np.random.default_rng(11)
    A, B = _twosum_pairs(rng, 4000)
    for a, b in zip(A, B):
        s, e = oracle.two_sum(a, b)
        if not np.isfinite(s):
            continue
        assert s == np.float32(a + b)
        assert F(s) + F(e) == F(a) + F(b), (a, b, s, e)


def test_twosum_keeps_tiny_addend():
    # The simplification the summation pages warn about (error := 0) would
    # lose the 2^-30: TwoSum(1, 2^-30) must return (1, 2^-30).
    s, e = oracle.two_sum(1.0, 2.0 ** -30)
    assert s == 1.0 and e == np.float32(2.0 ** -30)
    s, e = oracle.two_sum(2.0 ** 24, 1.0)
    assert s == 2.0 ** 24 and e == 1.0


def test_twosum_symmetric_bits():
    # The exact error is unique, so TwoSum(a, b) and TwoSum(b, a) agree bit
    # for bit on finite sums; the GPU relies on this to pair operands in
    # either order inside a tree node.
    rng = np.random.default_rng(12)
    A, B = _twosum_pairs(rng, 3000)
    for a, b in zip(A, B):
        s1, e1 = oracle.two_sum(a, b)
        s2, e2 = oracle.two_sum(b, a)
        if not np.isfinite(s1):
            continue
        assert bits(s1) == bits(s2) and bits(e1) == bits(e2), (a, b)


# ---------------------------------------------------------------- sums

def test_kahan_blog_outputs():
    # "Kahan's Summation Formula": printed naive and Kahan results of 10^6
    # additions of 0.001f, and the theoretical value (F10.5 format).
    g = read_kv("kahan_thousandths.txt")
    x = W.sum_thousandths(int(g["n"]))
    assert "%.5f" % oracle.seq_naive(x) == g["naive"]
    assert "%.5f" % oracle.seq_kahan(x) == g["kahan"]
    assert "%.5f" % oracle.fl32_exact_sum(x) == g["theoretical"]
    # The compensated tree lands on the correctly rounded exact sum.
    assert oracle.tree_sum(x) == oracle.fl32_exact_sum(x)


def test_pm1e16_quickstart():
    # SyclReproSum quick start: +/-1e16 pairs cancel, the ones remain.
    g = read_kv("pm1e16_quickstart.txt")
    x = W.sum_pm1e16(int(g["pairs"]), int(g["ones"]))
    assert oracle.tree_sum(x) == float(g["sum"])
    rng = np.random.default_rng(5)
    for _ in range(10):
        assert oracle.tree_sum(x[rng.permutation(x.size)]) == float(g["sum"])


def test_neumaier_controlled_example():
    # The summation-order page: Neumaier's branch recovers a contribution
    # that the plain Kahan recurrence loses.  [1, big, 1, -big] sums to 2.
    x = np.array([1.0, 1e30, 1.0, -1e30], np.float32)
    assert oracle.seq_kahan(x) == 0.0
    assert oracle.seq_neumaier(x) == 2.0
    assert oracle.tree_sum(x) == 2.0


def test_tree_pairing_hand_worked():
    # Worked by hand for the adjacent-pair topology.  x = [2^24, 1, -2^24, 1]:
    # plain tree: fl(2^24 + 1) = 2^24 (tie to even), fl(-2^24 + 1) exact,
    # root = 1.  A (k, k + P/2) pairing would give (0) + (2) = 2 instead.
    # Compensated tree: the lost 1 is carried up, the result is the exact 2.
    x = np.array([2.0 ** 24, 1.0, -(2.0 ** 24), 1.0], np.float32)
    assert oracle.tree_plain(x) == 1.0
    assert oracle.tree_sum(x) == 2.0
    # 3 values: padding with +0 to 4; [2^24, 1, 1] -> (2^24 + 1) + (1 + 0):
    # plain = 2^24 (the 1 + 1 would survive sequentially), compensated exact.
    y = np.array([2.0 ** 24, 1.0, 1.0], np.float32)
    assert oracle.tree_plain(y) == 2.0 ** 24
    assert oracle.tree_sum(y) == 2.0 ** 24 + 2.0
    # A wrong carry combination (dropping the right child's carry) fails here:
    # both halves lose a 1.
    z = np.array([2.0 ** 24, 1.0, 2.0 ** 24, 1.0], np.float32)
    assert oracle.tree_sum(z) == 2.0 ** 25 + 2.0


def test_compensated_tree_pairing_hand_worked():
    # The compensated tree's result depends on its pairing too.  Worked by
    # hand, x = [7*2^23, 3*2^-25, 2.5, -0.5] (ulp(7*2^23) = 4):
    # adjacent pairs (the reading): fl(7*2^23 + 3*2^-25) = 7*2^23 with
    #   e = 3*2^-25; fl(2.5 - 0.5) = 2, e = 0.  Root: fl(7*2^23 + 2) is a tie,
    #   to even: 7*2^23, e = 2; carry fl(fl(3*2^-25 + 0) + 2) = 2 (3*2^-25 is
    #   under half an ulp of 2); result fl(7*2^23 + 2) = 7*2^23 = 58720256.
    # (k, k + P/2) pairs: fl(7*2^23 + 2.5) = 7*2^23 + 4, e = -1.5;
    #   fl(3*2^-25 - 0.5) exact, e = 0; root fl(7*2^23 + 4 - 0.5 + 3*2^-25) =
    #   7*2^23 + 4, e = -0.5 + 3*2^-25; carry fl(-1.5 + e) = -2 + 2^-23
    #   (the float nearest -2 + 3*2^-25); result fl(7*2^23 + 2 + 2^-23) =
    #   7*2^23 + 4 = 58720260 (above the tie).  The pairings differ in the
    #   last bit.
    x = np.array([7 * 2.0 ** 23, 3 * 2.0 ** -25, 2.5, -0.5], np.float32)
    assert oracle.tree_sum(x) == np.float32(58720256.0)
    assert oracle.tree_sum(x[[0, 2, 1, 3]]) == np.float32(58720260.0)  # the other pairing, by reordering


@pytest.mark.parametrize("n", [2, 3, 5, 7, 8, 13, 64, 100, 1000, 4097])
def test_tree_exact_on_integer_data(n):
    # Big multiples of 2^24 that cancel in pairs, mixed with small integers.
    # Every TwoSum error is then a small integer and every carry addition is
    # exact, so the compensated tree must return the exact sum (brute force
    # over sizes, including non powers of two that exercise the zero
    # padding).  The plain tree loses the small values: the test has teeth
    # against a dropped or mis-combined carry.
    rng = np.random.default_rng(n)
    lost = 0
    for trial in range(20):
        nb = n // 4
        big = rng.integers(1, 9, nb) * rng.choice([-1, 1], nb) * 2.0 ** 24
        small = rng.integers(-7, 8, n - 2 * nb).astype(np.float64)
        x = np.concatenate([big, -big, small]).astype(np.float32)
        x = x[rng.permutation(x.size)]
        ex = oracle.exact_sum(x)
        assert ex == int(small.sum())
        assert F(oracle.tree_sum(x)) == ex
        lost += F(oracle.tree_plain(x)) != ex
    if n >= 8:
        assert lost > 0


def _cascade_bound(x, res):
    """Error bound of the compensated tree: u|S| for the final rounding plus
    4 h^2 u^2 sum|x| for the rounding of the carry additions (h = depth),
    plus a subnormal quantum per value."""
    n = x.size
    h = max(1, math.ceil(math.log2(n))) if n > 1 else 1
    S = oracle.exact_sum(x)
    A = oracle.exact_sum(np.abs(x))
    return abs(F(res) - S), Fraction(U) * abs(S) * Fraction(1 + 4 * U) + Fraction(4 * h * h) * Fraction(U) ** 2 * A \
        + Fraction(n) * Fraction(2) ** -149


@pytest.mark.parametrize("seed", range(6))
def test_tree_error_bound_brute_force(seed):
    # Tiny adversarial inputs (all exponent bands, subnormals, +/-0, massive
    # cancellation): the compensated result obeys the cascaded-sum bound.  A
    # plain tree (dropped carries) violates it on the cancelling cases.
    rng = np.random.default_rng(100 + seed)
    for trial in range(60):
        n = int(rng.integers(1, 17))
        x = W.adversarial_values(n, int(rng.integers(1 << 30)))
        if trial % 2:
            # append the negated big values except one: heavy cancellation
            x = np.concatenate([x, -x[:-1]]).astype(np.float32)
            x = x[rng.permutation(x.size)]
        with np.errstate(over="ignore"):
            if not np.isfinite(np.sum(np.abs(x.astype(np.float64)))):
                continue
        res = oracle.tree_sum(x)
        if not np.isfinite(res):
            continue
        err, bound = _cascade_bound(x, res)
        assert err <= bound, (x, res)


def test_plain_tree_fails_the_bound():
    # Sanity of the previous test: the plain tree does violate the bound on a
    # cancelling case, so the bound test can tell the two apart.
    x = np.array([2.0 ** 30, 1.0, 2.0 ** 30, 1.0, -(2.0 ** 30), -(2.0 ** 30), 0, 0], np.float32)
    err, bound = _cascade_bound(x, oracle.tree_plain(x))
    assert err > bound
    err, bound = _cascade_bound(x, oracle.tree_sum(x))
    assert err <= bound and oracle.tree_sum(x) == 2.0


def test_normal_permutations_same_bits():
    # 2^20 N(0,1) (seed 1) and 8 permutations: well conditioned, so the
    # compensated tree returns the correctly rounded exact sum every time.
    x, perms = W.sum_normal_perms()
    want = oracle.fl32_exact_sum(x)
    assert oracle.tree_sum(x) == want
    for p in perms:
        assert bits(oracle.tree_sum(p)) == bits(want)


@pytest.mark.parametrize("n", [1, 3, 8, 1000, 4096, 12345])
def test_extra_zero_padding_keeps_bits(n):
    # TwoSum(a, +0) = (a, +0) up to the sign of zero and the carries are
    # never -0, so padding further with zeros cannot change the result.  The
    # GPU uses power-of-two tiles larger than 2^ceil(log2 n) and relies on it.
    rng = np.random.default_rng(n)
    P = 1 << max(0, (n - 1).bit_length())
    cases = [W.adversarial_values(n, n), rng.normal(0, 1, n).astype(np.float32),
             np.full(n, -0.0, np.float32), np.where(rng.random(n) < .5, 0.0, -0.0).astype(np.float32)]
    inf = rng.normal(0, 1, n).astype(np.float32)
    inf[n // 2] = np.inf
    cases.append(inf)
    for x in cases:
        r0 = oracle.tree_sum(x)
        for k in (1, 2, 4):
            r = oracle.tree_sum(x, pad_to=P * 2 * k)
            assert bits(r) == bits(r0)
            # the plain tree's root is fl(s + 0), so the sign of an all -0
            # sum does not depend on the padding either
            assert bits(oracle.tree_plain(x, pad_to=P * 2 * k)) == bits(oracle.tree_plain(x))


def test_non_finite_inputs():
    # Inf stays Inf, +Inf and -Inf give NaN, NaN propagates (the root guard).
    x = np.array([1, 2, np.inf, 3], np.float32)
    assert oracle.tree_sum(x) == np.inf
    x = np.array([1, -np.inf, np.inf, 3], np.float32)
    assert np.isnan(oracle.tree_sum(x))
    x = np.array([1, np.nan, 3], np.float32)
    assert np.isnan(oracle.tree_sum(x))
    assert oracle.tree_sum(np.zeros(0, np.float32)) == 0.0
    assert bits(oracle.tree_sum(np.full(8, -0.0, np.float32))) == bits(0.0)
    assert bits(oracle.tree_plain(np.full(8, -0.0, np.float32))) == bits(0.0)
    assert bits(oracle.tree_plain(np.full(1, -0.0, np.float32))) == bits(0.0)


def test_c_and_numpy_forms_agree():
    # Cross-check of the scalar C code against the vectorised numpy levels
    # (two implementations of the same definition; catches indexing bugs in
    # either one).
    rng = np.random.default_rng(3)
    for n in [1, 2, 3, 31, 32, 33, 1000, 4096, 5000]:
        for x in (W.adversarial_values(n, n), rng.normal(1e4, 1, n).astype(np.float32)):
            assert bits(oracle.tree_sum(x)) == bits(oracle.np_tree_sum(x))
            assert bits(oracle.tree_plain(x)) == bits(oracle.np_tree_plain(x))


# ---------------------------------------------------------------- variance

# The two readings of the method page's §2 step 2 (m = sum(y) / n): the
# plain tree of y (the method) and the compensated tree of y.  Every pin of
# the kernel below holds for both; test_local_mean_readings_hand_worked
# tells them apart.
KERNELS = [oracle.METHOD_KERNEL, oracle.METHOD_KERNEL_COMP_SY]


@pytest.mark.parametrize("method", KERNELS)
def test_identical_values_table(method):
    # Method page §3: variance of three identical float32 values.  The naive
    # and two-term columns fix the reading of mean() as tree * fl(1/n); the
    # kernel returns exactly 0 up to 1e38 thanks to the shift.
    for c, naive, ref, ker in read_table("identical_values_table.txt"):
        x = np.full((1, 3), np.float32(float(c)))
        vn = oracle.variance(x, axis=1, method=oracle.METHOD_NAIVE)[0][0]
        vr = oracle.variance(x, axis=1, method=oracle.METHOD_REFERENCE)[0][0]
        vk, mk = oracle.variance(x, axis=1, method=method)
        assert "%g" % vn == naive and "%g" % vr == ref and "%g" % vk[0] == ker
        assert vk[0] == 0.0 and mk[0] == np.float32(float(c))


@pytest.mark.parametrize("method", KERNELS)
@pytest.mark.parametrize("c", [1.0, 1e10, 1e30, 1e38, -3.5e37, 7.5e10])
@pytest.mark.parametrize("ddof", [0, 1])
def test_constant_slices_zero(c, ddof, method):
    # Identical values give exactly 0.0 and mean == c (a missing shift
    # overflows to NaN at 1e38).
    x = W.constant(c)
    v, m = oracle.variance(x, axis=0, ddof=ddof, method=method)
    assert np.all(v == 0.0) and not np.any(np.signbit(v))
    assert np.all(m == np.float32(c))
    v, m = oracle.variance(x.T.copy(), axis=1, ddof=ddof, method=method)
    assert np.all(v == 0.0) and np.all(m == np.float32(c))


def test_local_mean_readings_hand_worked():
    # y = x - x0 = [0, 1, 2^24, 1] (x0 = 0).  The plain pairwise tree gives
    # fl(0 + 1) = 1 and fl(2^24 + 1) = 2^24 (a tie, to even), then
    # fl(1 + 2^24) = 2^24: m = 2^24 / 4 = 4194304.  The compensated tree
    # carries the two lost ones and returns the exact 2^24 + 2: m = 4194304.5.
    # mean = x0 + m shows which sum the local centring took.  Both readings
    # then give the variance of the same four values within the bound (the
    # two-term correction absorbs the error of m); the exact variance is
    # computed with Fractions.
    x = np.array([[0.0, 1.0, 2.0 ** 24, 1.0]], np.float32)
    vp, mp = oracle.variance(x, axis=1, method=oracle.METHOD_KERNEL)
    vc, mc = oracle.variance(x, axis=1, method=oracle.METHOD_KERNEL_COMP_SY)
    assert mp[0] == np.float32(4194304.0)
    assert mc[0] == np.float32(4194304.5)
    vals = [Fraction(0), Fraction(1), Fraction(2 ** 24), Fraction(1)]
    mu = sum(vals) / 4
    exact = sum((v - mu) ** 2 for v in vals) / 4
    for v in (vp[0], vc[0]):
        assert abs(F(v) - exact) <= Fraction(TOL_VAR) * exact


def test_sterbenz_shift_exact_d4():
    # Method page §2 step 1: on D4 every float32 shift equals the exact
    # difference (all 64000 entries).
    g = read_kv("sterbenz_d4.txt")
    d4 = W.datasets_d1_d4()[3][1]
    y = (d4 - d4[0:1, :]).astype(np.float32)
    exact = d4.astype(np.float64) - d4[0:1, :].astype(np.float64)
    assert y.size == int(g["entries"])
    assert np.mean(y.astype(np.float64) == exact) == float(g["equal_fraction"])


@pytest.mark.parametrize("method", KERNELS)
@pytest.mark.parametrize("n", [1000, 1024, 4096, 3])
def test_arithmetic_progression_closed_form(n, method):
    # x_i = 10000 + i: the shift, the centring and the squares are exact, so
    # var = fl32((n^2 - 1)/12) (ddof 0), mean = 10000 + (n-1)/2 exactly;
    # with ddof 1 the exact n(n+1)/12 is within 1 ulp.  A wrong sign in the
    # two-term formula, a wrong centring or a wrong ddof factor fails.  (Every
    # partial sum of y is an integer below 2^24, so the plain and the
    # compensated trees of y agree here.)
    x = (10000.0 + np.arange(n)).astype(np.float32)
    v, m = oracle.variance(x[None, :], axis=1, ddof=0, method=method)
    assert v[0] == oracle.round_f32(Fraction(n * n - 1, 12))
    assert m[0] == np.float32(10000 + (n - 1) / 2)
    v1, _ = oracle.variance(x[:, None], axis=0, ddof=1, method=method)
    exact = Fraction(n * (n + 1), 12)
    ulp = np.spacing(np.float32(float(exact)))
    assert abs(F(v1[0]) - exact) <= F(ulp)


@pytest.mark.parametrize("method", KERNELS)
def test_ddof_edge_cases(method):
    x = np.array([[5.0]], np.float32)
    v, m = oracle.variance(x, axis=1, ddof=0, method=method)
    assert v[0] == 0.0 and m[0] == 5.0
    v, _ = oracle.variance(x, axis=1, ddof=1, method=method)      # 0 * (1/0) = 0 * inf
    assert np.isnan(v[0])
    x = np.array([[1.0, 3.0]], np.float32)
    v, _ = oracle.variance(x, axis=1, ddof=2, method=method)      # 1 * inf
    assert v[0] == np.inf
    v, m = oracle.variance(np.zeros((3, 0), np.float32), axis=1, method=method)
    assert np.all(np.isnan(v)) and np.all(np.isnan(m))


@pytest.mark.parametrize("method", KERNELS)
def test_accuracy_d1_d4_and_no_worse_than_reference(method):
    # Against the float64 variance of the same float32 values: within
    # 4 * 2^-24 and no worse than the two-term reference on these
    # well-conditioned datasets; same order of magnitude as the page's tables.
    table = {r[0]: [float(v) for v in r[1:]] for r in read_table("accuracy_tables.txt")}
    for name, a, ax, _ in W.datasets_d1_d4():
        v64 = oracle.var_f64(a, axis=ax)
        ek = oracle.max_rel_err(oracle.variance(a, axis=ax, method=method)[0], v64)
        er = oracle.max_rel_err(oracle.variance(a, axis=ax, method=oracle.METHOD_REFERENCE)[0], v64)
        en = oracle.max_rel_err(oracle.variance(a, axis=ax, method=oracle.METHOD_NAIVE)[0], v64)
        naive_p, ref_p, ker_p = table[name][0], table[name][1], table[name][2]
        assert ek <= TOL_VAR, (name, ek)
        assert ek <= er, (name, ek, er)
        for ours, page in ((en, naive_p), (er, ref_p), (ek, ker_p)):
            assert page / 3 <= ours <= page * 3, (name, ours, page)


def test_naive_loses_digits_on_large_offset():
    # The problem statement of the method page §1: with a large offset the
    # naive formula's error is of order eps*|mean|/std, far above the kernel.
    d4 = W.datasets_d1_d4()[3][1]
    v64 = oracle.var_f64(d4, axis=0)
    assert oracle.max_rel_err(oracle.variance(d4, axis=0, method=oracle.METHOD_NAIVE)[0], v64) > 1e-3


def test_complex_check():
    # Method page §2/§3: complex data as re + im variances; printed value.
    g = read_kv("complex_check.txt")
    z = np.array([complex(s.replace(" ", "")) for s in g["values"].split(",")], np.complex64)
    v, _ = oracle.variance_complex(z[None, :], axis=1)
    assert v[0] == float(g["variance"])
    zc = np.full((1, int(g["identical_count"])), complex(g["identical"]), np.complex64)
    v, _ = oracle.variance_complex(zc, axis=1)
    assert v[0] == float(g["identical_variance"])


@pytest.mark.parametrize("method", KERNELS)
def test_kernel_steps_numpy_cross_check(method):
    # The variance kernel rebuilt from the numpy tree levels, step by step,
    # agrees bit for bit with the C oracle (cross-check, not a pin).
    rng = np.random.default_rng(9)
    for rows, cols in [(7, 1000), (5, 4096), (3, 33), (2, 1)]:
        x = rng.normal(1e4, 1, (rows, cols)).astype(np.float32)
        v, m = oracle.variance(x, axis=1, method=method)
        y = (x - x[:, :1]).astype(np.float32)
        sy = oracle.np_tree_plain(y) if method == oracle.METHOD_KERNEL else oracle.np_tree_sum(y)
        mm = (sy / np.float32(cols)).astype(np.float32)
        d = (y - mm[:, None]).astype(np.float32)
        q = (d * d).astype(np.float32)
        s1, s2 = oracle.np_tree_sum(d), oracle.np_tree_sum(q)
        a = (s2 / np.float32(cols)).astype(np.float32)
        b = (s1 / np.float32(cols)).astype(np.float32)
        vv = np.maximum((a - (b * b).astype(np.float32)).astype(np.float32), np.float32(0))
        assert np.array_equal(vv.view(np.uint32), v.view(np.uint32))
        assert np.array_equal((x[:, 0] + mm).astype(np.float32), m)


# ---------------------------------------------------------------- ablation variants

ABLATION = [oracle.METHOD_SHIFT_PLAIN_NO2T, oracle.METHOD_SHIFT_PLAIN_2T, oracle.METHOD_NOSHIFT_COMP_2T,
            oracle.METHOD_SHIFT_COMP_NO2T, oracle.METHOD_SHIFT_KAHAN_NO2T]
SHIFTED = [oracle.METHOD_KERNEL, oracle.METHOD_SHIFT_PLAIN_NO2T, oracle.METHOD_SHIFT_PLAIN_2T,
           oracle.METHOD_SHIFT_COMP_NO2T, oracle.METHOD_SHIFT_KAHAN_NO2T]


def test_ablation_identical_1e38_column():
    # Method page §4: every variant with the shift returns exactly 0 on
    # [1e38]*3 in every mode; the reference formula returns NaN.
    x = np.full((1, 3), np.float32(1e38))
    for m in SHIFTED:
        assert oracle.variance(x, axis=1, method=m)[0][0] == 0.0, m
    assert np.isnan(oracle.variance(x, axis=1, method=oracle.METHOD_REFERENCE)[0][0])


def test_ablation_rows_keep_the_plain_local_mean():
    # Each ablation row changes one step of the kernel; none of them names the
    # local centring's sum, so every shifted row keeps the kernel's plain tree
    # of y: on y = [0, 1, 2^24, 1] its mean is 2^24 / 4 (see
    # test_local_mean_readings_hand_worked), not the compensated 4194304.5.
    x = np.array([[0.0, 1.0, 2.0 ** 24, 1.0]], np.float32)
    for m in SHIFTED + [oracle.METHOD_KERNEL_DW]:
        assert oracle.variance(x, axis=1, method=m)[1][0] == np.float32(4194304.0), m
    # without the shift, y = x: the same plain tree of the same values
    assert oracle.variance(x, axis=1, method=oracle.METHOD_NOSHIFT_COMP_2T)[1][0] == np.float32(4194304.0)


def test_ablation_two_term_does_not_change_the_errors():
    # Method page §4: the kernel and the variant without the two-term
    # correction have the same errors on every dataset.
    for name, a, ax, _ in W.datasets_d1_d4():
        v64 = oracle.var_f64(a, axis=ax)
        ek = oracle.max_rel_err(oracle.variance(a, axis=ax)[0], v64)
        e7 = oracle.max_rel_err(oracle.variance(a, axis=ax, method=oracle.METHOD_SHIFT_COMP_NO2T)[0], v64)
        assert ek == e7, name


@pytest.mark.parametrize("n", [3, 1000, 1024])
def test_ablation_closed_form(n):
    # x_i = 10000 + i: every sum stays an exact integer (or half-integer)
    # below 2^24, so every variant returns fl((n^2-1)/12) and the exact mean.
    # The reference formula multiplies by fl(1/n), exact only for n = 2^k.
    x = (10000.0 + np.arange(n)).astype(np.float32)[None, :]
    want = oracle.round_f32(Fraction(n * n - 1, 12))
    extra = [oracle.METHOD_REFERENCE] if n & (n - 1) == 0 else []
    for m in ABLATION + [oracle.METHOD_KERNEL] + extra:
        v, mu = oracle.variance(x, axis=1, method=m)
        assert v[0] == want, m
        assert mu[0] == np.float32(10000 + (n - 1) / 2), m


def test_ablation_kahan_scan_is_the_blog_recurrence():
    # The Kahan-scan variant sums with the blog's loop: its mean of 10^6
    # copies of 0.001f shifted by the first value is exactly 0 (all y = 0),
    # and on a slice whose sums reduce to the blog's fixture it matches it.
    x = np.full((1, 1_000_000), np.float32(0.001))
    v, mu = oracle.variance(x, axis=1, method=oracle.METHOD_SHIFT_KAHAN_NO2T)
    assert v[0] == 0.0 and mu[0] == np.float32(0.001)
    # unshifted sum check through the d^2 tree is not available; the loop
    # itself is pinned by test_kahan_blog_outputs.


def test_threaded_oracle_splits_exactly():
    # The all-cores timing of the oracle cuts the sum into aligned subtrees
    # and the variance into blocks of slices; both must give the same bits.
    import workloads as W

    for n in (1, 2, 3, 5, 1000, 4097, 300_001):
        y = W.adversarial_values(n, seed=n)
        want = np.float32(oracle.tree_sum(y)).view(np.uint32)
        for t in (1, 2, 3, 8):
            assert np.float32(oracle.tree_sum_threads(y, t)).view(np.uint32) == want, (n, t)
    a = W.c4_matrix()[:300]
    v1, m1 = oracle.variance(a, axis=1)
    v8, m8 = oracle.variance_threads(a, 1, 8)
    assert np.array_equal(v1.view(np.uint32), v8.view(np.uint32)) and np.array_equal(m1.view(np.uint32), m8.view(np.uint32))
    b = np.ascontiguousarray(a[:, :200])
    v1, m1 = oracle.variance(b, axis=0)
    v8, m8 = oracle.variance_threads(b, 0, 8)
    assert np.array_equal(v1.view(np.uint32), v8.view(np.uint32)) and np.array_equal(m1.view(np.uint32), m8.view(np.uint32))
