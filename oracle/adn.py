"""Oracle for the Ahrens-Demmel-Nguyen (ADN) binned reproducible float32 sum.

TEST INFRASTRUCTURE ONLY (see the package docstring): only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg use it.

Source: [ADN] "SyclReproSum" README, sections "How It Works", "Accumulator
capacity" and "Template Parameters".  The page describes the method:

  * every value is deposited into K folds, K primary values aligned to a fixed
    global grid of exponent bins of width W = 13 bits (float), plus K carry
    counters; the deposit is a few plain float additions, with a sticky bit
    that makes the rounding into a bin independent of the order;
  * after every 2^(24 - W - 2) = 512 deposits each primary's drift moves into
    its carry counter;
  * accumulators merge exactly, bin by bin; the total is converted back to a
    float with a running double value;
  * NaN, or +Inf together with -Inf, gives the quiet NaN 0x7fc00000;
  * at most 4,294,966,784 values (float).

Where the page is silent this oracle takes the readings below (the GPU path
takes the same ones):

  R1 grid: bins b = 0..21; bin b holds the weights 2^(13b - 146) ..
     2^(13b - 134) ("grid" 2^(13b - 146) is its unit).  The finest unit,
     2^-146, keeps a float's lowest bit (>= 2^-149) below half a unit, which
     the sticky bit needs.
  R2 index: the folds are the bins top, top-1, .., top-K+1, where top is the
     smallest bin with |x| < 2^(13 top - 134) for every finite x summed (one
     bit of headroom), and at least K-1.
  R3 deposit: each fold rounds the remainder to its unit, to nearest with
     ties away from zero (what adding x with its lowest bit set to 1 does);
     the rest passes on to the next fold; the last fold's rounding is the
     only loss.
  R4 renormalisation keeps each primary in [1.25, 1.75) * 2^q (q = its
     binade) by moving quarters 2^(q-2) into the carry count.
  R5 conversion: each fold's value (primary minus its base, plus carry times
     quarter) is exact in double; the result is float(Y) with Y the running
     double sum of the fold values from the coarsest fold down.
  R6 an empty sum and a sum of zeros give +0.

Two formulations are here:

  * :func:`adn_sum`, the closed form implied by R1-R5: the exact sum, per
    fold, of every value's cascade of roundings at the final index, then R5.
    Vectorised numpy (float64 is exact for every step) with integer sums.
  * :func:`adn_deposit_sum`, the algorithm's own steps in float32: index
    raise, sticky-bit deposits, renormalisation every 512 deposits, exact
    merges of partial accumulators and the double conversion.  Slow (pure
    Python); for small inputs.  Agreement of the two, in any order and any
    split, is tested.
"""
from __future__ import annotations

import math

import numpy as np

W = 13                  # bin width for float ("Template Parameters")
MANT = 24               # float significand bits
NBINS = 22              # bins 0..21 cover 2^-146 .. 2^140
GRID0 = -146            # log2 of bin 0's unit (reading R1)
RENORM_EVERY = 1 << (MANT - W - 2)        # 512 deposits ("How It Works", step 2)
MAX_COUNT = 4_294_966_784                 # "Accumulator capacity", float
MAX_FOLD = 21                             # "Template Parameters", float
CANONICAL_NAN_BITS = 0x7FC00000           # "How It Works", Inf/NaN paragraph

# Bins whose primaries (1.5 * 2^q) would overflow a float are stored scaled
# by 2^-SCALE_SHIFT in the float32 formulation.
SCALE_FROM = 20
SCALE_SHIFT = 40


def unit_exp(b: int) -> int:
    """log2 of bin b's unit (its lowest weight)."""
    return GRID0 + W * b


def primary_exp(b: int) -> int:
    """Binade q of bin b's primary: ulp(1.5 * 2^q) equals the bin's unit."""
    return unit_exp(b) + MANT - 1


def bin_of(absx: float) -> int:
    """Smallest bin b with absx < 2^(13b - 134), for finite absx > 0 (R2)."""
    e = math.frexp(absx)[1] - 1          # absx in [2^e, 2^(e+1))
    return max(0, -(-(e + 135) // W))


def top_bin(absmax: float, fold: int) -> int:
    return max(fold - 1, bin_of(absmax) if absmax > 0 else 0)


def _check(fold: int, n: int) -> None:
    if not 2 <= fold <= MAX_FOLD:
        raise ValueError(f"fold {fold} outside 2..{MAX_FOLD}")
    if n > MAX_COUNT:
        raise ValueError(f"{n} values exceed the accumulator capacity {MAX_COUNT}")


def _special(x: np.ndarray):
    """Result forced by NaN / Inf inputs, or None ("How It Works")."""
    nan = bool(np.isnan(x).any())
    pinf = bool(np.isposinf(x).any())
    ninf = bool(np.isneginf(x).any())
    if nan or (pinf and ninf):
        return np.array([CANONICAL_NAN_BITS], np.uint32).view(np.float32)[0]
    if pinf:
        return np.float32(np.inf)
    if ninf:
        return np.float32(-np.inf)
    return None


def fold_values(x, fold: int = 3, chunk: int = 1 << 22):
    """Closed form (R1-R3): (top, [exact value of fold k as a Python int times 2^unit_exp])."""
    x = np.asarray(x, np.float32).ravel()
    _check(fold, x.size)
    fin = x[np.isfinite(x)]
    absmax = float(np.max(np.abs(fin))) if fin.size else 0.0
    top = top_bin(absmax, fold)
    ints = [0] * fold
    for i0 in range(0, fin.size, chunk):
        r = fin[i0:i0 + chunk].astype(np.float64)
        for k in range(fold):
            g = 2.0 ** unit_exp(top - k)
            y = r / g                                    # exact (power-of-two scaling)
            a = np.sign(y) * np.floor(np.abs(y) + 0.5)  # nearest, ties away from zero
            r = r - a * g                                # exact remainder
            ints[k] += int(a.astype(np.int64).sum())
    return top, ints


def convert(top: int, vals) -> np.float32:
    """R5: running double sum of the fold values, coarsest first, rounded to float."""
    y = 0.0
    for k, v in enumerate(vals):
        y += float(v)
    with np.errstate(over="ignore"):
        return np.float32(y)


def adn_sum(x, fold: int = 3) -> np.float32:
    """ADN binned sum of float32 values, closed form (R1-R6)."""
    x = np.asarray(x, np.float32).ravel()
    _check(fold, x.size)
    sp = _special(x)
    if sp is not None:
        return sp
    top, ints = fold_values(x, fold)
    vals = [math.ldexp(float(a), unit_exp(top - k)) for k, a in enumerate(ints)]
    return convert(top, vals)


# ---------------------------------------------------------------- float32 steps

_f32 = np.float32


def _sticky(v: np.float32) -> np.float32:
    return np.array([v], np.float32).view(np.uint32).__or__(np.uint32(1)).view(np.float32)[0]


def _scale_exp(b: int) -> int:
    return -SCALE_SHIFT if b >= SCALE_FROM else 0


def _base(b: int) -> np.float32:
    return _f32(math.ldexp(1.5, primary_exp(b) + _scale_exp(b)))


def _quarter(b: int) -> np.float32:
    return _f32(math.ldexp(1.0, primary_exp(b) - 2 + _scale_exp(b)))


class Accumulator:
    """K-fold binned accumulator in float32, as the page's steps describe."""

    def __init__(self, fold: int = 3):
        _check(fold, 0)
        self.fold = fold
        self.top = fold - 1
        self.p = [_base(self.top - k) for k in range(fold)]
        self.c = [_f32(0.0)] * fold
        self.count = 0
        self.nan = self.pinf = self.ninf = False

    def raise_to(self, top: int) -> None:
        d = top - self.top
        if d <= 0:
            return
        p, c = self.p, self.c
        self.p = [p[k - d] if k - d >= 0 else _base(top - k) for k in range(self.fold)]
        self.c = [c[k - d] if k - d >= 0 else _f32(0.0) for k in range(self.fold)]
        self.top = top

    def renorm(self) -> None:
        with np.errstate(all="ignore"):
            for k in range(self.fold):
                b = self.top - k
                base, q4 = _base(b), _quarter(b)
                if self.p[k] >= _f32(base + q4):
                    self.p[k] = _f32(self.p[k] - q4)
                    self.c[k] = _f32(self.c[k] + _f32(1.0))
                elif self.p[k] < _f32(base - q4):
                    self.p[k] = _f32(self.p[k] + q4)
                    self.c[k] = _f32(self.c[k] - _f32(1.0))

    def deposit(self, x) -> None:
        x = _f32(x)
        if np.isnan(x):
            self.nan = True
            return
        if np.isinf(x):
            if x > 0:
                self.pinf = True
            else:
                self.ninf = True
            return
        if x != 0:
            self.raise_to(bin_of(float(abs(x))))
        if self.count == RENORM_EVERY:
            self.renorm()
            self.count = 0
        self.count += 1
        r = x
        with np.errstate(all="ignore"):
            for k in range(self.fold):
                b = self.top - k
                se = _scale_exp(b)
                rs = _f32(r * _f32(math.ldexp(1.0, se))) if se else r
                xs = _sticky(rs)
                if k < self.fold - 1:
                    s = _f32(self.p[k] + xs)
                    d = _f32(self.p[k] - s)          # minus the part this fold took
                    self.p[k] = s
                    if se == 0:
                        r = _f32(r + d)
                    elif d != 0:
                        r = _f32(_f32(rs + d) * _f32(math.ldexp(1.0, -se)))
                else:
                    self.p[k] = _f32(self.p[k] + xs)

    def merge(self, other: "Accumulator") -> None:
        assert other.fold == self.fold
        top = max(self.top, other.top)
        self.raise_to(top)
        other.raise_to(top)
        self.renorm()
        other.renorm()
        for k in range(self.fold):
            base = _base(top - k)
            self.p[k] = _f32(self.p[k] + _f32(other.p[k] - base))
            self.c[k] = _f32(self.c[k] + other.c[k])
        self.renorm()
        self.count = 0
        self.nan |= other.nan
        self.pinf |= other.pinf
        self.ninf |= other.ninf

    def fold_values(self):
        """Exact value of each fold (double): (p - base) + c * quarter, unscaled."""
        out = []
        for k in range(self.fold):
            b = self.top - k
            v = float(_f32(self.p[k] - _base(b))) + float(self.c[k]) * float(_quarter(b))
            out.append(math.ldexp(v, -_scale_exp(b)))
        return out

    def result(self) -> np.float32:
        if self.nan or (self.pinf and self.ninf):
            return np.array([CANONICAL_NAN_BITS], np.uint32).view(np.float32)[0]
        if self.pinf:
            return np.float32(np.inf)
        if self.ninf:
            return np.float32(-np.inf)
        return convert(self.top, self.fold_values())


def adn_deposit_sum(x, fold: int = 3, parts: int = 1, seed: int = 0) -> np.float32:
    """The float32 steps: deposit in the given order into ``parts`` accumulators
    (contiguous pieces, cut at seeded random points), then merge them in a
    seeded random order."""
    x = np.asarray(x, np.float32).ravel()
    _check(fold, x.size)
    rng = np.random.default_rng(seed)
    cuts = sorted(rng.choice(np.arange(1, max(x.size, 2)), size=min(parts - 1, max(x.size - 1, 0)),
                             replace=False).tolist()) if parts > 1 and x.size > 1 else []
    pieces = np.split(x, cuts)
    accs = []
    for piece in pieces:
        a = Accumulator(fold)
        for v in piece:
            a.deposit(v)
        accs.append(a)
    order = rng.permutation(len(accs))
    total = accs[order[0]]
    for i in order[1:]:
        total.merge(accs[i])
    return total.result()
