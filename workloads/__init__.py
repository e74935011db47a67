"""Seeded synthetic inputs, shared by the tests, the smoke check and the bench.

This module only draws numbers: it holds none of the method's arithmetic
(no sum, no shift, no variance).  Both the oracle side and the GPU side take
their inputs from here.

Workloads (shapes and distributions of the method page, "Variance in float32
with a first-element shift, a local centring and a compensated tree sum" §3,
and of the fixtures on the summation pages):

  D1..D4  the four datasets of the method page's §3 tables, drawn in page
          order from ``numpy.random.default_rng(0)`` as float64 normals and
          cast to float32: D1 [1000,64] N(1000, 0.01) (axis 0), D2 [64,1000]
          N(10000, 1) (axis 1), D3 [1000,64] N(0, 1) (axis 0), D4 [1000,64]
          N(1e6, 1) (axis 0).
  const   [1000,64] filled with one constant c (axis 0).
  C4      [4096,4096] N(1e4, 1), seed 2, axis 1: the timing shape of §3.
  sums    (a) 10^6 copies of 0.001f, (b) 5 pairs +1e16/-1e16 then 10 000
          ones, (c) 2^20 N(0,1) from seed 1 and 8 permutations from the same
          generator, (d) 10^8 values: 99% N(0,1), 1% large values +/-U(1e6,1e8)
          placed as exactly cancelling pairs at random positions, seed 3.
"""
from __future__ import annotations

import numpy as np


def datasets_d1_d4():
    """The method page's D1..D4, drawn in page order from one generator.

    Returns a list of (name, array float32, axis, label).
    """
    rng = np.random.default_rng(0)
    d1 = rng.normal(1000.0, 0.01, (1000, 64)).astype(np.float32)
    d2 = rng.normal(10000.0, 1.0, (64, 1000)).astype(np.float32)
    d3 = rng.normal(0.0, 1.0, (1000, 64)).astype(np.float32)
    d4 = rng.normal(1e6, 1.0, (1000, 64)).astype(np.float32)
    return [
        ("D1", d1, 0, "[1000,64] axis 0 N(1000, 0.01)"),
        ("D2", d2, 1, "[64,1000] axis 1 N(10000, 1)"),
        ("D3", d3, 0, "[1000,64] axis 0 N(0, 1)"),
        ("D4", d4, 0, "[1000,64] axis 0 N(1e6, 1)"),
    ]


def constant(c: float, shape=(1000, 64)) -> np.ndarray:
    return np.full(shape, np.float32(c), dtype=np.float32)


def c4_matrix(seed: int = 2, shape=(4096, 4096)) -> np.ndarray:
    """[4096,4096] float32 N(1e4, 1) from default_rng(2)."""
    rng = np.random.default_rng(seed)
    return rng.normal(1e4, 1.0, shape).astype(np.float32)


def sum_thousandths(n: int = 1_000_000) -> np.ndarray:
    return np.full(n, np.float32(0.001), dtype=np.float32)


def sum_pm1e16(pairs: int = 5, ones: int = 10_000) -> np.ndarray:
    v = [1e16, -1e16] * pairs + [1.0] * ones
    return np.asarray(v, dtype=np.float32)


def sum_normal_perms(n: int = 1 << 20, perms: int = 8, seed: int = 1):
    """2^20 N(0,1) float32 from default_rng(1), then `perms` permutations
    drawn from the same generator.  Returns (x, [x[p] for p in perms])."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    out = [x[rng.permutation(n)] for _ in range(perms)]
    return x, out


def sum_cancelling_pairs(n: int = 100_000_000, frac_large: float = 0.01, seed: int = 3) -> np.ndarray:
    """99% N(0,1), 1% large values +/-U(1e6, 1e8) as exactly cancelling pairs
    at random positions (the 1e8-element workload; smaller n keeps the mix)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    k = int(round(n * frac_large)) // 2 * 2
    if k:
        pos = rng.choice(n, k, replace=False)
        v = rng.uniform(1e6, 1e8, k // 2).astype(np.float32)
        x[pos[: k // 2]] = v
        x[pos[k // 2:]] = -v
    return x


def random_matrix(rows: int, cols: int, seed: int, loc: float = 0.0, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(loc, scale, (rows, cols)).astype(np.float32)


def adversarial_values(n: int, seed: int) -> np.ndarray:
    """Mixed magnitudes and signs (huge/tiny/subnormal/zero/negative zero):
    every exponent band of float32 appears."""
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-140, 100, n)
    sign = rng.choice([-1.0, 1.0], n)
    v = (sign * mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    kinds = rng.integers(0, 10, n)
    v[kinds == 0] = 0.0
    v[kinds == 1] = -0.0
    v[kinds == 2] = (sign[kinds == 2] * rng.uniform(1, 2, (kinds == 2).sum()) * 2.0 ** -140).astype(np.float32)
    return v


def sum_mixed_sets(seed: int, scale: int = 1):
    """Named float32 vectors for order-independent sums: normal, wide exponent
    range, cancelling pairs, subnormal, huge (up to 3.3e38, including values
    at or above 2^113) and values on the halves of power-of-two units (ties).
    ``scale`` multiplies every length."""
    rng = np.random.default_rng(seed)
    s = scale
    yield "normal", rng.standard_normal(700 * s).astype(np.float32)
    yield "wide", (rng.standard_normal(600 * s) * np.exp2(rng.integers(-60, 60, 600 * s))).astype(np.float32)
    v = rng.uniform(1e6, 1e8, 200 * s).astype(np.float32)
    yield "cancel", np.concatenate([v, -v, rng.standard_normal(300 * s).astype(np.float32)])
    yield "subnormal", (rng.integers(-2000, 2000, 400 * s) * np.float32(2.0 ** -149)).astype(np.float32)
    yield "huge", (rng.standard_normal(300 * s) * np.float32(3e37)).astype(np.float32)
    yield "mixed_huge", np.concatenate([rng.standard_normal(200 * s).astype(np.float32),
                                        np.float32([2.0 ** 113, -2.0 ** 113, 3.3e38, 1.0e34])])
    yield "ties", (rng.integers(-40, 41, 500 * s) * 512.0
                   + rng.integers(-64, 65, 500 * s) * 2.0 ** -4).astype(np.float32)
