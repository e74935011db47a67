"""CPU oracle for the compensated-tree float32 sum and variance.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``stable_variance_amd``) never imports, links or runs anything here,
and nothing here imports the product path: the two share no code.

Contents
  * ``sv_oracle.c`` (built into ``liboracle.so`` by :func:`build`): the
    scalar, level-by-level float32 algorithm of the method page, plus the
    naive and two-term reference formulae and the sequential Kahan loop.
  * :func:`np_tree_sum` / :func:`np_tree_plain`: the same trees written as
    vectorised numpy float32 levels (a second implementation of the
    definition, used to cross-check the C code, not as a pin).
  * :mod:`oracle.adn`: the Ahrens-Demmel-Nguyen binned reproducible sum of
    the "SyclReproSum" README, as a closed form and as its float32 steps.
  * Exact truth: :func:`exact_sum` (integer arithmetic on the float32
    mantissas) and :func:`round_f32` (round-to-nearest-even of an exact
    dyadic value), :func:`var_f64` (float64 variance, the method page's
    accuracy reference, "Variance in float32 ..." §3).

Citations are to the pages by title and section:
  [VAR]   Pennacchio, "Variance in float32 with a first-element shift, a local
          centring and a compensated tree sum": §1, §2 steps 1-4, §3.
  [KAHAN] "Kahan's Summation Formula" (the C and Fortran loops and outputs).
  [ADN]   "SyclReproSum" README (the +/-1e16 quick-start example).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Strict IEEE float32 evaluation: SSE scalar code, no contraction, no
# fast-math, no CPU-specific code generation.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-fexcess-precision=standard", "-fPIC", "-shared", "-Wall", "-Wextra"]

# The kernel of [VAR] §2.  READING of step 2: the local mean's sum of y is
# the plain pairwise tree (METHOD_KERNEL); the compensated tree of step 3
# sums the residuals d and d^2.  METHOD_KERNEL_COMP_SY is the other reading,
# every sum of the slice on the compensated tree.
METHOD_KERNEL = 0
METHOD_KERNEL_COMP_SY = 1
METHOD_REFERENCE = 2
METHOD_NAIVE = 3
# Ablation rows of the method page's §4 (one step changed at a time)
METHOD_SHIFT_PLAIN_NO2T = 4      # shift + centring, plain tree, no two-term
METHOD_SHIFT_PLAIN_2T = 5        # shift + centring + two-term, plain tree
METHOD_NOSHIFT_COMP_2T = 6       # no shift, two-term, compensated tree
METHOD_SHIFT_COMP_NO2T = 7       # shift + centring, compensated tree, no two-term
METHOD_SHIFT_KAHAN_NO2T = 8      # shift + centring, sequential Kahan scan, no two-term
METHOD_KERNEL_DW = 9             # the method with double-word carries in its compensated trees

_lib = None


def build(force: bool = True) -> str:
    """Compile ``sv_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    """The loaded oracle library (built on first use if absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        i64 = ctypes.c_int64
        L.orc_two_sum.restype = ctypes.c_float
        L.orc_two_sum.argtypes = [ctypes.c_float, ctypes.c_float, fp]
        for name in ("orc_tree_sum_f32", "orc_tree_plain_f32", "orc_tree_sum_dw_f32"):
            f = getattr(L, name)
            f.restype = ctypes.c_float
            f.argtypes = [fp, i64, i64, i64]
        for name in ("orc_seq_naive_f32", "orc_seq_kahan_f32", "orc_seq_neumaier_f32"):
            f = getattr(L, name)
            f.restype = ctypes.c_float
            f.argtypes = [fp, i64]
        dp = ctypes.POINTER(ctypes.c_double)
        L.orc_two_sum_f64.restype = ctypes.c_double
        L.orc_two_sum_f64.argtypes = [ctypes.c_double, ctypes.c_double, dp]
        L.orc_tree_sum_f64.restype = ctypes.c_double
        L.orc_tree_sum_f64.argtypes = [dp, i64, i64, i64]
        L.orc_variance_f64.restype = ctypes.c_int
        L.orc_variance_f64.argtypes = [dp, i64, i64, ctypes.c_int, i64, ctypes.c_int, dp, dp]
        L.orc_tree_node_f32.restype = ctypes.c_int
        L.orc_tree_node_f32.argtypes = [fp, i64, i64, fp, fp]
        L.orc_variance_f32.restype = ctypes.c_int
        L.orc_variance_f32.argtypes = [fp, i64, i64, ctypes.c_int, i64, ctypes.c_int, fp, fp]
        _lib = L
    return _lib


def _f32c(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


# ---------------------------------------------------------------------------
# Scalar C oracle wrappers
# ---------------------------------------------------------------------------

def two_sum(a: float, b: float) -> tuple[np.float32, np.float32]:
    """TwoSum of two float32 values: (fl(a+b), exact error)."""
    e = ctypes.c_float(0.0)
    s = lib().orc_two_sum(ctypes.c_float(np.float32(a)), ctypes.c_float(np.float32(b)), ctypes.byref(e))
    return np.float32(s), np.float32(e.value)


def tree_sum(x, pad_to: int = 0) -> np.float32:
    """Compensated pairwise tree sum ([VAR] §2 step 3) of a 1-D float32 array."""
    a = _f32c(x).ravel()
    return np.float32(lib().orc_tree_sum_f32(_ptr(a), a.size, 1, int(pad_to)))


def tree_sum_dw(x, pad_to: int = 0) -> np.float32:
    """Compensated tree with double-word carries: each node's pair is
    renormalised with TwoSum (see ``orc_tree_sum_dw_f32``)."""
    a = _f32c(x).ravel()
    return np.float32(lib().orc_tree_sum_dw_f32(_ptr(a), a.size, 1, int(pad_to)))


def tree_sum_threads(x, threads: int) -> np.float32:
    """The compensated tree of ``x`` computed on up to ``threads`` host
    threads: the padded tree is cut into 2^k aligned subtrees (one per
    thread, in C, which runs without the GIL), whose root nodes are then
    combined level by level with the same node.  Same bits as tree_sum."""
    from concurrent.futures import ThreadPoolExecutor

    a = _f32c(x).ravel()
    n = a.size
    if n == 0:
        return np.float32(0.0)
    P = 1 << max(0, (n - 1).bit_length())
    T = 1
    while T * 2 <= max(1, threads) and P // (T * 2) >= 1:
        T *= 2
    cs = P // T

    def node(i):
        lo = i * cs
        piece = np.ascontiguousarray(a[lo:min(lo + cs, n)])
        s, c = ctypes.c_float(0.0), ctypes.c_float(0.0)
        rc = lib().orc_tree_node_f32(_ptr(piece), piece.size, cs, ctypes.byref(s), ctypes.byref(c))
        if rc != 0:
            raise RuntimeError("orc_tree_node_f32 failed")
        return np.float32(s.value), np.float32(c.value)

    with ThreadPoolExecutor(max_workers=T) as ex:
        nodes = list(ex.map(node, range(T)))
    with np.errstate(invalid="ignore", over="ignore"):
        while len(nodes) > 1:
            nxt = []
            for k in range(0, len(nodes), 2):
                (sl, cl), (sr, cr) = nodes[k], nodes[k + 1]
                s, e = two_sum(sl, sr)
                nxt.append((s, np.float32(np.float32(cl + cr) + e)))
            nodes = nxt
        s, c = nodes[0]
        return s if not np.isfinite(s) else np.float32(s + c)


def variance_threads(x, axis: int, threads: int, ddof: int = 0):
    """oracle.variance over blocks of slices on up to ``threads`` host
    threads (slices are independent; same bits)."""
    from concurrent.futures import ThreadPoolExecutor

    a = np.ascontiguousarray(x, np.float32)
    ax = axis % 2
    nsl = a.shape[0] if ax == 1 else a.shape[1]
    T = max(1, min(threads, nsl))
    bounds = [(i * nsl // T, (i + 1) * nsl // T) for i in range(T)]

    def part(b):
        lo, hi = b
        blk = a[lo:hi] if ax == 1 else np.ascontiguousarray(a[:, lo:hi])
        return variance(blk, axis=ax, ddof=ddof)

    with ThreadPoolExecutor(max_workers=T) as ex:
        res = list(ex.map(part, bounds))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def two_sum_f64(a: float, b: float) -> tuple[float, float]:
    e = ctypes.c_double(0.0)
    s = lib().orc_two_sum_f64(float(a), float(b), ctypes.byref(e))
    return s, e.value


def tree_sum_f64(x, pad_to: int = 0) -> np.float64:
    """Compensated pairwise tree in binary64 (same topology and readings)."""
    a = np.ascontiguousarray(x, np.float64).ravel()
    return np.float64(lib().orc_tree_sum_f64(_dptr(a), a.size, 1, int(pad_to)))


def variance_f64(x, axis: int = -1, ddof: int = 0, method: int = METHOD_KERNEL):
    """The method (METHOD_KERNEL, or METHOD_KERNEL_COMP_SY for the other
    reading of step 2) or the two-term reference (METHOD_REFERENCE) on a
    2-D float64 array, every operation in binary64."""
    a = np.ascontiguousarray(x, np.float64)
    if a.ndim == 1:
        a = a.reshape(1, -1)
        axis = 1
    rows, cols = a.shape
    ax = axis % 2
    ns = rows if ax == 1 else cols
    var = np.empty(ns, np.float64)
    mean = np.empty(ns, np.float64)
    rc = lib().orc_variance_f64(_dptr(a), rows, cols, ax, int(ddof), int(method), _dptr(var), _dptr(mean))
    if rc != 0:
        raise ValueError(f"orc_variance_f64 failed ({rc})")
    return var, mean


def tree_plain(x, pad_to: int = 0) -> np.float32:
    """Plain pairwise tree (same topology, no error array)."""
    a = _f32c(x).ravel()
    return np.float32(lib().orc_tree_plain_f32(_ptr(a), a.size, 1, int(pad_to)))


def seq_naive(x) -> np.float32:
    a = _f32c(x).ravel()
    return np.float32(lib().orc_seq_naive_f32(_ptr(a), a.size))


def seq_kahan(x) -> np.float32:
    """The sequential Kahan loop of [KAHAN]."""
    a = _f32c(x).ravel()
    return np.float32(lib().orc_seq_kahan_f32(_ptr(a), a.size))


def seq_neumaier(x) -> np.float32:
    a = _f32c(x).ravel()
    return np.float32(lib().orc_seq_neumaier_f32(_ptr(a), a.size))


def variance(x, axis: int = -1, ddof: int = 0, method: int = METHOD_KERNEL):
    """Variance and mean of a 2-D float32 array along ``axis``.

    method: METHOD_KERNEL (the [VAR] §2 kernel: plain tree of y for the
    local mean, compensated trees of d and d^2), METHOD_KERNEL_COMP_SY (the
    same with a compensated tree of y), METHOD_REFERENCE (the two-term
    formula of [VAR] §1), METHOD_NAIVE, and the ablation rows 4..9.
    Returns (var, mean) as float32 arrays.
    """
    a = _f32c(x)
    if a.ndim == 1:
        a = a.reshape(1, -1)
        axis = 1
    if a.ndim != 2:
        raise ValueError("variance: expects a 1-D or 2-D array")
    ax = axis % 2
    rows, cols = a.shape
    ns = rows if ax == 1 else cols
    var = np.empty(ns, np.float32)
    mean = np.empty(ns, np.float32)
    rc = lib().orc_variance_f32(_ptr(a), rows, cols, ax, int(ddof), int(method), _ptr(var), _ptr(mean))
    if rc != 0:
        raise ValueError(f"orc_variance_f32 rejected the arguments (rc={rc})")
    return var, mean


# ---------------------------------------------------------------------------
# Vectorised numpy form of the same trees (cross-check of the C code)
# ---------------------------------------------------------------------------

def _pad_pow2(a: np.ndarray, pad_to: int = 0) -> np.ndarray:
    n = a.shape[-1]
    P = 1
    while P < n:
        P <<= 1
    if pad_to:
        P = pad_to
    out = np.zeros(a.shape[:-1] + (P,), np.float32)
    out[..., :n] = a
    return out


def np_tree_sum(x, pad_to: int = 0) -> np.ndarray:
    """Compensated tree along the last axis, one vectorised level at a time."""
    a = np.asarray(x, dtype=np.float32)
    if a.shape[-1] == 0:
        return np.zeros(a.shape[:-1], np.float32)
    s = _pad_pow2(a, pad_to)
    c = np.zeros_like(s)
    with np.errstate(invalid="ignore", over="ignore"):
        while s.shape[-1] > 1:
            l, r = s[..., 0::2], s[..., 1::2]
            t = l + r
            bv = t - l
            av = t - bv
            e = (l - av) + (r - bv)
            c = (c[..., 0::2] + c[..., 1::2]) + e
            s = t
        s, c = s[..., 0], c[..., 0]
        return np.where(np.isfinite(s), s + c, s).astype(np.float32)


def np_tree_sum_dw(x, pad_to: int = 0) -> np.ndarray:
    """Double-word-carry tree along the last axis, vectorised levels."""
    a = np.asarray(x, dtype=np.float32)
    if a.shape[-1] == 0:
        return np.zeros(a.shape[:-1], np.float32)
    s = _pad_pow2(a, pad_to)
    c = np.zeros_like(s)
    with np.errstate(invalid="ignore", over="ignore"):
        while s.shape[-1] > 1:
            l, r = s[..., 0::2], s[..., 1::2]
            t = l + r
            bv = t - l
            av = t - bv
            e = (l - av) + (r - bv)
            u = (c[..., 0::2] + c[..., 1::2]) + e
            s2 = t + u                     # renormalise (t, u) with TwoSum ...
            bv = s2 - t
            av = s2 - bv
            c2 = (t - av) + (u - bv)
            fin = np.isfinite(t)           # ... unless the sum is Inf or NaN
            s = np.where(fin, s2, t).astype(np.float32)
            c = np.where(fin, c2, u).astype(np.float32)
        s, c = s[..., 0], c[..., 0]
        return np.where(np.isfinite(s), s + c, s).astype(np.float32)


def np_tree_plain(x, pad_to: int = 0) -> np.ndarray:
    a = np.asarray(x, dtype=np.float32)
    if a.shape[-1] == 0:
        return np.zeros(a.shape[:-1], np.float32)
    s = _pad_pow2(a, pad_to)
    with np.errstate(invalid="ignore", over="ignore"):
        while s.shape[-1] > 1:
            s = s[..., 0::2] + s[..., 1::2]
        return (s[..., 0] + np.float32(0.0)).astype(np.float32)  # root: fl(s + 0)


# ---------------------------------------------------------------------------
# Exact truth
# ---------------------------------------------------------------------------

def exact_sum(x) -> Fraction:
    """The exact sum of finite float32 values, as a Fraction.

    Each value is m * 2^e with |m| < 2^24 an integer.  The integer mantissas
    are summed per exponent (in float64, exact because every partial sum is
    an integer below 2^53 for fewer than 2^29 values), then combined with
    Python integers.
    """
    a = np.asarray(x, dtype=np.float32).ravel()
    if a.size == 0:
        return Fraction(0)
    if not np.all(np.isfinite(a)):
        raise ValueError("exact_sum: non-finite input")
    if a.size >= (1 << 29):
        raise ValueError("exact_sum: too many values for exact float64 bins")
    mant, ex = np.frexp(a.astype(np.float64))          # a = mant * 2^ex, 0.5 <= |mant| < 1
    m_int = np.rint(mant * (1 << 24)).astype(np.int64)  # exact: float32 has 24 bits
    e_int = ex.astype(np.int64) - 24
    emin = int(e_int.min())
    bins = np.bincount(e_int - emin, weights=m_int.astype(np.float64))
    total = 0
    for k in range(bins.size - 1, -1, -1):
        total = (total << 1) + int(bins[k])
    # total is now sum_k bins[k] * 2^k, value = total * 2^emin
    return Fraction(total) * (Fraction(2) ** emin)


def round_f32(v: Fraction) -> np.float32:
    """Round an exact rational value to float32, nearest-even (subnormals and
    overflow to infinity included)."""
    v = Fraction(v)
    if v == 0:
        return np.float32(0.0)
    neg = v < 0
    v = -v if neg else v
    top = v.numerator.bit_length() - v.denominator.bit_length()
    if v < Fraction(2) ** top:
        top -= 1                      # now 2^top <= v < 2^(top+1)
    q = max(top - 23, -149)           # exponent of the float32 ulp at v
    scaled = v / (Fraction(2) ** q)
    keep = scaled.numerator // scaled.denominator
    rem = scaled - keep
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (keep & 1)):
        keep += 1
    if keep * Fraction(2) ** q >= Fraction(2) ** 128:
        r = np.float32(np.inf)
    else:
        r = np.float32(math.ldexp(keep, q))
    return np.float32(-r) if neg else r


def fl32_exact_sum(x) -> np.float32:
    """The correctly rounded float32 of the exact sum."""
    return round_f32(exact_sum(x))


def var_f64(x, axis: int = -1, ddof: int = 0) -> np.ndarray:
    """float64 variance of the same float32 values ([VAR] §3's reference)."""
    return np.var(np.asarray(x, dtype=np.float32).astype(np.float64), axis=axis, ddof=ddof)


def max_rel_err(v, v64) -> float:
    """Maximum relative error over slices; a slice whose float64 variance is
    0 must be exactly 0 (counts as inf otherwise)."""
    v = np.asarray(v, dtype=np.float64)
    v64 = np.asarray(v64, dtype=np.float64)
    zero = v64 == 0
    err = np.zeros_like(v64)
    nz = ~zero
    err[nz] = np.abs(v[nz] - v64[nz]) / np.abs(v64[nz])
    err[zero & (v != 0)] = np.inf
    return float(err.max()) if err.size else 0.0


def variance_complex(z, axis: int = -1, ddof: int = 0, method: int = METHOD_KERNEL):
    """Variance of complex64 data as the method page's §2 describes it: the
    real and imaginary parts are taken as two float32 arrays and their
    variances are added (in float32), which is E|z - mean(z)|^2."""
    z = np.asarray(z, dtype=np.complex64)
    vr, mr = variance(np.ascontiguousarray(z.real), axis=axis, ddof=ddof, method=method)
    vi, mi = variance(np.ascontiguousarray(z.imag), axis=axis, ddof=ddof, method=method)
    mean = np.empty(mr.shape, np.complex64)
    mean.real = mr
    mean.imag = mi
    return (vr + vi).astype(np.float32), mean
