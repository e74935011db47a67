"""Seeded random shapes through every dispatch path, bit for bit.

Rows and columns are drawn log-uniformly, up to 3 M values per case. Each case
varies the dtype (float32, float64, complex64), the axis, ddof and the base
alignment: a view one element into a larger buffer makes the rows misaligned
for 16-byte loads. Every case is compared with the oracle on the same
values, bit for bit.

The draws cover the boundaries between the kernels by chance rather than by
choice: short rows sharing waves; the power-of-two tiles; long rows; short,
one-launch and chunked columns; narrow matrices; ragged and odd widths. The
generator is seeded, so the cases are the same on every run.
"""
import numpy as np
import pytest
import torch  # noqa: F401  (imported at collection: the first import is slow on a fresh box)

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

N_CASES = 72
MAX_VALUES = 3_000_000


def _draw_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    while len(cases) < N_CASES:
        r = int(np.exp(rng.uniform(0.0, np.log(400_000))))
        c = int(np.exp(rng.uniform(0.0, np.log(400_000))))
        if not 1 <= r * c <= MAX_VALUES:
            continue
        dtype = ("f32", "f32", "f64", "c64")[int(rng.integers(4))]
        axis = int(rng.integers(2))
        ddof = (0, 0, 1, 3)[int(rng.integers(4))]
        offset = int(rng.integers(2))
        seed = int(rng.integers(1 << 30))
        cases.append((dtype, r, c, axis, ddof, offset, seed))
    return cases


CASES = _draw_cases()


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stable_variance_amd import build as libbuild

    if libbuild.is_stale():
        libbuild.build()
    return torch, torch.device("cuda:0")


def _bits(a, dt):
    a = np.ascontiguousarray(a, dt)
    return a.view(np.uint64 if dt == np.float64 else np.uint32)


def _same(a, b, dt):
    a = np.ascontiguousarray(a, dt).ravel()
    b = np.ascontiguousarray(b, dt).ravel()
    if a.shape != b.shape:
        return False
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (_bits(a, dt) == _bits(b, dt))))


def _values(rng, r, c, seed):
    # mostly well-conditioned data with a random offset, some adversarial
    # (huge, tiny, signed zeros, cancelling) values
    if rng.random() < 0.25:
        return W.adversarial_values(r * c, seed).reshape(r, c).astype(np.float64)
    return rng.normal(rng.uniform(-1e5, 1e5), rng.uniform(0.01, 10.0), (r, c))


def _device_view(torch, dev, host, offset):
    """host copied into a device buffer, `offset` elements in (a contiguous
    view whose base is then not 16-byte aligned)."""
    flat = torch.from_numpy(np.ascontiguousarray(host).ravel())
    buf = torch.empty(flat.numel() + offset, dtype=flat.dtype, device=dev)
    buf[offset:] = flat.to(dev)
    return buf[offset:].view(host.shape)


@pytest.mark.parametrize("case", range(N_CASES), ids=[f"{d}-{r}x{c}-ax{a}-ddof{k}-off{o}"
                                                     for d, r, c, a, k, o, _ in CASES])
def test_random_shape(torch_dev, case):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    dtype, r, c, axis, ddof, offset, seed = CASES[case]
    rng = np.random.default_rng(seed)
    base = _values(rng, r, c, seed)
    if dtype == "f32":
        a = base.astype(np.float32)
        want_v, want_m = oracle.variance(a, axis=axis, ddof=ddof)
        check_dt = np.float32
    elif dtype == "f64":
        a = base
        want_v, want_m = oracle.variance_f64(a, axis=axis, ddof=ddof)
        check_dt = np.float64
    else:
        a = (base + 1j * _values(rng, r, c, seed + 1)).astype(np.complex64)
        want_v, want_m = oracle.variance_complex(a, axis=axis, ddof=ddof)
        check_dt = np.float32
    t = _device_view(torch, dev, a, offset)
    v, m = sv.var(t, dim=axis, ddof=ddof, return_mean=True)
    torch.cuda.synchronize()
    v, m = v.cpu().numpy(), m.cpu().numpy()
    if dtype == "c64":
        m, want_m = m.view(np.float32), np.ascontiguousarray(want_m).view(np.float32)
    assert _same(v, want_v, check_dt), (CASES[case], np.flatnonzero(~np.isclose(v, want_v, equal_nan=True))[:5])
    assert _same(m, want_m, check_dt), CASES[case]


# ------------------------------------------------------------------ sums

def _draw_sum_cases():
    rng = np.random.default_rng(31337)
    cases = []
    for _ in range(24):
        n = int(np.exp(rng.uniform(0.0, np.log(6_000_000))))
        kind = ("f32", "f32", "dw", "f64", "adn")[int(rng.integers(5))]
        offset = int(rng.integers(4))
        fold = int(rng.integers(2, 9))
        seed = int(rng.integers(1 << 30))
        cases.append((kind, n, offset, fold, seed))
    return cases


SUM_CASES = _draw_sum_cases()


@pytest.mark.parametrize("case", range(len(SUM_CASES)),
                         ids=[f"{k}-n{n}-off{o}" + (f"-K{f}" if k == "adn" else "") for k, n, o, f, _ in SUM_CASES])
def test_random_sum(torch_dev, case):
    # tree sums (plain and double-word carries, float32 and float64) and the
    # ADN sum over random lengths, from bases 0..3 elements into a buffer
    import stable_variance_amd as sv
    from oracle import adn

    torch, dev = torch_dev
    kind, n, offset, fold, seed = SUM_CASES[case]
    rng = np.random.default_rng(seed)
    if rng.random() < 0.5:
        x = W.sum_cancelling_pairs(n, 0.01, seed=seed)
    else:
        x = W.adversarial_values(n, seed) if rng.random() < 0.5 else rng.normal(0, 1, n).astype(np.float32)
    if kind == "f64":
        x = x.astype(np.float64) * 1e100
    t = _device_view(torch, dev, x, offset)
    if kind == "f32":
        got, want, dt = sv.tree_sum(t), oracle.tree_sum(x), np.float32
    elif kind == "dw":
        got, want, dt = sv.tree_sum(t, carry="dw"), oracle.tree_sum_dw(x), np.float32
    elif kind == "f64":
        got, want, dt = sv.tree_sum(t), oracle.tree_sum_f64(x), np.float64
    else:
        got, want, dt = sv.adn_sum(t, fold=fold), adn.adn_sum(x, fold), np.float32
    torch.cuda.synchronize()
    assert _same(np.asarray(got.item(), dt), np.asarray(want, dt), dt), (SUM_CASES[case], got.item(), want)
