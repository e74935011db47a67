"""GPU parity of the ADN binned reproducible sum against the CPU oracle.

Bit-exact for every input, fold count, launch geometry and order of the
values ([ADN] "SyclReproSum" README: same bits for any order and schedule).
"""
import numpy as np
import pytest
import torch  # noqa: F401  (imported at collection: the first import is slow on a fresh box)

import workloads as W
from oracle import adn

pytestmark = pytest.mark.gpu

GEOMETRIES = {
    "default": {},
    "e32": {"adn_e": 32},
    "few_blocks": {"adn_blocks": 7},
    "single_workgroup": {"adn_blocks": 1},
    "many_blocks": {"adn_blocks": 8192},
}


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stable_variance_amd import build as libbuild

    if libbuild.is_stale():
        libbuild.build()
    return torch, torch.device("cuda:0")


@pytest.fixture(params=list(GEOMETRIES), ids=list(GEOMETRIES))
def geometry(request, torch_dev):
    import stable_variance_amd as sv

    sv.set_tuning("reset", 0)
    for k, v in GEOMETRIES[request.param].items():
        sv.set_tuning(k, v)
    yield request.param
    sv.set_tuning("reset", 0)


def bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def gpu_adn(torch_dev, x, fold=3, offset=0):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    x = np.ascontiguousarray(x, np.float32)
    if offset:
        buf = torch.zeros(x.size + offset, dtype=torch.float32, device=dev)
        buf[offset:] = torch.from_numpy(x).to(dev)
        t = buf[offset:]
    else:
        t = torch.from_numpy(x).to(dev)
    r = sv.adn_sum(t, fold)
    torch.cuda.synchronize()
    return np.float32(r.item())


@pytest.mark.parametrize("fold", list(range(2, 22)))
def test_mixed_sets_every_fold(torch_dev, fold):
    # every fold count the page allows for float (2..21); from 21 folds the
    # index always reaches the scaled coarsest bins (the general path)
    for seed in range(2):
        for name, x in W.sum_mixed_sets(seed, scale=20):
            want = adn.adn_sum(x, fold)
            assert bits(gpu_adn(torch_dev, x, fold)) == bits(want), (name, fold, seed)


def test_geometries_sizes_and_alignment(torch_dev, geometry):
    rng = np.random.default_rng(11)
    for n in (1, 63, 64, 2047, 2048, 2049, 8191, 65537, 64 * 32 * 4 * 3 + 5, 1_000_003):
        x = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
        want = adn.adn_sum(x, 3)
        assert bits(gpu_adn(torch_dev, x)) == bits(want), (geometry, n)
        assert bits(gpu_adn(torch_dev, x, offset=1)) == bits(want), (geometry, n, "unaligned")


def test_order_independence(torch_dev):
    # a million wide-range values and six permutations: one bit pattern, the oracle's
    rng = np.random.default_rng(12)
    n = 1_000_000
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    want = bits(adn.adn_sum(x, 3))
    got = {bits(gpu_adn(torch_dev, x[rng.permutation(n)])) for _ in range(6)}
    got.add(bits(gpu_adn(torch_dev, x[::-1])))
    assert got == {want}


def test_quick_start_and_empty(torch_dev):
    x = W.sum_pm1e16()
    assert gpu_adn(torch_dev, x, 3) == adn.adn_sum(x, 3) == 0.0
    assert gpu_adn(torch_dev, x, 5) == 10000.0
    assert bits(gpu_adn(torch_dev, np.zeros(0, np.float32))) == 0
    assert bits(gpu_adn(torch_dev, np.full(5000, -0.0, np.float32))) == 0


@pytest.mark.parametrize("fold", [9, 16, 21])
def test_high_folds_sizes_alignment_and_specials(torch_dev, fold):
    rng = np.random.default_rng(14 + fold)
    for n in (1, 2049, 65537, 300_003):
        x = (rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(np.float32)
        want = adn.adn_sum(x, fold)
        assert bits(gpu_adn(torch_dev, x, fold)) == bits(want), (fold, n)
        assert bits(gpu_adn(torch_dev, x, fold, offset=1)) == bits(want), (fold, n, "unaligned")
    big = np.array([3e38, -3e38, 1e30, 1.0, -2.5e-40], np.float32)
    assert bits(gpu_adn(torch_dev, big, fold)) == bits(adn.adn_sum(big, fold))
    assert bits(gpu_adn(torch_dev, np.array([1.0, np.inf], np.float32), fold)) == bits(np.float32(np.inf))
    assert bits(gpu_adn(torch_dev, np.array([np.nan, 1.0], np.float32), fold)) == 0x7FC00000


def test_specials(torch_dev):
    rng = np.random.default_rng(13)
    n = 300_000
    base = rng.standard_normal(n).astype(np.float32)
    snan = np.array([0x7FA12345], np.uint32).view(np.float32)[0]
    negnan = np.array([0xFFC00001], np.uint32).view(np.float32)[0]
    cases = [([snan], 0x7FC00000), ([negnan], 0x7FC00000), ([np.inf, -np.inf], 0x7FC00000),
             ([np.nan, np.inf], 0x7FC00000), ([np.inf], 0x7F800000), ([-np.inf, -np.inf], 0xFF800000)]
    for extra, want in cases:
        x = base.copy()
        pos = rng.choice(n, len(extra), replace=False)
        x[pos] = np.array(extra, np.float32)
        assert bits(gpu_adn(torch_dev, x)) == want, extra
        assert bits(adn.adn_sum(x)) == want
    big = np.float32(3.0e38)
    x = np.concatenate([base, np.array([big, big], np.float32)])
    assert gpu_adn(torch_dev, x) == np.inf == adn.adn_sum(x)


def test_workspace_counters_left_zero(torch_dev):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    x = W.sum_cancelling_pairs(3_000_000, 0.01, seed=4)
    t = torch.from_numpy(x).to(dev)
    want = bits(adn.adn_sum(x))
    for _ in range(3):
        assert bits(sv.adn_sum(t).item()) == want
    torch.cuda.synchronize()
    ws = [v for k, v in sv._workspaces.items() if k[0] == "adn"]
    assert ws and all(int(w[:33024].count_nonzero().item()) == 0 for w in ws)


def test_full_size_1e8(torch_dev):
    # the 10^8-value sum workload (99% N(0,1), 1% large cancelling pairs, seed 3)
    import stable_variance_amd as sv

    x = W.sum_cancelling_pairs()
    want = bits(adn.adn_sum(x, 3))
    for knobs in ({}, {"adn_e": 32}, {"adn_blocks": 8192}):
        sv.set_tuning("reset", 0)
        for k, v in knobs.items():
            sv.set_tuning(k, v)
        assert bits(gpu_adn(torch_dev, x)) == want, knobs
    sv.set_tuning("reset", 0)
