"""The Python binding: argument checks on the host (CPU tensors never reach
the library) and, on the GPU, the shape and dtype conventions of ``var``,
``tree_sum`` and ``adn_sum`` against the oracle."""
import numpy as np
import pytest
import torch

import oracle


def test_host_side_refusals():
    import stable_variance_amd as sv

    x = torch.zeros(8)
    with pytest.raises(ValueError):
        sv.var(x)  # a CPU tensor: refused before any library call
    with pytest.raises(ValueError):
        sv.tree_sum(x)
    with pytest.raises(TypeError):
        sv.var(torch.zeros(8, dtype=torch.float16))
    with pytest.raises(TypeError):
        sv.tree_sum(torch.zeros(8, dtype=torch.int32))
    with pytest.raises(TypeError):
        sv.var([1.0, 2.0])
    with pytest.raises(TypeError):
        sv.adn_sum(torch.zeros(8, dtype=torch.float64))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stable_variance_amd import build as libbuild

    if libbuild.is_stale():
        libbuild.build()
    return torch.device("cuda:0")


def bits(a, dt=np.float32):
    return np.ascontiguousarray(a, dt).view(np.uint32 if dt == np.float32 else np.uint64)


@pytest.mark.gpu
def test_var_shapes_dims_and_dtypes(dev):
    import stable_variance_amd as sv

    rng = np.random.default_rng(3)
    a = rng.normal(50.0, 2.0, (37, 300)).astype(np.float32)
    t = torch.from_numpy(a).to(dev)
    for dim, axis in ((1, 1), (-1, 1), (0, 0), (-2, 0)):
        v, m = sv.var(t, dim=dim, ddof=1, return_mean=True)
        ov, om = oracle.variance(a, axis=axis, ddof=1)
        assert v.dtype == torch.float32 and v.shape == (a.shape[0] if axis == 1 else a.shape[1],)
        assert np.array_equal(bits(v.cpu().numpy()), bits(ov)) and np.array_equal(bits(m.cpu().numpy()), bits(om))
    # 1-D input: a 0-d result
    v = sv.var(t[3])
    assert v.shape == () and bits(v.cpu().numpy().reshape(1))[0] == bits(oracle.variance(a[3:4], axis=1)[0])[0]
    # a transposed (non-contiguous) view is copied first: same as its contiguous copy
    vt = sv.var(t.t(), dim=1)
    assert np.array_equal(bits(vt.cpu().numpy()), bits(oracle.variance(np.ascontiguousarray(a.T), axis=1)[0]))
    # float64 keeps its dtype
    d = torch.from_numpy(a.astype(np.float64)).to(dev)
    v64 = sv.var(d, dim=0)
    assert v64.dtype == torch.float64
    assert np.array_equal(bits(v64.cpu().numpy(), np.float64), bits(oracle.variance_f64(a.astype(np.float64), axis=0)[0], np.float64))
    # complex64: float32 variance, complex64 mean
    z = (a + 1j * a[::-1]).astype(np.complex64)
    vz, mz = sv.var(torch.from_numpy(z).to(dev), dim=1, return_mean=True)
    assert vz.dtype == torch.float32 and mz.dtype == torch.complex64
    with pytest.raises(ValueError):
        sv.var(t, dim=2)
    with pytest.raises(ValueError):
        sv.var(t[0], dim=1)
    with pytest.raises(ValueError):
        sv.var(t.reshape(1, 37, 300))
    with pytest.raises(ValueError):
        sv.var(t, ddof=-1)


@pytest.mark.gpu
def test_sums_flatten_and_empty(dev):
    import stable_variance_amd as sv

    a = np.random.default_rng(4).normal(0, 1, (50, 999)).astype(np.float32)
    t = torch.from_numpy(a).to(dev)
    s = sv.tree_sum(t)  # any shape: all elements, row-major order
    assert s.shape == () and bits(s.cpu().numpy().reshape(1))[0] == bits(oracle.tree_sum(a.ravel()))[0]
    s = sv.tree_sum(t.t())  # a transposed view sums its own (column-major) order
    assert bits(s.cpu().numpy().reshape(1))[0] == bits(oracle.tree_sum(np.ascontiguousarray(a.T).ravel()))[0]
    assert sv.tree_sum(t, carry="dw").item() == float(oracle.tree_sum_dw(a.ravel()))
    e = torch.zeros(0, device=dev)
    assert sv.tree_sum(e).item() == 0.0 and sv.adn_sum(e).item() == 0.0
    with pytest.raises(ValueError):
        sv.tree_sum(t, carry="kahan")
