"""The C ABI under HIP graph capture.

The entry points allocate nothing, clear no memory with a runtime call and
leave their ticket counters at zero, so a caller can capture them once and
replay them.  The graph here holds the tree sum, the row variance, the
chunked column variance (several launches) and the ADN sum; it is replayed
several times with eager work between the replays (outputs overwritten,
new input data copied in) and every replay is checked bit for bit against
the oracle for the data it saw.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import adn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stable_variance_amd import build as libbuild

    if libbuild.is_stale():
        libbuild.build()
    return torch, torch.device("cuda:0")


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def test_capture_and_replay(torch_dev):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    L = sv.capi()
    N, (RR, RC), (CR, CC) = 2_000_003, (300, 4096), (3000, 256)

    def data(seed):
        rng = np.random.default_rng(seed)
        return (W.sum_cancelling_pairs(N, 0.01, seed=seed),
                rng.normal(1e4, 1, (RR, RC)).astype(np.float32),
                rng.normal(-2e3, 3, (CR, CC)).astype(np.float32))

    def expected(d):
        s, a, b = d
        return (oracle.tree_sum(s), oracle.variance(a, axis=1), oracle.variance(b, axis=0), adn.adn_sum(s))

    first, second = data(1), data(2)
    xs = [torch.from_numpy(v).to(dev) for v in first]
    sum_out = torch.empty(1, device=dev)
    adn_out = torch.empty(1, device=dev)
    rv, rm = torch.empty(RR, device=dev), torch.empty(RR, device=dev)
    cv, cm = torch.empty(CC, device=dev), torch.empty(CC, device=dev)
    ws_sum = torch.zeros(L.sv_tree_sum_f32_workspace_size(N), dtype=torch.uint8, device=dev)
    ws_adn = torch.zeros(L.sv_adn_sum_f32_workspace_size(N), dtype=torch.uint8, device=dev)
    ws_col = torch.zeros(L.sv_variance_f32_workspace_size(CR, CC, 0), dtype=torch.uint8, device=dev)
    assert L.sv_variance_f32_workspace_size(RR, RC, 1) == 0

    def enqueue(h):
        p = ctypes.c_void_p
        st = [L.sv_tree_sum_f32(p(xs[0].data_ptr()), N, p(sum_out.data_ptr()), p(ws_sum.data_ptr()),
                                ws_sum.numel(), p(h)),
              L.sv_variance_f32(p(xs[1].data_ptr()), RR, RC, 1, 0, p(rv.data_ptr()), p(rm.data_ptr()), None, 0,
                                p(h)),
              L.sv_variance_f32(p(xs[2].data_ptr()), CR, CC, 0, 0, p(cv.data_ptr()), p(cm.data_ptr()),
                                p(ws_col.data_ptr()), ws_col.numel(), p(h)),
              L.sv_adn_sum_f32(p(xs[0].data_ptr()), N, 3, p(adn_out.data_ptr()), p(ws_adn.data_ptr()),
                               ws_adn.numel(), p(h))]
        assert st == [0, 0, 0, 0], (st, L.sv_last_error_message())

    def check(want, tag):
        torch.cuda.synchronize()
        s, (v1, m1), (v0, m0), a = want
        assert bits(sum_out.cpu().numpy())[0] == bits(s)[0], tag
        assert np.array_equal(bits(rv.cpu().numpy()), bits(v1)) and np.array_equal(bits(rm.cpu().numpy()), bits(m1)), tag
        assert np.array_equal(bits(cv.cpu().numpy()), bits(v0)) and np.array_equal(bits(cm.cpu().numpy()), bits(m0)), tag
        assert bits(adn_out.cpu().numpy())[0] == bits(a)[0], tag

    want1, want2 = expected(first), expected(second)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        enqueue(s.cuda_stream)  # eager, on the stream the graph is captured from
    s.synchronize()
    check(want1, "eager")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        enqueue(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    for rep in range(6):
        # eager work between replays: outputs overwritten, inputs swapped
        for t in (sum_out, adn_out, rv, rm, cv, cm):
            t.fill_(float("nan"))
        d, want = (second, want2) if rep % 2 else (first, want1)
        for t, v in zip(xs, d):
            t.copy_(torch.from_numpy(v))
        torch.cuda.synchronize()
        g.replay()
        check(want, f"replay {rep}")
    # the counters of both sums are back at zero after the replays
    torch.cuda.synchronize()
    assert int(ws_sum[:33024].count_nonzero().item()) == 0  # SV_TREE_SUM_COUNTER_BYTES
    assert int(ws_adn[:33024].count_nonzero().item()) == 0  # SV_ADN_SUM_COUNTER_BYTES
