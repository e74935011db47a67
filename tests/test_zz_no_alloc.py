"""The tree sum without a workspace argument (sv_tree_sum_f32_noalloc).

It runs the same kernels as sv_tree_sum_f32 on a scratch array inside the
library, so its results must be the workspace entry point's bit for bit,
also on consecutive calls that reuse the array (the second one smaller, so
that stale partial nodes of the first would show), and it must reject what
it cannot serve before touching the device.
"""
import ctypes

import numpy as np
import pytest

import workloads as W

SV_OK, SV_ERR_INVALID_ARGUMENT, SV_ERR_UNSUPPORTED = 0, 1, 5
BAD = ctypes.c_void_p(0x1000)  # never dereferenced: these calls fail on the host


def test_noalloc_argument_errors():
    import stable_variance_amd as sv

    L = sv.capi()
    assert L.sv_tree_sum_f32_noalloc(BAD, -1, BAD, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_tree_sum_f32_noalloc(BAD, (1 << 36) + 1, BAD, None) == SV_ERR_UNSUPPORTED
    assert b"2^36" in L.sv_last_error_message()
    assert L.sv_tree_sum_f32_noalloc(BAD, 5, None, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_tree_sum_f32_noalloc(None, 5, BAD, None) == SV_ERR_INVALID_ARGUMENT


def _bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point():
    import torch

    import oracle
    import stable_variance_amd as sv

    L = sv.capi()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    ws_bytes = L.sv_tree_sum_f32_workspace_size(1 << 30)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out_ws = torch.empty((), dtype=torch.float32, device=dev)
    out_na = torch.empty((), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(77)
    big = W.sum_cancelling_pairs(3_000_017, seed=4)
    cases = [
        big,                                                   # many workgroups, both ticket levels
        rng.normal(0, 1, 1000).astype(np.float32),             # second call smaller: one workgroup
        W.sum_pm1e16(),
        W.adversarial_values(40_000, 3),
        np.zeros(0, np.float32),
        np.full(7, -0.0, np.float32),
    ]
    for x in cases:
        t = torch.from_numpy(x).to(dev)
        p = t.data_ptr() if x.size else None
        print("noalloc case n =", x.size, flush=True)
        assert L.sv_tree_sum_f32(p, x.size, out_ws.data_ptr(), ws.data_ptr(), ws_bytes, stream.cuda_stream) == SV_OK
        st = L.sv_tree_sum_f32_noalloc(p, x.size, out_na.data_ptr(), stream.cuda_stream)
        assert st == SV_OK, L.sv_last_error_message()
        torch.cuda.synchronize()
        a, b = np.float32(out_ws.item()), np.float32(out_na.item())
        assert _bits(a) == _bits(b), (x.size, a, b)
        assert _bits(b) == _bits(oracle.tree_sum(x)), (x.size, b)
    # two calls in a row with no host synchronisation between them, the
    # second on a smaller input: the shared array must not carry anything over
    x1 = torch.from_numpy(big).to(dev)
    x2 = torch.from_numpy(big[:123_457].copy()).to(dev)
    o1 = torch.empty((), dtype=torch.float32, device=dev)
    o2 = torch.empty((), dtype=torch.float32, device=dev)
    assert L.sv_tree_sum_f32_noalloc(x1.data_ptr(), x1.numel(), o1.data_ptr(), stream.cuda_stream) == SV_OK
    assert L.sv_tree_sum_f32_noalloc(x2.data_ptr(), x2.numel(), o2.data_ptr(), stream.cuda_stream) == SV_OK
    torch.cuda.synchronize()
    assert _bits(o1.item()) == _bits(oracle.tree_sum(big))
    assert _bits(o2.item()) == _bits(oracle.tree_sum(big[:123_457]))
