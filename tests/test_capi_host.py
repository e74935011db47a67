"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every function the header declares, and
reject bad arguments on the host before touching the device.
"""
import ctypes
import os
import re

import pytest

import stable_variance_amd as sv
from stable_variance_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stable_variance.h")

SV_ERR_INVALID_ARGUMENT, SV_ERR_WORKSPACE, SV_ERR_NO_DEVICE, SV_ERR_UNSUPPORTED = 1, 2, 3, 5
BAD = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails on the host first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(libbuild.LIB):
        libbuild.build()
    return sv.capi()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sv_tree_sum_f32", "sv_variance_f32", "sv_tree_sum_f32_workspace_size",
              "sv_variance_f32_workspace_size", "sv_status_string", "sv_last_error_message", "sv_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings(L):
    assert L.sv_abi_version() == 1
    assert L.sv_status_string(0) == b"SV_OK"
    assert L.sv_status_string(3) == b"SV_ERR_NO_DEVICE"
    assert L.sv_status_string(99) == b"SV_ERR_UNKNOWN"


def test_workspace_sizes(L):
    assert L.sv_tree_sum_f32_workspace_size(0) == 0
    # counters (one top + one per 64 workgroups, 256 bytes apart), then a node
    # per workgroup (up to 8192) and per group of 64 workgroups
    want = 33024 + 8 * (8192 + 128)
    for n in (1, 4096, 4097, 10 ** 8, 1 << 36):
        assert L.sv_tree_sum_f32_workspace_size(n) == want
    assert L.sv_tree_sum_f32_workspace_size((1 << 36) + 1) == ctypes.c_size_t(-1).value
    assert L.sv_variance_f32_workspace_size(4096, 4096, 1) == 0
    assert L.sv_variance_f32_workspace_size(1, 64, 3) == ctypes.c_size_t(-1).value
    # axis 0: three node arrays of 8 bytes per 64-row chunk per column and 4
    # bytes of m per column, each rounded up to 256 bytes
    r256 = lambda b: (b + 255) // 256 * 256
    for R, C in ((1000, 64), (1025, 7), (4096, 4096), (1, 1), (64, 65), (65, 1000)):
        want = 3 * r256(-(-R // 64) * C * 8) + r256(4 * C)
        assert L.sv_variance_f32_workspace_size(R, C, 0) == want, (R, C)
        assert L.sv_variance_f32_workspace_size(R, C, -2) == want, (R, C)
    assert L.sv_variance_f32_workspace_size(0, 5, 0) == 0
    assert L.sv_variance_f32_workspace_size(5, 0, 0) == 0
    # long rows: 24 bytes per 16384-value chunk + 4 per row
    assert L.sv_variance_f32_workspace_size(3, 16385, 1) == 3 * 2 * 24 + 3 * 4
    assert L.sv_variance_f32_workspace_size(1, 8192 * 16384, 1) == 8192 * 24 + 4
    assert L.sv_variance_f32_workspace_size(1, 8192 * 16384 + 1, 1) == ctypes.c_size_t(-1).value


def test_sum_argument_errors(L):
    assert L.sv_tree_sum_f32(BAD, -1, BAD, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert b"n = -1" in L.sv_last_error_message()
    assert L.sv_tree_sum_f32(BAD, 10, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_tree_sum_f32(None, 10, BAD, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_tree_sum_f32(BAD, 10, BAD, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_tree_sum_f32(BAD, 10, BAD, ctypes.c_void_p(0x100000), 8, None) == SV_ERR_WORKSPACE
    assert L.sv_tree_sum_f32(BAD, 10, BAD, ctypes.c_void_p(0x100010), 1 << 20, None) == SV_ERR_WORKSPACE
    assert b"aligned" in L.sv_last_error_message()
    assert L.sv_tree_sum_f32(BAD, (1 << 36) + 1, BAD, None, 0, None) == SV_ERR_UNSUPPORTED
    # the double-word-carry sum shares the checks and the workspace rules
    assert L.sv_tree_sum_dw_f32(BAD, -1, BAD, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_tree_sum_dw_f32(BAD, 10, BAD, None, 0, None) == SV_ERR_WORKSPACE
    assert b"sv_tree_sum_dw_f32" in L.sv_last_error_message()
    assert L.sv_tree_sum_dw_f32(BAD, (1 << 36) + 1, BAD, None, 0, None) == SV_ERR_UNSUPPORTED


def test_variance_argument_errors(L):
    out = ctypes.c_void_p(0x2000)
    assert L.sv_variance_f32(BAD, -1, 4, 1, 0, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f32(BAD, 4, 4, 2, 0, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f32(BAD, 4, 4, 1, -1, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f32(BAD, 4, 4, 1, 0, None, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f32(None, 4, 4, 1, 0, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f32(BAD, 1 << 21, 1 << 20, 1, 0, out, None, None, 0, None) == SV_ERR_UNSUPPORTED
    # at most 2^36 values (every launch within 2^32 - 1 work-items)
    assert L.sv_variance_f32(BAD, (1 << 18) + 1, 1 << 18, 1, 0, out, None, None, 0, None) == SV_ERR_UNSUPPORTED
    assert L.sv_variance_f32_workspace_size((1 << 18) + 1, 1 << 18, 0) == ctypes.c_size_t(-1).value
    assert L.sv_variance_f32_workspace_size(1 << 18, 1 << 18, 0) != ctypes.c_size_t(-1).value
    # an empty set of slices is a successful no-op
    assert L.sv_variance_f32(None, 0, 5, 1, 0, None, None, None, 0, None) == 0
    # long slices need a workspace of the advertised size, 256-byte aligned
    assert L.sv_variance_f32(BAD, 2, 20000, 1, 0, out, None, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_f32(BAD, 2, 20000, 1, 0, out, None, ctypes.c_void_p(0x100000), 8, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_f32(BAD, 2, 20000, 1, 0, out, None, ctypes.c_void_p(0x100040), 4096, None) == \
        SV_ERR_WORKSPACE
    assert L.sv_variance_f32(BAD, 1, 8192 * 16384 + 1, 1, 0, out, None, None, 0, None) == SV_ERR_UNSUPPORTED
    # axis-0 columns beyond the per-column chunk trees (2^27 chunks of >= 64 rows)
    assert L.sv_variance_f32_workspace_size(1 << 34, 2, 0) == ctypes.c_size_t(-1).value
    assert L.sv_variance_f32_workspace_size(1 << 33, 2, 0) != ctypes.c_size_t(-1).value
    assert L.sv_variance_f32(BAD, 1 << 34, 2, 0, 0, out, None, BAD, 1 << 40, None) == SV_ERR_UNSUPPORTED


def test_adn_sizes_and_argument_errors(L):
    # counters (33024 bytes), then a 176-byte record (room for 21 folds) per
    # workgroup (up to 8192) and per group of 64 workgroups
    want = 33024 + 176 * (8192 + 128)
    assert L.sv_adn_sum_f32_workspace_size(0) == 0
    for n in (1, 4097, 10 ** 8, 4_294_966_784):
        assert L.sv_adn_sum_f32_workspace_size(n) == want
    assert L.sv_adn_sum_f32_workspace_size(4_294_966_785) == ctypes.c_size_t(-1).value
    assert L.sv_adn_sum_f32_workspace_size(-1) == ctypes.c_size_t(-1).value
    ws = ctypes.c_void_p(0x100000)
    assert L.sv_adn_sum_f32(BAD, -1, 3, BAD, ws, want, None) == SV_ERR_INVALID_ARGUMENT
    for fold in (0, 1, 22):
        assert L.sv_adn_sum_f32(BAD, 10, fold, BAD, ws, want, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_adn_sum_f32(BAD, 4_294_966_785, 3, BAD, ws, want, None) == SV_ERR_UNSUPPORTED
    assert b"capacity" in L.sv_last_error_message()
    assert L.sv_adn_sum_f32(BAD, 10, 3, None, ws, want, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_adn_sum_f32(None, 10, 3, BAD, ws, want, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_adn_sum_f32(BAD, 10, 3, BAD, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_adn_sum_f32(BAD, 10, 3, BAD, ws, want - 1, None) == SV_ERR_WORKSPACE
    assert L.sv_adn_sum_f32(BAD, 10, 3, BAD, ctypes.c_void_p(0x100080), want, None) == SV_ERR_WORKSPACE
    assert L.sv_set_tuning(b"adn_e", 16) == 0 and L.sv_set_tuning(b"adn_e", 8) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_set_tuning(b"adn_blocks", 1) == 0 and L.sv_set_tuning(b"adn_blocks", 8193) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_set_tuning(b"reset", 0) == 0


def test_f64_sizes_and_argument_errors(L):
    # same counter header as the float32 sum, 16-byte nodes
    assert L.sv_tree_sum_f64_workspace_size(0) == 0
    assert L.sv_tree_sum_f64_workspace_size(10 ** 8) == 33024 + 16 * (8192 + 128)
    assert L.sv_tree_sum_f64_workspace_size((1 << 35) + 1) == ctypes.c_size_t(-1).value
    assert L.sv_tree_sum_f64(BAD, -1, BAD, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_tree_sum_f64(ctypes.c_void_p(0x1004), 10, BAD, ctypes.c_void_p(0x100000), 1 << 20, None) == \
        SV_ERR_INVALID_ARGUMENT  # not 8-byte aligned
    assert L.sv_tree_sum_f64(BAD, 10, BAD, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_tree_sum_f64(BAD, (1 << 35) + 1, BAD, None, 0, None) == SV_ERR_UNSUPPORTED
    out = ctypes.c_void_p(0x2000)
    assert L.sv_variance_f64(BAD, 4, 4, 3, 0, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f64(BAD, 4, 4, 1, -1, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_f64(ctypes.c_void_p(0x1004), 4, 4, 1, 0, out, None, None, 0, None) == \
        SV_ERR_INVALID_ARGUMENT  # not 8-byte aligned
    assert L.sv_variance_f64(None, 0, 5, 1, 0, None, None, None, 0, None) == 0
    # workspace: none for single-workgroup slices; long slices three arrays
    # of 16 bytes per chunk per slice and 8 bytes per slice, each rounded to 256
    r256 = lambda b: (b + 255) // 256 * 256
    ws = L.sv_variance_f64_workspace_size
    assert ws(7, 16384, 1) == 0 and ws(1024, 9, 0) == 0 and ws(0, 5, 0) == 0
    assert ws(3, 16385, 1) == 3 * r256(3 * 3 * 16) + r256(3 * 8)
    assert ws(1025, 7, 0) == 3 * r256(9 * 7 * 16) + r256(7 * 8)
    assert ws(4096, 4096, 0) == 3 * r256(32 * 4096 * 16) + r256(4096 * 8)
    assert ws(1, 8192 * 8192, 1) == 3 * r256(8192 * 16) + r256(8)
    assert ws(1, 8192 * 8192 + 1, 1) == ctypes.c_size_t(-1).value
    assert ws((1 << 20) + 1, 1 << 19, 1) == ctypes.c_size_t(-1).value
    assert ws((1 << 18) + 1, 1 << 17, 0) == ctypes.c_size_t(-1).value  # above 2^35 values
    assert ws(1 << 18, 1 << 17, 0) != ctypes.c_size_t(-1).value
    assert ws(2, 3, 4) == ctypes.c_size_t(-1).value
    # long slices need it: missing, short and misaligned workspaces are refused
    assert L.sv_variance_f64(BAD, 2, 20000, 1, 0, out, None, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_f64(BAD, 2000, 3, 0, 0, out, None, ctypes.c_void_p(0x100000), 8, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_f64(BAD, 2000, 3, 0, 0, out, None, ctypes.c_void_p(0x100040), 1 << 20, None) == \
        SV_ERR_WORKSPACE
    assert L.sv_variance_f64(BAD, 1, 8192 * 8192 + 1, 1, 0, out, None, None, 0, None) == SV_ERR_UNSUPPORTED
    # axis-0 columns beyond the per-column chunk trees (2^27 chunks of >= 128 rows)
    assert ws(1 << 35, 2, 0) == ctypes.c_size_t(-1).value
    assert L.sv_variance_f64(BAD, 1 << 35, 2, 0, 0, out, None, BAD, 1 << 40, None) == SV_ERR_UNSUPPORTED


def test_complex_argument_errors_and_sizes(L):
    out = ctypes.c_void_p(0x2000)
    # axis 0: per-component variances (2*cols floats) + the float view's own
    # workspace ([1000, 128] along axis 0)
    assert L.sv_variance_c64_workspace_size(1000, 64, 0) == 512 + L.sv_variance_f32_workspace_size(1000, 128, 0)
    # axis 1: none up to 32768 values per row (one pass); above, the
    # per-component variances + the pair chunks' nodes (three 8-byte nodes
    # per 8192-value chunk per part, and 4 bytes per part); beyond 8192 such
    # chunks the split rows (8 bytes per value) + the float view's workspace
    assert L.sv_variance_c64_workspace_size(64, 1000, 1) == 0
    assert L.sv_variance_c64_workspace_size(3, 16385, 1) == 0
    assert L.sv_variance_c64_workspace_size(3, 32768, 1) == 0
    assert L.sv_variance_c64_workspace_size(3, 32769, 1) == 256 + 6 * 5 * 24 + 6 * 4
    n = 8192 * 8192 + 1
    assert L.sv_variance_c64_workspace_size(1, n, 1) == 256 + (n * 8 + 255) // 256 * 256 + \
        L.sv_variance_f32_workspace_size(2, n, 1)
    assert L.sv_variance_c64_workspace_size(2, 3, 5) == ctypes.c_size_t(-1).value
    assert L.sv_variance_c64(BAD, -1, 4, 1, 0, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_c64(BAD, 4, 4, 7, 0, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_c64(BAD, 4, 4, 1, -2, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_c64(ctypes.c_void_p(0x1004), 4, 4, 1, 0, out, None, None, 0, None) == \
        SV_ERR_INVALID_ARGUMENT  # not 8-byte aligned
    assert L.sv_variance_c64(BAD, 4, 40000, 1, 0, out, None, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_c64(None, 0, 4, 1, 0, None, None, None, 0, None) == 0


def test_tuning_knob_validation(L):
    assert L.sv_set_tuning(b"sum_load_path", 2) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_set_tuning(b"nope", 0) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_set_tuning(None, 0) == SV_ERR_INVALID_ARGUMENT
    for key, good, bad in ((b"sum_load_path", 1, 2), (b"sum_nt", 0, -1), (b"var_load_path", 2, 5),
                           (b"var_nt", 1, 2), (b"var_full_rows", 0, 2), (b"var_cols_once", 2, 3), (b"var_cols_once", 0, -1), (b"sum_e", 16, 64), (b"sum_depth", 4, 3), (b"sum_blocks", 8192, 0),
                           (b"sum_xcd", 1, 2), (b"var_xcd", 1, -1), (b"var_split", 0, 3), (b"var_split", 8, 16),
                           (b"var_lds_pad", 65536, 65537), (b"var_short_rows", 0, 2), (b"var_cols_one", 3, 4), (b"var_cols_one", 0, -1), (b"var_long_rows", 0, 2), (b"var_cols_short", 0, 3),
                           (b"launch_items", 1024, 1023), (b"launch_items", 0xffffffff, 1 << 32)):
        assert L.sv_set_tuning(key, good) == 0, key
        assert L.sv_set_tuning(key, bad) == SV_ERR_INVALID_ARGUMENT, key
    assert L.sv_set_tuning(b"sum_blocks", 8193) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_set_tuning(b"reset", 0) == 0


def test_no_device_is_reported(L):
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; the no-device path is checked on GPU-less hosts")
    ws = ctypes.c_void_p(0x100000)
    assert L.sv_tree_sum_f32(BAD, 10, BAD, ws, 1 << 20, None) == SV_ERR_NO_DEVICE
    assert L.sv_variance_f32(BAD, 4, 4, 1, 0, BAD, None, None, 0, None) == SV_ERR_NO_DEVICE
    assert L.sv_adn_sum_f32(BAD, 10, 3, BAD, ws, 1 << 21, None) == SV_ERR_NO_DEVICE


def test_python_binding_rejects_bad_tensors():
    import torch

    with pytest.raises(TypeError):
        sv.tree_sum([1.0, 2.0])
    with pytest.raises(TypeError):
        sv.var(torch.zeros(3, 3, dtype=torch.float16))
    with pytest.raises(ValueError):
        sv.var(torch.zeros(3, 3))  # CPU tensor: no fallback


def test_product_path_does_not_touch_the_oracle():
    # The package must not import, link or run anything under oracle/.
    pkg = os.path.join(ROOT, "stable_variance_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "sv_oracle" not in text, f


def test_variant_workspace_sizes_and_errors(L):
    # the variants beyond one workgroup: long rows take the chunk nodes of
    # the long-row path (24 bytes per chunk per row, 4 per row), long
    # columns the transposed matrix (256-byte rounded) first
    ws = L.sv_variance_variant_f32_workspace_size
    big = ctypes.c_size_t(-1).value
    assert ws(4, 16384, 1, 0) == 0 and ws(1024, 9, 0, 3) == 0 and ws(0, 70000, 1, 0) == 0
    assert ws(3, 20001, 1, 2) == 3 * 2 * 24 + 3 * 4
    assert ws(1025, 3, 0, 0) == 12544
    assert ws(20001, 3, 0, 5) == 240128 + 3 * 2 * 24 + 3 * 4
    assert ws(1, 8192 * 16384, 1, 1) == 8192 * 24 + 4
    assert ws(1, 8192 * 16384 + 1, 1, 1) == big
    assert ws(3, 5000, 1, 8) == 0 and ws(3, (1 << 22) + 1, 1, 8) == big  # the Kahan scan: no workspace
    assert ws(3, 5, 1, 9) == big and ws(3, 5, 2, 0) == big and ws(-1, 5, 1, 0) == big
    out = ctypes.c_void_p(0x2000)
    # the form without a workspace refuses the long slices; the other asks
    # for the workspace it lacks (both before any device call)
    assert L.sv_variance_variant_f32(BAD, 3, 20001, 1, 0, 2, out, None, None) == SV_ERR_UNSUPPORTED
    assert L.sv_variance_variant_ws_f32(BAD, 3, 20001, 1, 0, 2, out, None, None, 0, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_variant_ws_f32(BAD, 2000, 5, 0, 0, 2, out, None, BAD, 100, None) == SV_ERR_WORKSPACE
    assert L.sv_variance_variant_ws_f32(BAD, 2000, 5, 0, 0, 2, out, None, ctypes.c_void_p(0x1010), 1 << 20,
                                        None) == SV_ERR_WORKSPACE  # misaligned
    assert L.sv_variance_variant_ws_f32(BAD, 3, 5, 1, 0, 9, out, None, None, 0, None) == SV_ERR_INVALID_ARGUMENT
    assert L.sv_variance_variant_ws_f32(BAD, 1, 8192 * 16384 + 1, 1, 0, 0, out, None, BAD, 1 << 30,
                                        None) == SV_ERR_UNSUPPORTED
