"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact where the tree topology is mirrored (always, for this library);
NaN results only need to be NaN on both sides (payloads are not specified).
Every input is seeded; shapes span several tiles and ragged tails.
"""
import numpy as np
import pytest
import torch  # noqa: F401  (imported at collection: the first import is slow on a fresh box)

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def torch_dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stable_variance_amd import build as libbuild

    if libbuild.is_stale():
        libbuild.build()
    return torch, torch.device("cuda:0")


# Launch geometries the results must not depend on (knobs of sv_set_tuning).
SUM_GEOMETRIES = {
    "default": {},
    "e16": {"sum_e": 16},
    "depth4_few_blocks": {"sum_depth": 4, "sum_blocks": 64},
    "one_chunk_per_wave": {"sum_blocks": 8192, "sum_e": 16},
    "lane_loads_plain": {"sum_load_path": 1, "sum_nt": 0},
    "single_workgroup": {"sum_blocks": 1},
    "xcd_contiguous": {"sum_xcd": 1},
    "xcd_contiguous_few_blocks": {"sum_xcd": 1, "sum_blocks": 61},
}
VAR_GEOMETRIES = {
    "default": {},
    "lds_transpose_nt": {"var_load_path": 0, "var_nt": 1},
    "lds_transpose": {"var_load_path": 0, "var_nt": 0},
    "staged_transpose": {"var_load_path": 2},
    "split1": {"var_split": 1},
    "split2": {"var_split": 2},
    "split4": {"var_split": 4},
    "occupancy_capped": {"var_lds_pad": 20000},
    "split8": {"var_split": 8},
    "xcd_contiguous": {"var_xcd": 1},
    "xcd_contiguous_split1": {"var_xcd": 1, "var_split": 1},
    "short_rows_one_per_workgroup": {"var_short_rows": 0},
    "general_kernel_for_full_tiles": {"var_full_rows": 0},
    "general_kernel_split1": {"var_full_rows": 0, "var_split": 1},
}

# Axis-0 paths: one workgroup per column tile (rows up to var_cols_single_max)
# or row chunks of 16 * var_cols_waves rows in three launches.
COL_GEOMETRIES = {
    "default": {},
    "chunked_w4": {"var_cols_single_max": 0},
    "chunked_w8": {"var_cols_single_max": 0, "var_cols_waves": 8},
    "chunked_w16": {"var_cols_single_max": 0, "var_cols_waves": 16},
    "single_upto_64": {"var_cols_single_max": 64, "var_cols_waves": 8},
    "single_lane_per_column": {"var_cols_one": 0, "var_cols_short": 0},
    "single_four_columns_per_lane": {"var_cols_one": 2},
    "single_one_column_per_lane": {"var_cols_one": 3},
    "row_chunk_launches": {"var_cols_once": 0},
    "one_read_whatever_the_fill": {"var_cols_once": 2},
}


def _apply(knobs):
    import stable_variance_amd as sv

    sv.set_tuning("reset", 0)
    for k, v in knobs.items():
        sv.set_tuning(k, v)


@pytest.fixture(params=list(SUM_GEOMETRIES), ids=list(SUM_GEOMETRIES))
def sum_geometry(request, torch_dev):
    import stable_variance_amd as sv

    _apply(SUM_GEOMETRIES[request.param])
    yield request.param
    sv.set_tuning("reset", 0)


@pytest.fixture(params=list(COL_GEOMETRIES), ids=list(COL_GEOMETRIES))
def col_geometry(request, torch_dev):
    import stable_variance_amd as sv

    _apply(COL_GEOMETRIES[request.param])
    yield request.param
    sv.set_tuning("reset", 0)


@pytest.fixture(params=list(VAR_GEOMETRIES), ids=list(VAR_GEOMETRIES))
def var_geometry(request, torch_dev):
    import stable_variance_amd as sv

    _apply(VAR_GEOMETRIES[request.param])
    yield request.param
    sv.set_tuning("reset", 0)


def same_bits(a, b):
    a = np.asarray(a, np.float32).ravel()
    b = np.asarray(b, np.float32).ravel()
    if a.shape != b.shape:
        return False
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a.view(np.uint32) == b.view(np.uint32))))


def gpu_sum(torch_dev, x):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    r = sv.tree_sum(t)
    torch.cuda.synchronize()
    return np.float32(r.item())


def gpu_var(torch_dev, a, axis, ddof=0):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    v, m = sv.var(t, dim=axis, ddof=ddof, return_mean=True)
    torch.cuda.synchronize()
    return v.cpu().numpy(), m.cpu().numpy()


# ------------------------------------------------------------------ sums

def test_sum_printed_fixtures(torch_dev, sum_geometry):
    for x in (W.sum_thousandths(), W.sum_pm1e16()):
        assert same_bits(gpu_sum(torch_dev, x), oracle.tree_sum(x))
    assert gpu_sum(torch_dev, W.sum_pm1e16()) == 10000.0


def test_sum_permutations_same_bits(torch_dev):
    x, perms = W.sum_normal_perms()
    want = oracle.tree_sum(x)
    assert same_bits(gpu_sum(torch_dev, x), want)
    for p in perms:
        assert same_bits(gpu_sum(torch_dev, p), oracle.tree_sum(p))
        assert same_bits(gpu_sum(torch_dev, p), want)


SUM_SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 4095, 4096, 4097, 16383, 16384, 16385,
             65537, 1_000_003]


@pytest.mark.parametrize("n", SUM_SIZES)
def test_sum_sizes_random_and_adversarial(torch_dev, sum_geometry, n):
    rng = np.random.default_rng(n)
    for x in (rng.normal(0, 1, n).astype(np.float32), W.adversarial_values(n, n + 7),
              W.sum_cancelling_pairs(n, 0.02, seed=n)):
        assert same_bits(gpu_sum(torch_dev, x), oracle.tree_sum(x)), n


def test_sum_unaligned_pointer(torch_dev, sum_geometry):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    rng = np.random.default_rng(77)
    base = rng.normal(0, 1, 100_003).astype(np.float32)
    t = torch.from_numpy(base).to(dev)
    for off in (1, 2, 3):
        r = sv.tree_sum(t[off:])
        assert same_bits(r.item(), oracle.tree_sum(base[off:]))


def test_sum_zero_signs_and_specials(torch_dev):
    cases = [np.zeros(0, np.float32), np.full(5, -0.0, np.float32), np.full(16384, -0.0, np.float32),
             np.array([-0.0, 0.0, -0.0], np.float32), np.array([1, np.inf, 2], np.float32),
             np.array([np.inf, -np.inf], np.float32), np.array([np.nan, 1.0], np.float32),
             np.array([3e38, 3e38, -3e38], np.float32), np.array([1e-45, 1e-45, -2e-45, 1e-40], np.float32)]
    for x in cases:
        assert same_bits(gpu_sum(torch_dev, x), oracle.tree_sum(x)), x


def test_sum_workspace_left_zero_and_deterministic(torch_dev):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    x = W.sum_cancelling_pairs(3_000_000, 0.01, seed=5)
    t = torch.from_numpy(x).to(dev)
    r0 = sv.tree_sum(t).item()
    for _ in range(5):
        assert same_bits(sv.tree_sum(t).item(), r0)
    torch.cuda.synchronize()
    for (kind, _, _), ws in sv._workspaces.items():
        if kind == "sum":
            assert int(ws[:33024].count_nonzero().item()) == 0  # the ticket counters are back to 0
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r1 = sv.tree_sum(t)
    s.synchronize()
    assert same_bits(r1.item(), r0)


def test_concurrent_streams_own_workspaces(torch_dev):
    # two default-priority streams, each with its own workspaces (the binding
    # keeps one per stream), running sums and both variance paths at once
    import stable_variance_amd as sv

    torch, dev = torch_dev
    xs = [W.sum_cancelling_pairs(3_000_000, 0.01, seed=s) for s in (21, 22)]
    cols = [np.random.default_rng(s).normal(7e3, 2, (2500, 300)).astype(np.float32) for s in (23, 24)]
    rows = [np.random.default_rng(s).normal(-4e2, 1, (700, 3000)).astype(np.float32) for s in (25, 26)]
    dx = [torch.from_numpy(a).to(dev) for a in xs]
    dc = [torch.from_numpy(a).to(dev) for a in cols]
    dr = [torch.from_numpy(a).to(dev) for a in rows]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = [[], []]
    for rep in range(3):
        for k, st in enumerate(streams):
            with torch.cuda.stream(st):
                out[k].append((sv.tree_sum(dx[k]), sv.var(dc[k], dim=0), sv.var(dr[k], dim=1)))
    torch.cuda.synchronize()
    for k in range(2):
        want = (oracle.tree_sum(xs[k]), oracle.variance(cols[k], axis=0)[0], oracle.variance(rows[k], axis=1)[0])
        for s_, vc, vr in out[k]:
            assert same_bits(np.float32(s_.item()), want[0])
            assert same_bits(vc.cpu().numpy(), want[1]) and same_bits(vr.cpu().numpy(), want[2])


def test_sum_full_size_1e8(torch_dev):
    # 10^8 values (400 MB): 99% N(0,1), 1% large cancelling pairs, seed 3,
    # in the benchmark's launch configuration and in two others.
    import stable_variance_amd as sv

    x = W.sum_cancelling_pairs()
    want = oracle.tree_sum(x)
    for knobs in ({}, {"sum_e": 16, "sum_depth": 4, "sum_blocks": 512}, {"sum_blocks": 8192}):
        _apply(knobs)
        assert same_bits(gpu_sum(torch_dev, x), want), knobs
    sv.set_tuning("reset", 0)
    # float64 context: the 1e8 sum is ill-conditioned (large cancelling pairs)
    exact = float(oracle.exact_sum(x))
    assert abs(float(want) - exact) <= 1e-6 * abs(exact) + 1e-3


def test_sum_grouped_tiles(torch_dev):
    # Above 8192 tiles each workgroup combines a group of tiles: 1.5e8 values.
    x = np.random.default_rng(8).normal(0, 1, 150_000_000).astype(np.float32)
    assert same_bits(gpu_sum(torch_dev, x), oracle.tree_sum(x))


# ------------------------------------------------------------------ variance

def check_var(torch_dev, a, axis, ddof=0):
    v, m = gpu_var(torch_dev, a, axis, ddof)
    ov, om = oracle.variance(a, axis=axis, ddof=ddof)
    assert same_bits(v, ov), (a.shape, axis, ddof, np.flatnonzero(v.view(np.uint32) != ov.view(np.uint32))[:5])
    assert same_bits(m, om), (a.shape, axis, ddof)
    return v


@pytest.mark.parametrize("ddof", [0, 1])
def test_variance_page_datasets(torch_dev, var_geometry, ddof):
    for name, a, axis, _ in W.datasets_d1_d4():
        v = check_var(torch_dev, a, axis, ddof)
        v64 = oracle.var_f64(a, axis=axis, ddof=ddof)
        er = oracle.max_rel_err(oracle.variance(a, axis=axis, ddof=ddof, method=oracle.METHOD_REFERENCE)[0], v64)
        ek = oracle.max_rel_err(v, v64)
        assert ek <= 4 * U and ek <= er, (name, ddof, ek, er)


@pytest.mark.parametrize("c", [1.0, 1e10, 1e30, 1e38])
@pytest.mark.parametrize("ddof", [0, 1])
def test_variance_constants_exact_zero(torch_dev, c, ddof):
    a = W.constant(c)
    v = check_var(torch_dev, a, 0, ddof)
    assert np.all(v == 0.0)
    v = check_var(torch_dev, a.T.copy(), 1, ddof)
    assert np.all(v == 0.0)


def test_variance_4096_square(torch_dev, var_geometry):
    # the timing shape: bit-exact, within 4 * 2^-24 of the float64 variance
    # and no worse than the two-term reference formula
    a = W.c4_matrix()
    v = check_var(torch_dev, a, 1)
    v64 = oracle.var_f64(a, axis=1)
    ek = oracle.max_rel_err(v, v64)
    er = oracle.max_rel_err(oracle.variance(a, axis=1, method=oracle.METHOD_REFERENCE)[0], v64)
    assert ek <= 4 * U and ek <= er, (ek, er)


ROW_NS = [1, 2, 3, 5, 64, 255, 256, 257, 1000, 1023, 1024, 1025, 1500, 2048, 2049, 4095, 4096, 4097, 6000, 8192,
          8193, 10000, 16384]


@pytest.mark.parametrize("n", ROW_NS)
def test_variance_rows_shapes(torch_dev, var_geometry, n):
    rng = np.random.default_rng(n)
    rows = 37
    a = rng.normal(1e4, 1, (rows, n)).astype(np.float32)
    check_var(torch_dev, a, 1, 0)
    check_var(torch_dev, a, 1, 1)
    b = W.adversarial_values(rows * n, n).reshape(rows, n)
    check_var(torch_dev, b, 1, 0)


@pytest.mark.parametrize("shape", [(1000, 4), (4099, 1), (2050, 2), (513, 16), (777, 33), (3000, 100), (65, 500),
                                   (4096, 512), (301, 7), (100, 129), (257, 255), (1000, 250), (300, 6),
                                   (129, 18), (200, 130)])
def test_variance_many_short_rows(torch_dev, var_geometry, shape):
    # short rows share waves (a row per group of S lanes): partial last
    # workgroups, odd widths (scalar loads), even widths (8-byte loads),
    # widths below and above each tile
    rng = np.random.default_rng(shape[0] + 17 * shape[1])
    a = rng.normal(3e3, 1.5, shape).astype(np.float32)
    check_var(torch_dev, a, 1, 0)
    check_var(torch_dev, a, 1, 1)
    b = W.adversarial_values(shape[0] * shape[1], shape[1]).reshape(shape)
    check_var(torch_dev, b, 1, 0)


def special_rows(n, seed):
    """Rows with NaN, +Inf, -Inf, both infinities, values whose differences
    or squares overflow, and subnormal-only rows, at seeded positions."""
    rng = np.random.default_rng(seed)
    a = rng.normal(5.0, 2.0, (8, n)).astype(np.float32)
    pos = lambda: int(rng.integers(0, n))
    a[0, pos()] = np.nan
    a[1, pos()] = np.inf
    a[2, pos()] = -np.inf
    a[3, pos()] = np.inf
    a[3, pos()] = -np.inf
    a[4, :] = rng.choice(np.float32([3e38, -3e38]), n)          # d = x - x0 and d^2 overflow
    a[5, :] = (rng.integers(-50, 50, n) * np.float32(2.0 ** -149)).astype(np.float32)
    a[6, :] = np.float32(1e38)
    a[6, pos()] = np.float32(-1e38)                            # one far value: d^2 = inf
    a[7, :] = np.nan
    return a


@pytest.mark.parametrize("n", [3, 64, 1000, 4096, 10000, 20000])
def test_variance_specials_rows(torch_dev, var_geometry, n):
    a = special_rows(n, seed=n)
    for ddof in (0, 1):
        check_var(torch_dev, a, 1, ddof)


@pytest.mark.parametrize("R", [3, 64, 1000, 1500])
def test_variance_specials_cols(torch_dev, col_geometry, R):
    a = np.ascontiguousarray(special_rows(R, seed=R + 7).T)
    check_var(torch_dev, a, 0, 0)


COL_RS = [1, 2, 3, 4, 5, 16, 17, 64, 65, 100, 128, 129, 256, 257, 512, 513, 1000, 1024]


@pytest.mark.parametrize("R", COL_RS)
def test_variance_cols_shapes(torch_dev, col_geometry, R):
    rng = np.random.default_rng(R)
    for C in (1, 63, 64, 65, 200):
        a = rng.normal(-3e3, 2, (R, C)).astype(np.float32)
        check_var(torch_dev, a, 0, 0)
        check_var(torch_dev, a, 0, 2)
    b = W.adversarial_values(R * 70, R).reshape(R, 70)
    check_var(torch_dev, b, 0, 0)


def test_variance_empty_slices(torch_dev):
    v, m = gpu_var(torch_dev, np.zeros((3, 0), np.float32), 1)
    assert np.all(np.isnan(v)) and np.all(np.isnan(m))
    v, m = gpu_var(torch_dev, np.zeros((0, 4), np.float32), 0)
    assert np.all(np.isnan(v)) and v.shape == (4,)


def test_variance_unsupported_shape_leaves_output(torch_dev):
    # Rejected on the host (a slice of more than 8192 chunks) before any
    # access: the small buffer is never read and the output is untouched.
    import ctypes

    import stable_variance_amd as sv

    torch, dev = torch_dev
    L = sv.capi()
    x = torch.zeros(16, device=dev)
    out = torch.full((1,), 7.0, device=dev)
    big = 8192 * 16384 + 1
    st = L.sv_variance_f32(x.data_ptr(), 1, big, 1, 0, out.data_ptr(), None, None, 0, None)
    assert st == 5
    assert torch.all(out == 7.0)
    assert L.sv_variance_f32_workspace_size(1, big, 1) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("n", [16385, 20001, 32768, 32769, 50002, 65536])
@pytest.mark.parametrize("long_rows", [1, 0])
def test_variance_long_rows_one_workgroup(torch_dev, n, long_rows):
    # 256+ rows of 16385..65536 values: one workgroup of 16 waves per row
    # (32 or 64 values per lane), or the chunked path; odd lengths load
    # without 16-byte vectors
    import stable_variance_amd as sv

    sv.set_tuning("var_long_rows", long_rows)
    try:
        rng = np.random.default_rng(n + long_rows)
        a = rng.normal(-2e4, 5, (300, n)).astype(np.float32)
        check_var(torch_dev, a, 1, 0)
        check_var(torch_dev, a, 1, 2)
    finally:
        sv.set_tuning("reset", 0)


LONG_ROW_NS = [16385, 20000, 32768, 50001, 100003]


@pytest.mark.parametrize("n", LONG_ROW_NS)
def test_variance_long_rows(torch_dev, n):
    # axis-1 slices beyond one workgroup: chunked two-pass path
    rng = np.random.default_rng(n)
    a = rng.normal(5e3, 3, (5, n)).astype(np.float32)
    check_var(torch_dev, a, 1, 0)
    check_var(torch_dev, a, 1, 3)
    b = W.adversarial_values(3 * n, n).reshape(3, n)
    check_var(torch_dev, b, 1, 0)
    c = np.ascontiguousarray(a[:, 1:])  # misaligned rows (n-1 values, odd row stride)
    check_var(torch_dev, c, 1, 0)


@pytest.mark.parametrize("R", [1025, 2048, 3000, 5000])
def test_variance_long_cols(torch_dev, col_geometry, R):
    rng = np.random.default_rng(R)
    for C in (1, 64, 130):
        a = rng.normal(-7e3, 0.5, (R, C)).astype(np.float32)
        check_var(torch_dev, a, 0, 0)
        check_var(torch_dev, a, 0, 1)
    b = W.adversarial_values(R * 33, R).reshape(R, 33)
    check_var(torch_dev, b, 0, 0)


@pytest.mark.parametrize("R,C", [(4096, 1000), (2000, 4100), (5000, 257), (300, 4096), (70000, 12), (1, 3000),
                                 (100000, 4), (50000, 16), (20000, 7), (8193, 2), (30000, 1), (9000, 40),
                                 (40000, 130), (70000, 65), (20000, 8), (300000, 8), (33000, 20), (70000, 24),
                                 (9000, 32)])
def test_variance_cols_wide(torch_dev, col_geometry, R, C):
    # several column blocks with a ragged last block (16-byte loads of four
    # columns when C % 4 == 0, one column per lane otherwise) and ragged chunks;
    # narrow matrices take 8 or 32 row groups per wave in the chunks (20..32
    # and 8 columns; 35-37 chunks at [70000, 24] and [300000, 8], beyond the
    # chunk count whose m each workgroup forms itself)
    rng = np.random.default_rng(R + C)
    a = rng.normal(2.5e4, 4, (R, C)).astype(np.float32)
    check_var(torch_dev, a, 0, 0)
    check_var(torch_dev, a, 0, 5)
    b = W.adversarial_values(R * C, R + 1).reshape(R, C)
    check_var(torch_dev, b, 0, 0)


@pytest.mark.parametrize("R,C", [(100, 140_000), (400, 40_000), (65, 140_000), (1000, 36_000), (77, 300_000),
                                 (200, 40_000), (129, 4096), (1024, 64), (65, 8), (16, 140_000), (600, 9001),
                                 (900, 8193), (300, 3), (100, 140_001), (200, 40_001), (400, 40_001)])
@pytest.mark.parametrize("mode", [1, 2, 3])
def test_variance_cols_one_launch(torch_dev, R, C, mode):
    # whole columns in one launch: every (G, W) choice of four columns per
    # lane (16-byte loads, or four 4-byte loads for odd widths) and of one
    import stable_variance_amd as sv

    sv.set_tuning("var_cols_one", mode)
    try:
        _cols_one_cases(torch_dev, R, C)
    finally:
        sv.set_tuning("reset", 0)


def _cols_one_cases(torch_dev, R, C):
    rng = np.random.default_rng(R * 3 + C)
    a = rng.normal(8e3, 3, (R, C)).astype(np.float32)
    check_var(torch_dev, a, 0, 0)
    check_var(torch_dev, a, 0, 1)
    b = W.adversarial_values(R * C, R + 5).reshape(R, C)
    check_var(torch_dev, b, 0, 0)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 9, 15, 16])
def test_variance_short_cols_wide(torch_dev, R):
    # columns of at most 15 rows, four per lane, every tree in-lane (16: the
    # lane-per-column kernel)
    rng = np.random.default_rng(R + 77)
    for C in (4, 8, 1028, 250_000):
        a = rng.normal(3e3, 2, (R, C)).astype(np.float32)
        check_var(torch_dev, a, 0, 0)
        check_var(torch_dev, a, 0, 1)
        check_var(torch_dev, a, 0, 5)
    b = W.adversarial_values(R * 4096, R + 3).reshape(R, 4096)
    check_var(torch_dev, b, 0, 0)


@pytest.mark.parametrize("R,C,waves", [(500_000, 129, 16), (1_100_000, 7, 16), (1_050_000, 65, 16),
                                       (600_000, 65, 4)])
def test_variance_cols_many_chunks(torch_dev, R, C, waves):
    # 1025..4096 chunks per column: 64 chunk nodes per lane of a wave per
    # column; beyond (4102 chunks, and 9375 chunks of 64 rows at four
    # waves): runs of 64*P nodes per lane merged by a binary counter
    import stable_variance_amd as sv

    rng = np.random.default_rng(R + C)
    a = rng.normal(-1e3, 3, (R, C)).astype(np.float32)
    sv.set_tuning("var_cols_waves", waves)
    try:
        check_var(torch_dev, a, 0, 0)
    finally:
        sv.set_tuning("reset", 0)


@pytest.mark.parametrize("R,C", [(4096, 4096), (1025, 256), (3000, 4100), (4095, 260), (2048, 8192), (1088, 4),
                                 (4096, 1000), (2000, 10), (2049, 17), (1025, 1), (3999, 33)])
@pytest.mark.parametrize("once", [1, 2])
def test_variance_cols_one_read(torch_dev, R, C, once):
    # Columns of 1025..4096 rows in one launch that reads the input once
    # (once=2 forces it; once=1 lets the grid's fill choose): 2048 and 4096
    # rows (every wave full), ragged lengths (only the reached waves, a
    # partial last one), a partial last block of 16 columns, one-lane and
    # narrow widths, and widths that are not a multiple of 4.
    rng = np.random.default_rng(R + C)
    a = rng.normal(-2e3, 5, (R, C)).astype(np.float32)
    import stable_variance_amd as sv

    sv.set_tuning("var_cols_once", once)
    try:
        for ddof in (0, 1):
            check_var(torch_dev, a, 0, ddof)
        v = check_var(torch_dev, np.full((R, C), np.float32(1e38)), 0, 0)
        assert np.all(v == 0.0)
    finally:
        sv.set_tuning("reset", 0)


def test_variance_4096_square_axis0(torch_dev, col_geometry):
    a = W.c4_matrix()
    v = check_var(torch_dev, a, 0)
    assert oracle.max_rel_err(v, oracle.var_f64(a, axis=0)) <= 4 * U


def test_variance_cols_datasets_and_constants(torch_dev, col_geometry):
    for name, a, axis, _ in W.datasets_d1_d4():
        check_var(torch_dev, a, axis)
    for c in (1.0, 1e10, 1e38):
        for R in (3, 1000, 3000):
            v = check_var(torch_dev, np.full((R, 20), np.float32(c)), 0, 1)
            assert np.all(v == 0.0)


def test_variance_single_long_row(torch_dev):
    # one slice of 2^22 + 3 values (256 chunks) and its constant version
    rng = np.random.default_rng(22)
    n = (1 << 22) + 3
    a = rng.normal(1e6, 1, (1, n)).astype(np.float32)
    check_var(torch_dev, a, 1, 0)
    v = check_var(torch_dev, np.full((1, n), np.float32(1e38)), 1, 0)
    assert v[0] == 0.0


@pytest.mark.parametrize("n", [(1 << 24) + 1, (1 << 25) + 7])
@pytest.mark.parametrize("axis", [1, 0])
def test_variance_slices_beyond_2_24(torch_dev, n, axis):
    # Step 2 divides by fl(n): above 2^24 it rounds (2^24 + 1 -> 2^24, and
    # 2^25 + 7 -> 2^25 + 8).  The axis-1 slice of 2^25 + 7 values has 2049
    # chunks, so its top trees take 32 chunk nodes per thread; the axis-0
    # column takes the per-column chunk trees of one column.
    assert float(np.float32(n)) != n
    rng = np.random.default_rng(n % 1000)
    a = rng.normal(3e3, 2, n).astype(np.float32)
    a = a[None, :] if axis == 1 else a[:, None]
    for ddof in (0, 1):
        v = check_var(torch_dev, a, axis, ddof)
        v64 = oracle.var_f64(a, axis=axis, ddof=ddof)
        assert oracle.max_rel_err(v, v64) <= 4 * U


# ------------------------------------------------------------------ complex64

def gpu_var_c64(torch_dev, z, axis, ddof=0):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    t = torch.from_numpy(np.ascontiguousarray(z, np.complex64)).to(dev)
    v, m = sv.var(t, dim=axis, ddof=ddof, return_mean=True)
    torch.cuda.synchronize()
    return v.cpu().numpy(), m.cpu().numpy()


def check_var_c64(torch_dev, z, axis, ddof=0):
    v, m = gpu_var_c64(torch_dev, z, axis, ddof)
    ov, om = oracle.variance_complex(z, axis=axis, ddof=ddof)
    assert same_bits(v, ov), (z.shape, axis, ddof)
    assert same_bits(m.view(np.float32), om.view(np.float32)), (z.shape, axis, ddof)
    return v


def test_complex_printed_values(torch_dev):
    # Method page §2/§3: the complex check and the complex identical-values row.
    from conftest import read_kv

    g = read_kv("complex_check.txt")
    z = np.array([complex(s.replace(" ", "")) for s in g["values"].split(",")], np.complex64)[None, :]
    v = check_var_c64(torch_dev, z, 1)
    assert v[0] == float(g["variance"])
    zc = np.full((1, int(g["identical_count"])), complex(g["identical"]), np.complex64)
    v = check_var_c64(torch_dev, zc, 1)
    assert v[0] == float(g["identical_variance"])


# rows of up to 32768 values take the one-pass kernel (odd widths: per-lane
# scalar loads; 16385 and up: 32 values per lane); longer rows the staged split
@pytest.mark.parametrize("shape", [(64, 1000), (3, 4096), (5, 20000), (1000, 64), (2000, 3), (1, 1), (7, 2),
                                   (9, 257), (4, 1025), (6, 2047), (3, 5000), (2, 8191), (2, 8192), (2, 8193),
                                   (3, 12001), (2, 16384), (2, 16385), (3, 20001), (40, 24576), (2, 32767),
                                   (2, 32768), (2, 32769),
                                   (11, 0), (3000, 4), (777, 9), (500, 30), (260, 64), (129, 200), (70, 512)])
@pytest.mark.parametrize("axis", [0, 1])
def test_complex_shapes(torch_dev, shape, axis):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    re = rng.normal(1e4, 1, shape)
    im = rng.normal(-3e3, 0.5, shape)
    z = (re + 1j * im).astype(np.complex64)
    check_var_c64(torch_dev, z, axis, 0)
    check_var_c64(torch_dev, z, axis, 1)


def test_complex_rows_specials(torch_dev):
    # NaN / Inf / overflow in one part only: the other part's variance is
    # unaffected and the sum follows IEEE addition
    a = special_rows(3000, seed=5)
    b = np.random.default_rng(6).normal(0, 1, a.shape).astype(np.float32)
    for re, im in ((a, b), (b, a)):
        z = np.empty(a.shape, np.complex64)  # parts set directly: 1j * inf would be nan + inf j
        z.real, z.imag = re, im
        check_var_c64(torch_dev, z, 1)


def test_complex_then_sum_share_nothing(torch_dev):
    # a scratch-using variance between two sums must not disturb the sums'
    # ticket counters
    x = W.sum_cancelling_pairs(2_000_000, 0.01, seed=9)
    want = oracle.tree_sum(x)
    assert same_bits(gpu_sum(torch_dev, x), want)
    z = (np.random.default_rng(1).normal(0, 1, (3, 30000)) * (1 + 1j)).astype(np.complex64)
    check_var_c64(torch_dev, z, 1)
    assert same_bits(gpu_sum(torch_dev, x), want)


# ------------------------------------------------------------------ ablation variants

GPU_VARIANTS = {"kernel": 0, "kernel_comp_y": 1, "reference": 2, "naive": 3, "shift_plain_no2t": 4,
                "shift_plain_2t": 5, "noshift_comp_2t": 6, "shift_comp_no2t": 7, "shift_kahan_no2t": 8}


@pytest.mark.parametrize("name", list(GPU_VARIANTS))
def test_variants_against_oracle(torch_dev, name):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    code = GPU_VARIANTS[name]
    cases = [(a, ax) for _, a, ax, _ in W.datasets_d1_d4()]
    rng = np.random.default_rng(code)
    cases += [(rng.normal(1e4, 1, (9, 4096)).astype(np.float32), 1), (rng.normal(0, 3, (5, 10000)).astype(np.float32), 1),
              (rng.normal(-5, 1, (700, 70)).astype(np.float32), 0), (W.adversarial_values(6 * 300, code).reshape(6, 300), 1),
              (np.full((1, 3), np.float32(1e38)), 1), (W.constant(1e30), 0),
              (rng.normal(7, 2, (4, 1500)).astype(np.float32), 1),  # a wave wholly past the row
              (np.full((3, 5), np.float32(-0.0)), 1), (np.full((5, 3), np.float32(-0.0)), 0),  # all -0 slices
              (np.array([[0.0, 1.0, 2.0 ** 24, 1.0]], np.float32), 1)]  # separates the two local means
    for a, ax in cases:
        for ddof in (0, 1):
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            v, m = sv.var_variant(t, code, dim=ax, ddof=ddof, return_mean=True)
            torch.cuda.synchronize()
            ov, om = oracle.variance(a, axis=ax, ddof=ddof, method=code)
            assert same_bits(v.cpu().numpy(), ov), (name, a.shape, ax, ddof)
            assert same_bits(m.cpu().numpy(), om), (name, a.shape, ax, ddof)


@pytest.mark.parametrize("name", [n for n in GPU_VARIANTS if n != "shift_kahan_no2t"])
def test_variants_on_long_slices(torch_dev, name):
    # slices longer than one workgroup holds: rows of more than 16384 values
    # in 16384-value chunks (aligned nodes of the tree), columns of more than
    # 1024 rows transposed into the workspace and reduced as rows (in one
    # workgroup up to 16384 rows, in chunks beyond); aligned, odd and
    # misaligned widths; bit for bit against the oracle's variant
    import stable_variance_amd as sv

    torch, dev = torch_dev
    code = GPU_VARIANTS[name]
    rng = np.random.default_rng(code + 100)
    cases = [(rng.normal(1e4, 1, (3, 20001)).astype(np.float32), 1), (rng.normal(-7, 2, (2, 40000)).astype(np.float32), 1),
             (rng.normal(3e3, 5, (1, 70003)).astype(np.float32), 1), (rng.normal(5, 1, (1500, 7)).astype(np.float32), 0),
             (rng.normal(-2e4, 3, (2000, 64)).astype(np.float32), 0), (rng.normal(9, 4, (20001, 3)).astype(np.float32), 0),
             (W.adversarial_values(2 * 33000, code + 7).reshape(2, 33000), 1),
             (W.adversarial_values(1100 * 5, code + 8).reshape(1100, 5), 0)]
    for a, ax in cases:
        for ddof in (0, 1):
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            v, m = sv.var_variant(t, code, dim=ax, ddof=ddof, return_mean=True)
            torch.cuda.synchronize()
            ov, om = oracle.variance(a, axis=ax, ddof=ddof, method=code)
            assert same_bits(v.cpu().numpy(), ov), (name, a.shape, ax, ddof)
            assert same_bits(m.cpu().numpy(), om), (name, a.shape, ax, ddof)
        if ax == 1 and a.shape[1] % 4 == 0:  # a misaligned base: per-value loads
            buf = torch.zeros(a.size + 1, dtype=torch.float32, device=dev)
            buf[1:] = torch.from_numpy(a.reshape(-1)).to(dev)
            v = sv.var_variant(buf[1:].view(a.shape), code, dim=ax)
            torch.cuda.synchronize()
            assert same_bits(v.cpu().numpy(), oracle.variance(a, axis=ax, method=code)[0]), (name, a.shape)
    if code == 0:  # variant 0 is the method: the main entry point's bits
        a = torch.from_numpy(cases[0][0]).to(dev)
        assert torch.equal(sv.var_variant(a, 0, dim=1).view(torch.int32), sv.var(a, dim=1).view(torch.int32))


@pytest.mark.parametrize("shape,axis", [((3, 70000), 1), ((2, 5001), 1), ((130, 4097), 1), ((3000, 70), 0),
                                        ((1, 64), 1), ((65, 1), 0), ((4096, 4096), 1)])
def test_kahan_scan_variant_long_and_ragged_slices(torch_dev, shape, axis):
    # The Kahan-scan row has no one-workgroup limit: slices beyond 16384
    # values, widths that are not a multiple of 4 (per-value loads), a partial
    # last wave of 64 slices, the chunk counter past 64 chunks, and the
    # timing shape.  Bit for bit against the oracle's loop.
    import stable_variance_amd as sv

    torch, dev = torch_dev
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    a = rng.normal(5e3, 3, shape).astype(np.float32)
    if shape == (4096, 4096):
        a = W.c4_matrix()
    t = torch.from_numpy(a).to(dev)
    for ddof in (0, 1):
        v, m = sv.var_variant(t, "shift_kahan_no2t", dim=axis, ddof=ddof, return_mean=True)
        torch.cuda.synchronize()
        ov, om = oracle.variance(a, axis=axis, ddof=ddof, method=oracle.METHOD_SHIFT_KAHAN_NO2T)
        assert same_bits(v.cpu().numpy(), ov), (shape, axis, ddof)
        assert same_bits(m.cpu().numpy(), om), (shape, axis, ddof)


def test_variant_zero_matches_the_main_entry_point(torch_dev):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    a = torch.from_numpy(W.c4_matrix()).to(dev)
    v0 = sv.var_variant(a, "kernel", dim=1)
    v1 = sv.var(a, dim=1)
    torch.cuda.synchronize()
    assert torch.equal(v0.view(torch.int32), v1.view(torch.int32))


# ------------------------------------------------------------------ double-word carries

def gpu_sum_dw(torch_dev, x, offset=0):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    x = np.ascontiguousarray(x, np.float32)
    if offset:
        buf = torch.zeros(x.size + offset, dtype=torch.float32, device=dev)
        buf[offset:] = torch.from_numpy(x).to(dev)
        t = buf[offset:]
    else:
        t = torch.from_numpy(x).to(dev)
    r = sv.tree_sum(t, carry="dw")
    torch.cuda.synchronize()
    return np.float32(r.item())


DW_GEOMETRIES = {"default": {}, "e16_few_blocks": {"sum_e": 16, "sum_blocks": 64}, "single_workgroup": {"sum_blocks": 1},
                 "xcd_contiguous": {"sum_xcd": 1, "sum_blocks": 1000}}


@pytest.mark.parametrize("knobs", list(DW_GEOMETRIES.values()), ids=list(DW_GEOMETRIES))
def test_sum_dw_sizes_and_specials(torch_dev, knobs):
    import stable_variance_amd as sv

    _apply(knobs)
    try:
        for n in (0, 1, 2, 3, 63, 2048, 2049, 65536 + 7, 1_000_003):
            for x in (W.adversarial_values(n, seed=n), W.sum_cancelling_pairs(n, 0.3, seed=n + 1)):
                assert same_bits(gpu_sum_dw(torch_dev, x), oracle.tree_sum_dw(x)), (knobs, n)
                assert same_bits(gpu_sum_dw(torch_dev, x, offset=1), oracle.tree_sum_dw(x)), (knobs, n, "unaligned")
        for special in ([np.inf, 1.0, -3.0], [np.inf, -np.inf, 2.0], [np.nan, 1.0], [3e38, 3e38, -1.0]):
            x = np.concatenate([np.random.default_rng(3).standard_normal(5000).astype(np.float32),
                                np.array(special, np.float32)])
            assert same_bits(gpu_sum_dw(torch_dev, x), oracle.tree_sum_dw(x)), special
    finally:
        sv.set_tuning("reset", 0)


def test_sum_dw_cancelling_sets_and_full_workload(torch_dev):
    for n, frac, seed in ((1 << 16, 0.3, 1), (1 << 20, 0.1, 1), (1 << 22, 0.05, 0)):
        x = W.sum_cancelling_pairs(n, frac, seed=seed)
        assert same_bits(gpu_sum_dw(torch_dev, x), oracle.tree_sum_dw(x)), (n, frac, seed)
    x = W.sum_cancelling_pairs()
    want = oracle.tree_sum_dw(x)
    assert same_bits(gpu_sum_dw(torch_dev, x), want)
    assert want == oracle.round_f32(oracle.exact_sum(x))   # 3735.104, correctly rounded


# ---------------------------------------------------------------- batched launches

# Every shape class with each grid cut into launches of at most 1024 or 4096
# work-items (sv_set_tuning "launch_items"): the batched launches, with their
# first-workgroup offsets, that only the largest inputs take at the default
# limit of 2^32 - 1, here on small inputs and bit for bit against the oracle.
BATCH_F32 = [((2000, 3), 1), ((3000, 300), 1), ((300, 3000), 1), ((260, 17000), 1), ((3, 20000), 1),
             ((3, 2000), 0), ((40, 700), 0), ((700, 70), 0), ((700, 1030), 0), ((1500, 300), 0), ((3000, 40), 0),
             ((5000, 33), 0), ((2049, 300), 0), ((520, 8192), 0), ((9000, 8), 0), ((9000, 24), 0)]


@pytest.mark.parametrize("items", [1024, 4096])
@pytest.mark.parametrize("shape,axis", BATCH_F32)
def test_variance_batched_launches(torch_dev, shape, axis, items):
    import stable_variance_amd as sv

    rng = np.random.default_rng(shape[0] * 7 + shape[1] + items)
    a = rng.normal(-3e3, 11, shape).astype(np.float32)
    once = [1, 2] if axis == 0 and 1024 < shape[0] <= 4096 else [1]
    for o in once:
        sv.set_tuning("reset", 0)
        sv.set_tuning("launch_items", items)
        sv.set_tuning("var_cols_once", o)
        try:
            check_var(torch_dev, a, axis, 1)
        finally:
            sv.set_tuning("reset", 0)


@pytest.mark.parametrize("items", [1024, 4096])
def test_complex_and_variants_batched_launches(torch_dev, items):
    import stable_variance_amd as sv

    rng = np.random.default_rng(items)
    sv.set_tuning("launch_items", items)
    try:
        for shape in ((3000, 5), (900, 700), (300, 2000)):
            z = (rng.normal(size=shape) + 1j * rng.normal(size=shape)).astype(np.complex64) + (50 + 20j)
            for axis in (0, 1):
                check_var_c64(torch_dev, z, axis)
        torch, dev = torch_dev
        a = rng.normal(7e2, 3, (1100, 900)).astype(np.float32)
        for code in (0, 2, 4, 6):  # the variant codes are the oracle's method numbers
            for axis in (0, 1):
                b = a if axis == 1 else np.ascontiguousarray(a[:1000])
                v = sv.var_variant(torch.from_numpy(b).to(dev), code, dim=axis)
                torch.cuda.synchronize()
                assert same_bits(v.cpu().numpy(), oracle.variance(b, axis=axis, method=code)[0]), (code, axis, items)
    finally:
        sv.set_tuning("reset", 0)


@pytest.mark.parametrize("R", [1, 5, 64, 1000, 16385, 70000, 1 << 21])
def test_variance_single_column_as_a_row(torch_dev, R):
    # a [R, 1] column is read as the row [1, R] (the same values in the same
    # order): bit for bit the oracle's column, and the row's
    rng = np.random.default_rng(R)
    a = rng.normal(3e3, 7, (R, 1)).astype(np.float32)
    for ddof in (0, 1):
        v = check_var(torch_dev, a, 0, ddof)
        assert same_bits(v, check_var(torch_dev, np.ascontiguousarray(a.T), 1, ddof))


@pytest.mark.parametrize("R", [4097, 8192, 8193, 50001, 1 << 20, 3_000_001])
@pytest.mark.parametrize("pairs", [1, 0])
def test_variance_two_columns(torch_dev, R, pairs):
    # [R, 2] along axis 0: one row of R pairs in chunks (two interleaved
    # slices), or the column chunks; aligned even, odd and misaligned
    import stable_variance_amd as sv

    torch, dev = torch_dev
    rng = np.random.default_rng(R + pairs)
    a = rng.normal(-6e3, 13, (R, 2)).astype(np.float32)
    sv.set_tuning("var_cols_pairs", pairs)
    try:
        for ddof in (0, 1):
            check_var(torch_dev, a, 0, ddof)
        buf = torch.zeros(2 * R + 1, dtype=torch.float32, device=dev)
        buf[1:] = torch.from_numpy(a.reshape(-1)).to(dev)
        v = sv.var(buf[1:].view(R, 2), dim=0)
        torch.cuda.synchronize()
        assert same_bits(v.cpu().numpy(), oracle.variance(a, axis=0)[0])
    finally:
        sv.set_tuning("reset", 0)


@pytest.mark.parametrize("shape,axis", [((3, 32769), 1), ((2, 100_001), 1), ((1, 1 << 21), 1), ((70, 40_000), 1),
                                        ((1 << 20, 1), 0), ((50001, 1), 0)])
def test_complex_long_rows_and_single_column(torch_dev, shape, axis):
    # complex rows beyond 32768 values take the pair chunks (parts split in
    # registers); a single complex column is a [R, 2] float matrix along axis 0
    rng = np.random.default_rng(shape[0] + shape[1])
    z = (rng.normal(3, 2, shape) + 1j * rng.normal(-1, 5, shape)).astype(np.complex64) + (4e3 - 2e3j)
    for ddof in (0, 1):
        check_var_c64(torch_dev, z, axis, ddof)
