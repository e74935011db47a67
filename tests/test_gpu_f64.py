"""GPU parity of the float64 path (the method with every operation in
double) against the binary64 oracle: bit-exact, NaN as NaN."""
import numpy as np
import pytest
import torch  # noqa: F401  (imported at collection: the first import is slow on a fresh box)

import oracle
import workloads as W

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


def same_bits64(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    if a.shape != b.shape:
        return False
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a.view(np.uint64) == b.view(np.uint64))))


def gpu_sum64(torch_dev, x, offset=0):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    x = np.ascontiguousarray(x, np.float64)
    if offset:
        buf = torch.zeros(x.size + offset, dtype=torch.float64, device=dev)
        buf[offset:] = torch.from_numpy(x).to(dev)
        t = buf[offset:]
    else:
        t = torch.from_numpy(x).to(dev)
    r = sv.tree_sum(t)
    torch.cuda.synchronize()
    return np.float64(r.item())


def check_var64(torch_dev, a, axis, ddof=0):
    import stable_variance_amd as sv

    torch, dev = torch_dev
    v, m = sv.var(torch.from_numpy(np.ascontiguousarray(a, np.float64)).to(dev), dim=axis, ddof=ddof,
                  return_mean=True)
    torch.cuda.synchronize()
    ov, om = oracle.variance_f64(a, axis=axis, ddof=ddof)
    v, m = v.cpu().numpy(), m.cpu().numpy()
    assert same_bits64(v, ov), (a.shape, axis, ddof, np.flatnonzero(v.view(np.uint64) != ov.view(np.uint64))[:5])
    assert same_bits64(m, om), (a.shape, axis, ddof)
    return v


@pytest.mark.parametrize("n", [0, 1, 2, 3, 1023, 1024, 1025, 4096 + 3, 65537, 1_000_003])
def test_sum64_sizes(torch_dev, n):
    rng = np.random.default_rng(n)
    for x in (rng.standard_normal(n) * np.exp2(rng.integers(-300, 300, n)),
              W.adversarial_values(n, seed=n).astype(np.float64),
              W.sum_cancelling_pairs(n, 0.3, seed=n).astype(np.float64) * 1e200):
        want = oracle.tree_sum_f64(x)
        assert same_bits64(gpu_sum64(torch_dev, x), want), n
        assert same_bits64(gpu_sum64(torch_dev, x, offset=1), want), (n, "8-byte aligned only")


def test_sum64_specials_and_large(torch_dev):
    rng = np.random.default_rng(40)
    base = rng.standard_normal(100_000)
    for extra in ([np.inf], [np.inf, -np.inf], [np.nan], [1.7e308, 1.7e308]):
        x = np.concatenate([base, np.array(extra)])
        assert same_bits64(gpu_sum64(torch_dev, x), oracle.tree_sum_f64(x)), extra
    x = rng.standard_normal(30_000_000)
    assert same_bits64(gpu_sum64(torch_dev, x), oracle.tree_sum_f64(x))


def test_var64_page_datasets_and_square(torch_dev):
    for name, a, axis, _ in W.datasets_d1_d4():
        check_var64(torch_dev, a.astype(np.float64), axis)
        check_var64(torch_dev, a.astype(np.float64), axis, 1)
    check_var64(torch_dev, W.c4_matrix().astype(np.float64)[:1024], 1)


@pytest.mark.parametrize("n", [1, 2, 3, 64, 255, 256, 257, 1000, 1024, 1025, 1500, 2048, 4095, 4096, 4097, 8192, 8193, 16384,
                               16385, 40000])
def test_var64_rows(torch_dev, n):
    rng = np.random.default_rng(n)
    a = rng.normal(1e8, 3, (19, n))
    check_var64(torch_dev, a, 1)
    check_var64(torch_dev, a, 1, 2)
    b = W.adversarial_values(19 * n, n).astype(np.float64).reshape(19, n) * 1e250
    check_var64(torch_dev, b, 1)


@pytest.mark.parametrize("shape", [(5000, 4), (999, 7), (600, 16), (301, 33), (130, 100), (97, 255), (66, 512),
                                   (1000, 6)])
def test_var64_many_short_rows(torch_dev, shape):
    # rows of at most 512 doubles share waves (a group of lanes per row)
    rng = np.random.default_rng(shape[0] + shape[1])
    a = rng.normal(-2e5, 3, shape)
    check_var64(torch_dev, a, 1)
    check_var64(torch_dev, a, 1, 1)
    b = W.adversarial_values(shape[0] * shape[1], shape[1]).astype(np.float64).reshape(shape) * 1e200
    check_var64(torch_dev, b, 1)


@pytest.mark.parametrize("R", [1, 2, 4, 5, 16, 17, 64, 65, 256, 257, 512, 513, 1000, 1024, 1025, 3000, 8192, 9001])
def test_var64_cols(torch_dev, R):
    # 65 to 1024 rows: one launch, two adjacent columns per lane (16-byte
    # loads) when the width is even, one otherwise; above 1024 rows: 128-row
    # chunks in the same layout, more than 32 chunks per column take a
    # separate m launch
    rng = np.random.default_rng(R)
    for C in (1, 63, 64, 65, 130):
        a = rng.normal(-5e3, 2, (R, C))
        check_var64(torch_dev, a, 0)
        check_var64(torch_dev, a, 0, 1)
    if R > 64:
        b = W.adversarial_values(R * 300, R).astype(np.float64).reshape(R, 300) * 1e250
        check_var64(torch_dev, b, 0)


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 9, 15, 16])
def test_var64_short_cols(torch_dev, R):
    # columns of at most 15 rows: two per lane, every tree in-lane (16 rows
    # and odd widths: a lane per column)
    rng = np.random.default_rng(R + 41)
    for C in (2, 3, 1000, 100_000):
        a = rng.normal(7e5, 3, (R, C))
        check_var64(torch_dev, a, 0)
        check_var64(torch_dev, a, 0, 1)
        check_var64(torch_dev, a, 0, 4)
    b = W.adversarial_values(R * 2048, R + 8).astype(np.float64).reshape(R, 2048) * 1e150
    check_var64(torch_dev, b, 0)


@pytest.mark.parametrize("R,C", [(100, 70_000), (400, 20_000), (65, 70_000), (1000, 18_000), (200, 20_000),
                                 (200, 40_000), (129, 2048), (1024, 32), (65, 4), (300, 7), (777, 3001), (513, 1),
                                 (1000, 20_001), (600, 3)])
def test_var64_cols_one_launch(torch_dev, R, C):
    # whole columns of 65..1024 rows in one launch: up to 512 rows one column
    # per lane in every (G, W) choice; above, two columns per lane (even
    # widths) or one (odd widths)
    rng = np.random.default_rng(R * 5 + C)
    a = rng.normal(-6e4, 5, (R, C))
    check_var64(torch_dev, a, 0)
    check_var64(torch_dev, a, 0, 1)
    check_var64(torch_dev, np.ascontiguousarray(a[:, 1:]) if C > 2 else a, 0)
    b = W.adversarial_values(R * C, R + 9).astype(np.float64).reshape(R, C) * 1e100
    check_var64(torch_dev, b, 0)


@pytest.mark.parametrize("R,C", [(30000, 1), (100000, 1), (300000, 1), (8_400_000, 1), (50000, 2), (20000, 3),
                                 (70000, 4), (2_100_000, 4), (9000, 7), (5000, 10), (3000, 12), (40000, 17),
                                 (8193, 40), (2000, 130), (257, 5), (600, 64)])
def test_var64_cols_narrow(torch_dev, R, C):
    # narrow matrices: G row groups per wave (chunks of 128*G rows, G from 1
    # to 64 as the column groups number 65 down to 1); per-column trees by a
    # lane group (up to 32 chunks), a wave (up to 1024) or a thread (beyond:
    # 8,400,000 rows in 8192-row chunks)
    rng = np.random.default_rng(R * 7 + C)
    a = rng.normal(-3e5, 9, (R, C))
    check_var64(torch_dev, a, 0)
    check_var64(torch_dev, a, 0, 2)
    if R * C <= 400_000:
        b = W.adversarial_values(R * C, R + C).astype(np.float64).reshape(R, C) * 1e200
        check_var64(torch_dev, b, 0)


@pytest.mark.parametrize("R", [200_000, 600_000])
def test_var64_cols_many_chunks(torch_dev, R):
    # 1563 chunks of 128 rows per column: a wave per column, 64 nodes per
    # lane; 4688 chunks: runs of 128 nodes per lane merged by a binary counter
    a = np.random.default_rng(R).normal(4e4, 2, (R, 65))
    check_var64(torch_dev, a, 0)


@pytest.mark.parametrize("shape,axis", [((3, 300_001), 1), ((1, 1 << 20), 1), ((70_000, 6), 0), ((4096, 4096), 0)])
def test_var64_long_slices(torch_dev, shape, axis):
    # chunked paths: long rows (8192-value chunks, per-row top trees) and
    # tall columns (128-row chunks; 547 chunks per column for 70,000 rows)
    rng = np.random.default_rng(shape[0] + shape[1])
    a = rng.normal(3e9, 7, shape)
    check_var64(torch_dev, a, axis)
    check_var64(torch_dev, np.full(shape, 1e307), axis)


def test_var64_top_of_range_and_specials(torch_dev):
    # float64 [1e307]*3 (the page's "not measured" case): the method gives 0
    for c in (1e307, 1e308, -1.7e308):
        v = check_var64(torch_dev, np.full((2, 3), c), 1)
        assert np.all(v == 0.0)
    a = np.random.default_rng(41).normal(0, 1, (6, 500))
    a[0, 7] = np.nan
    a[1, 9] = np.inf
    a[2, 3] = np.inf
    a[2, 4] = -np.inf
    a[3, :] = 1.7e308 * np.sign(np.random.default_rng(42).standard_normal(500))
    check_var64(torch_dev, a, 1)
    check_var64(torch_dev, np.ascontiguousarray(a.T), 0)
    import stable_variance_amd as sv

    torch, dev = torch_dev
    v = sv.var(torch.zeros((3, 0), dtype=torch.float64, device=dev), dim=1)
    assert torch.isnan(v).all()


# at least 256 rows of 16385..32768 values: one workgroup of 16 waves, 32
# doubles per lane (odd widths: 8-byte loads), or the chunks under
# var_long_rows 0; fewer rows keep the chunks
@pytest.mark.parametrize("shape", [(256, 16385), (300, 20001), (256, 32768), (257, 24576), (255, 20000)])
@pytest.mark.parametrize("long_rows", [1, 0])
def test_var64_long_rows_one_workgroup(torch_dev, shape, long_rows):
    import stable_variance_amd as sv

    sv.set_tuning("var_long_rows", long_rows)
    try:
        rng = np.random.default_rng(shape[0] + shape[1])
        a = rng.normal(-3e7, 5, shape)
        check_var64(torch_dev, a, 1)
        check_var64(torch_dev, a, 1, 1)
        b = W.adversarial_values(shape[0] * shape[1], shape[1]).astype(np.float64).reshape(shape) * 1e200
        check_var64(torch_dev, b, 1)
    finally:
        sv.set_tuning("reset", 0)


@pytest.mark.parametrize("items", [1024, 4096])
def test_var64_batched_launches(torch_dev, items):
    # every float64 shape class with each grid cut into launches of at most
    # `items` work-items (first-workgroup offsets), bit for bit
    import stable_variance_amd as sv

    rng = np.random.default_rng(items + 64)
    sv.set_tuning("launch_items", items)
    try:
        for shape, axis in (((3000, 5), 1), ((800, 700), 1), ((300, 20000), 1), ((260, 17000), 1),
                            ((6, 3000), 0), ((40, 900), 0), ((300, 900), 0), ((700, 901), 0), ((1100, 300), 0),
                            ((3000, 7), 0)):
            a = rng.normal(-4e3, 9, shape)
            check_var64(torch_dev, a, axis, 1)
    finally:
        sv.set_tuning("reset", 0)


@pytest.mark.parametrize("R", [3, 1000, 20000, 1 << 20])
def test_var64_single_column_as_a_row(torch_dev, R):
    rng = np.random.default_rng(R + 64)
    a = rng.normal(-3e3, 5, (R, 1))
    for ddof in (0, 2):
        v = check_var64(torch_dev, a, 0, ddof)
        assert same_bits64(v, check_var64(torch_dev, np.ascontiguousarray(a.T), 1, ddof))


@pytest.mark.parametrize("once", [2, 0])
@pytest.mark.parametrize("R,C", [(1025, 2), (1025, 3), (2048, 9), (2049, 4), (3000, 33), (4096, 64), (4096, 7),
                                 (1500, 1030), (2048, 40), (4096, 34)])
def test_var64_cols_one_read(torch_dev, once, R, C):
    # columns of 1025..4096 rows: read once by workgroups of whole columns
    # (8 waves; 16 row groups per wave up to 2048 rows, 32 above; the
    # mask-free instance at exactly 2048 or 4096 rows, and there the 16-wave
    # tile for even widths) -- forced on (2) and off (0, the 128-row chunks)
    # whatever the grid's fill
    import stable_variance_amd as sv

    rng = np.random.default_rng(R * 3 + C + once)
    sv.set_tuning("var_cols_once", once)
    try:
        a = rng.normal(2e6, 3, (R, C))
        check_var64(torch_dev, a, 0)
        check_var64(torch_dev, a, 0, 1)
        check_var64(torch_dev, np.ascontiguousarray(a[:, 1:]), 0)
        b = W.adversarial_values(R * C, R + 5).astype(np.float64).reshape(R, C) * 1e200
        check_var64(torch_dev, b, 0)
        sv.set_tuning("launch_items", 1024)
        check_var64(torch_dev, a, 0, 2)
    finally:
        sv.set_tuning("reset", 0)


@pytest.mark.parametrize("R,C", [(4096, 2048), (2048, 4096), (4096, 2046), (4096, 1024)])
def test_var64_cols_wide_tiles(torch_dev, R, C):
    # the default choice at sizes whose grid fills the chip: the 16-wave
    # tiles of 4096 and 2048 rows (eight and sixteen columns per workgroup;
    # [4096, 2046] ends in a partial block), and the mask-free 8-wave tile
    # where the wide grid would not fill ([4096, 1024])
    rng = np.random.default_rng(R + C + 640)
    a = rng.normal(7e4, 2, (R, C))
    check_var64(torch_dev, a, 0)
    check_var64(torch_dev, a, 0, 1)


@pytest.mark.parametrize("pairs", [1, 0])
@pytest.mark.parametrize("R", [4097, 4096 * 3, 100_003, 1 << 20])
def test_var64_two_columns(torch_dev, R, pairs):
    # [R, 2] doubles along axis 0 beyond 4096 rows: one row of R pairs in
    # 4096-row chunks (two interleaved slices), or the column chunks; an
    # aligned and a misaligned (8-byte) base
    import stable_variance_amd as sv

    torch, dev = torch_dev
    rng = np.random.default_rng(R + pairs + 64)
    a = rng.normal(-6e5, 13, (R, 2))
    sv.set_tuning("var_cols_pairs", pairs)
    try:
        for ddof in (0, 1):
            check_var64(torch_dev, a, 0, ddof)
        buf = torch.zeros(2 * R + 1, dtype=torch.float64, device=dev)
        buf[1:] = torch.from_numpy(a.reshape(-1)).to(dev)
        v = sv.var(buf[1:].view(R, 2), dim=0)
        torch.cuda.synchronize()
        assert same_bits64(v.cpu().numpy(), oracle.variance_f64(a, axis=0)[0])
        b = W.adversarial_values(2 * R, R + 3).astype(np.float64).reshape(R, 2) * 1e200
        check_var64(torch_dev, b, 0)
    finally:
        sv.set_tuning("reset", 0)
