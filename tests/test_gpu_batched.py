"""GPU parity for per-row top-k (topk_batched_i32) and for merging top-k
lists (topk_merge_i32), through the C ABI, against the CPU oracle.

Every workload is integer, so the bar is bit-exact equality.  Row shapes
cover both kernels (rows of at most 4096 elements go one wave per row,
longer rows stream through the top-k kernel, with one or several
workgroups per row), ragged lengths around every boundary of the
short-row buckets and of the 4096-element tiles, strided and misaligned
rows whose padding holds INT32_MAX (it must never reach a result), and
tie-heavy rows.  Merges cover one and two levels (more than 1024 lists),
lists shorter than k, and the shard identity that stage 2 rests on.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

I32_MIN = -(2 ** 31)
I32_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module")
def ltk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_selection_two_amd as m
    m.set_grid(0)
    yield m
    m.set_grid(0)


def dev_rows(x, pad=0, offset=0, fill=I32_MAX):
    """Device copy of the (rows, cols) array x with row stride cols + pad,
    starting `offset` int32s past a 16-byte boundary; padding holds `fill`.
    Returns the strided (rows, cols) view."""
    import torch
    rows, cols = x.shape
    ld = cols + pad
    buf = torch.full((rows * ld + offset + 4,), fill, dtype=torch.int32,
                     device="cuda")
    full = buf[offset:offset + rows * ld].view(rows, ld)
    full[:, :cols].copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return full[:, :cols]


def check_batched(ltk, x, k, pad=0, offset=0):
    rows, cols = x.shape
    got = ltk.topk_batched(dev_rows(x, pad, offset), k).cpu().numpy()
    want = oracle.topk_batched(x, k)
    if not np.array_equal(got, want):
        bad = np.nonzero((got != want).any(axis=1))[0]
        r = int(bad[0])
        raise AssertionError("rows=%d cols=%d k=%d pad=%d offset=%d: %d rows "
                             "differ, first %d: %s vs %s"
                             % (rows, cols, k, pad, offset, bad.size, r,
                                got[r][:8], want[r][:8]))


def rand_rows(rng, rows, cols, hi=None):
    if hi is None:
        return rng.integers(I32_MIN, I32_MAX, size=(rows, cols),
                            dtype=np.int64, endpoint=True).astype(np.int32)
    return rng.integers(0, hi, size=(rows, cols)).astype(np.int32)


# --------------------------------------------------------- the 1e8 shapes
@pytest.mark.parametrize("rows,cols", [(1000, 100_000), (97_656, 1024),
                                       (8, 12_500_000)])
def test_full_1e8_rows_topk20(ltk, rows, cols):
    x = synth.workload("full_1e8")[:rows * cols].reshape(rows, cols)
    check_batched(ltk, x, 20)


def test_shards_merge_to_the_whole(ltk):
    """Eight shards of the 1e8 array (one row each), their top-20 lists,
    merged: the top-20 of the whole array."""
    import torch
    x = synth.workload("full_1e8")
    xd = torch.from_numpy(x).cuda().view(8, -1)
    tops = ltk.topk_batched(xd, 20)
    got = ltk.topk_merge(tops, 20).cpu().numpy()
    assert np.array_equal(got, oracle.topk(x, 20))
    assert np.array_equal(got, ltk.topk(xd.view(-1), 20).cpu().numpy())


# --------------------------------------------------------- sizes and strides
COLS = [1, 2, 5, 63, 64, 65, 100, 255, 256, 257, 511, 512, 513, 1000, 1023,
        1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8192, 8193,
        12_289, 40_000, 300_001]


@pytest.mark.parametrize("cols", COLS)
def test_row_lengths(ltk, rng, cols):
    rows = 37 if cols <= 40_000 else 5
    x = rand_rows(rng, rows, cols)
    for k in sorted({1, min(cols, 20), min(cols, 100), min(cols, 128)}):
        check_batched(ltk, x, k)


@pytest.mark.parametrize("pad,offset", [(1, 0), (3, 1), (17, 2), (0, 3),
                                        (4, 0), (1000, 1)])
@pytest.mark.parametrize("cols", [30, 64, 100, 1024, 3001, 4096, 5000, 70_001])
def test_strided_and_misaligned_rows(ltk, rng, cols, pad, offset):
    x = rand_rows(rng, 9, cols)
    check_batched(ltk, x, 20, pad=pad, offset=offset)


@pytest.mark.parametrize("k", [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65,
                               100, 127, 128])
@pytest.mark.parametrize("cols", [300, 1024, 4096, 20_000])
def test_every_k(ltk, rng, cols, k):
    check_batched(ltk, rand_rows(rng, 13, cols), k)
    check_batched(ltk, rand_rows(rng, 13, cols, hi=50), k)


# --------------------------------------------------------- ties and extremes
@pytest.mark.parametrize("cols", [64, 1000, 4096, 6000, 100_000])
def test_tie_heavy_rows(ltk, rng, cols):
    rows = 20
    dup = rand_rows(rng, rows, cols, hi=1000)
    for k in (20, 100, 128):
        if k > cols:
            continue
        check_batched(ltk, dup, k)
        check_batched(ltk, np.sort(dup, axis=1), k)          # ascending rows
        check_batched(ltk, np.sort(dup, axis=1)[:, ::-1], k)  # descending
        eq = np.repeat(dup[:, :1], cols, axis=1)             # all-equal rows
        check_batched(ltk, eq, k)


@pytest.mark.parametrize("cols", [10, 777, 4096, 9000])
def test_extreme_values(ltk, rng, cols):
    k = min(cols, 20)
    rows = 6
    for v in (I32_MIN, I32_MAX, 0, -1):
        check_batched(ltk, np.full((rows, cols), v, np.int32), k)
    alt = np.tile(np.array([I32_MIN, I32_MAX], np.int32), (rows, cols))
    check_batched(ltk, alt[:, :cols], k)
    # one real value above a sea of INT32_MIN, at a different place per row
    sea = np.full((rows, cols), I32_MIN, np.int32)
    sea[np.arange(rows), rng.integers(0, cols, size=rows)] = 5
    check_batched(ltk, sea, k)
    # INT32_MIN as the k-th value with few larger ones
    few = np.full((rows, cols), I32_MIN, np.int32)
    few[:, : min(cols, 3)] = rng.integers(-5, 5, size=(rows, min(cols, 3)))
    check_batched(ltk, few, k)


# --------------------------------------------------------- workgroups per row
@pytest.mark.parametrize("rows,cols", [(1, 1_000_000), (3, 1_000_000),
                                       (200, 100_000), (511, 50_000),
                                       (600, 20_000), (2, 8193)])
def test_workgroups_per_row(ltk, rng, rows, cols):
    x = rand_rows(rng, rows, cols)
    check_batched(ltk, x, 20)
    check_batched(ltk, x, 100, pad=3, offset=1)


@pytest.mark.parametrize("cols", [4097, 4098, 4099, 5000])
def test_block_list_filled_exactly(ltk, rng, cols):
    """Rows with at most one full tile and a large k: every element goes
    through the lists' tail path and the workgroup's bound depends on how
    far its other waves have got, so the count of list entries that reach
    it varies from call to call and sometimes lands exactly on the LDS
    list's capacity (256).  That case must not be taken as complete while
    deeper entries remain.  Repeated calls cover many such counts."""
    x = rand_rows(rng, 64, cols)
    for k in (64, 100, 128):
        for rep in range(4):
            check_batched(ltk, x, k)


@pytest.mark.parametrize("grid", [1, 7, 64, 1024])
def test_grid_setting_does_not_change_results(ltk, rng, grid):
    x = rand_rows(rng, 5, 300_000)
    try:
        ltk.set_grid(grid)
        check_batched(ltk, x, 20)
        check_batched(ltk, rand_rows(rng, 5, 300_000, hi=100), 64)
    finally:
        ltk.set_grid(0)


def test_repeated_calls_on_two_streams(ltk, rng):
    import torch
    xs = [rand_rows(rng, 6, 200_000) for _ in range(2)]
    ds = [dev_rows(x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for x, d, s in zip(xs, ds, streams):
            with torch.cuda.stream(s):
                outs.append((x, ltk.topk_batched(d, 20)))
    torch.cuda.synchronize()
    for x, o in outs:
        assert np.array_equal(o.cpu().numpy(), oracle.topk_batched(x, 20))


def test_zero_rows(ltk):
    import torch
    x = torch.empty((0, 100), dtype=torch.int32, device="cuda")
    assert ltk.topk_batched(x, 5).shape == (0, 5)


# --------------------------------------------------------- merging lists
def desc_lists(rng, m, length, hi=None):
    x = rand_rows(rng, m, length, hi)
    return np.sort(x, axis=1)[:, ::-1].copy()


def check_merge(ltk, lists, k):
    import torch
    d = torch.from_numpy(lists).cuda()
    got = ltk.topk_merge(d, k).cpu().numpy()
    want = oracle.topk_merge(lists, k)
    assert np.array_equal(got, want), (lists.shape, k, got[:8], want[:8])


@pytest.mark.parametrize("m", [1, 2, 8, 100, 1000, 1024, 1025, 5000,
                               100_000])
def test_merge_shard_results(ltk, m):
    """The 1e6 workload cut into m shards, each shard's top-k by the GPU,
    merged: the top-k of the whole (the two-stage identity)."""
    import torch
    x = synth.workload("full_1e6")
    n = (x.size // m) * m
    xs = x[:n]
    k = min(20, n // m)
    tops = ltk.topk_batched(torch.from_numpy(xs).cuda().view(m, -1), k)
    got = ltk.topk_merge(tops, k).cpu().numpy()
    assert np.array_equal(got, oracle.topk(xs, k)), (m, k)


@pytest.mark.parametrize("length", [1, 3, 20, 128, 500])
@pytest.mark.parametrize("m", [1, 7, 300, 1024, 3000])
def test_merge_sizes(ltk, rng, m, length):
    lists = desc_lists(rng, m, length)
    for k in sorted({1, 20, 100, 128}):
        if k <= m * length:
            check_merge(ltk, lists, k)


@pytest.mark.parametrize("m", [3, 1024, 3000])
def test_merge_top_in_few_lists(ltk, rng, m):
    # All of the top-k in one list, or spread over a few: those lists have
    # more survivors than stage 2 reads first from each (eight).
    for length in (9, 64, 200):
        lists = desc_lists(rng, m, length, hi=10**6)
        for owners in (1, 2, 3):
            big = lists.copy()
            for j in range(owners):
                row = (j * 977) % m
                big[row] = np.sort(10**6 + 10 + rng.integers(
                    0, 10**5, length).astype(np.int32))[::-1]
            for k in (20, 100, 128):
                if k <= m * length:
                    check_merge(ltk, big, k)


@pytest.mark.parametrize("m", [5, 1024, 2500])
def test_merge_ties(ltk, rng, m):
    for k in (20, 128):
        check_merge(ltk, desc_lists(rng, m, 64, hi=3), k)
        check_merge(ltk, np.full((m, 32), 7, np.int32), k)
        check_merge(ltk, np.full((m, 32), I32_MIN, np.int32), k)
        few = np.full((m, 40), I32_MIN, np.int32)
        few[0, :2] = [9, 4]
        check_merge(ltk, few, k)
