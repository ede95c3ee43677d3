"""Lists shorter than k (k > 32 runs on 32-entry lane lists) when one lane
meets more of its workgroup's top-k than its list holds.

A lane's 16 elements of a 16 KiB tile sit at 16-byte slots 0, 1 KiB, 2 KiB
and 3 KiB of the tile (lane 0: elements 0-3, 1024-1027, 2048-2051 and
3072-3075).  Putting distinct large values there in four tiles of one
workgroup gives that lane 64 of the workgroup's top-k: the workgroup must
notice that its lists dropped some and find its top-k again by counting
over memory.  Every entry point that streams through the register lists is
covered: top-k (one workgroup, or a few per row), long rows of the batched
call, and a medium segment of the segmented call.  Results are compared
with the oracle element by element.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

LANE0 = np.array([0, 1, 2, 3, 1024, 1025, 1026, 1027,
                  2048, 2049, 2050, 2051, 3072, 3073, 3074, 3075])


@pytest.fixture(scope="module")
def ltk():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import top_selection_two_amd as m
    m.set_grid(0)
    yield m
    m.set_grid(0)


def plant(rng, n, tiles, base=0):
    """Small values in [0, 1000), and 16 large distinct values at lane 0's
    slots of each listed tile (tile indices relative to `base`)."""
    x = rng.integers(0, 1000, n).astype(np.int32)
    idx = np.concatenate([base + LANE0 + 4096 * t for t in tiles])
    x[idx] = 1_000_000 + rng.permutation(idx.size).astype(np.int32)
    return x


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("k", [33, 64, 100, 128])
@pytest.mark.parametrize("grid", [1, 3])
def test_topk(ltk, k, grid):
    rng = np.random.default_rng(k * 10 + grid)
    # the first workgroup's tiles are 0, grid, 2 grid, ...
    x = plant(rng, 64 * 4096 + 77, [0, grid, 2 * grid, 3 * grid])
    ltk.set_grid(grid)
    try:
        got = ltk.topk(dev(x), k).cpu().numpy()
    finally:
        ltk.set_grid(0)
    assert np.array_equal(got, oracle.topk(x, k))


@pytest.mark.parametrize("k", [40, 128])
@pytest.mark.parametrize("target", [2, 6])
def test_batched_long_rows(ltk, k, target):
    # Two rows of 64 tiles; target 2 gives one workgroup per row (its
    # result is the row's), target 6 three (workgroup 0 of a row has tiles
    # 0, 3, 6, 9).
    rng = np.random.default_rng(k + target)
    rows, cols = 2, 64 * 4096
    per = (target + rows - 1) // rows
    x = np.concatenate([plant(rng, cols, [0, per, 2 * per, 3 * per])
                        for _ in range(rows)]).reshape(rows, cols)
    ltk.set_grid(target)
    try:
        got = ltk.topk_batched(dev(x), k).cpu().numpy()
    finally:
        ltk.set_grid(0)
    assert np.array_equal(got, oracle.topk_batched(x, k))


@pytest.mark.parametrize("k", [40, 128])
def test_segmented_medium_segment(ltk, k):
    # A segment of 60,000 elements (one workgroup streams it) starting at a
    # 16-byte boundary, between two short ones.
    rng = np.random.default_rng(k)
    a, b = 4096, 4096 + 60_000
    x = rng.integers(0, 1000, b + 500).astype(np.int32)
    idx = np.concatenate([a + LANE0 + 4096 * t for t in range(4)])
    x[idx] = 1_000_000 + rng.permutation(idx.size).astype(np.int32)
    offsets = np.array([0, a, b, x.size], np.int64)
    out, cnt = ltk.topk_segmented(dev(x), dev(offsets), k)
    want, wcnt = oracle.topk_segmented(x, offsets, k)
    assert np.array_equal(out.cpu().numpy(), want)
    assert np.array_equal(cnt.cpu().numpy(), wcnt)
