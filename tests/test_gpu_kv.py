"""GPU parity for key-value Top-K (topk_kv_i32 / topk_kv_f32) against the
CPU oracle.  The tie rule (value descending, then position ascending) makes
the answer unique, so values and positions must match bit for bit: on the
workloads, on heavy ties (where the positions decide), around tile
boundaries with misaligned starts, at every list capacity, on float special
values (signed zeros, infinities, NaNs of both signs, subnormals), across a
grid sweep and on two streams.
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


def dev(x, offset=0):
    import torch
    buf = torch.empty(x.size + 4, dtype=torch.from_numpy(x[:0]).dtype,
                      device="cuda")
    view = buf[offset:offset + x.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return view


def check(ltk, x, k, offset=0):
    v, i = ltk.topk_kv(dev(x, offset), k)
    gv, gi = v.cpu().numpy(), i.cpu().numpy()
    wv, wi = oracle.topk_kv(x, k)
    assert np.array_equal(gi, wi), (x.size, k, offset, gi[:8], wi[:8])
    # values compared as bit patterns (NaNs included)
    assert np.array_equal(gv.view(np.uint32), wv.view(np.uint32)), (
        x.size, k, offset, gv[:8], wv[:8])


def as_float(bits):
    """Seeded int32 words read as float32 (every bit pattern, NaNs and
    infinities included)."""
    return bits.view(np.float32)


# ------------------------------------------------------------- workloads
def test_full_1e6_k20(ltk):
    x = synth.workload("full_1e6")
    check(ltk, x, 20)
    check(ltk, as_float(x), 20)


def test_full_1e8_k20(ltk):
    x = synth.workload("full_1e8")
    check(ltk, x, 20)
    check(ltk, as_float(x), 20)


@pytest.mark.parametrize("variant", [None, "sorted", "equal"])
def test_dup1000_1e7_k100(ltk, variant):
    # heavy ties: 1000 distinct values over 1e7 elements; positions decide
    x = synth.workload("dup1000_1e7", variant)
    check(ltk, x, 100)
    check(ltk, x, 20)


@pytest.mark.parametrize("k", [32, 40, 64, 128])
@pytest.mark.parametrize("grid", [0, 512, 1024])
def test_dup1000_stage2_tie_bound(ltk, k, grid):
    # About 19 copies of the largest value per workgroup at 512 workgroups:
    # the group-maxima bound leaves over 512 survivors (runs of consecutive
    # blocks, whose first tiles come early), and stage 2 takes the k-th
    # largest of all block maxima instead.
    x = synth.workload("dup1000_1e7")
    ltk.set_grid(grid)
    try:
        check(ltk, x, k)
    finally:
        ltk.set_grid(0)


@pytest.mark.parametrize("k", [33, 100, 128])
@pytest.mark.parametrize("grid", [1, 3])
@pytest.mark.parametrize("f32", [False, True])
def test_short_lists_one_lane_overflows(ltk, k, grid, f32):
    # k > 32 runs on lists of 32 keys per lane.  Here one lane of the first
    # workgroup meets 16 large values in each of its first 4 tiles (its
    # 16-byte slots at 0, 1 KiB, 2 KiB and 3 KiB of each 16 KiB tile): 64
    # of the workgroup's top-k, more than its list holds, so the workgroup
    # finds its top-k again by counting over memory.
    rng = np.random.default_rng(k + grid)
    tiles = 64
    x = rng.integers(0, 1000, tiles * 4096).astype(np.int32)
    lane0 = np.concatenate([[0, 1, 2, 3], [1024, 1025, 1026, 1027],
                            [2048, 2049, 2050, 2051], [3072, 3073, 3074, 3075]])
    big = []
    for t in range(4):
        # the first workgroup's t-th tile
        big.append(lane0 + t * grid * 4096)
    big = np.concatenate(big)
    x[big] = 1_000_000 + rng.permutation(big.size).astype(np.int32)
    if f32:
        x = x.astype(np.float32)
    ltk.set_grid(grid)
    try:
        check(ltk, x, k)
    finally:
        ltk.set_grid(0)


def test_pm1000_2p26_floats(ltk):
    # about 33,000 copies of each value: ties by position again
    x = (synth.workload("pm1000_2p26").astype(np.float32) / 8.0)
    check(ltk, x, 20)
    check(ltk, x, 128)


# ------------------------------------------------------------- edge cases
SIZES = [1, 2, 3, 5, 64, 65, 257, 4095, 4096, 4097, 3 * 4096 + 17,
         65536 + 3, (1 << 20) + 1, 517 * 4096 + 1029]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_sizes_and_misalignment(ltk, n, offset):
    x = synth.fill(3000 + n, n)
    for k in sorted({1, min(n, 7), min(n, 20), min(n, 128)}):
        check(ltk, x, k, offset)
    y = synth.fill(3000 + n, n, -3, 7)   # ties everywhere
    check(ltk, y, min(n, 20), offset)


@pytest.mark.parametrize("k", [1, 2, 15, 16, 17, 24, 25, 32, 33, 64, 65,
                               100, 128])
def test_every_list_capacity(ltk, k):
    x = synth.fill(91, 300_001)
    check(ltk, x, k)
    y = synth.fill(92, 300_001, 0, 50)
    check(ltk, y, k)
    check(ltk, as_float(x), k)


@pytest.mark.parametrize("pattern", ["equal", "int_min", "ascending",
                                     "descending", "one_max_many_next"])
def test_int_patterns(ltk, pattern):
    n = 200_003
    if pattern == "equal":
        x = np.full(n, 17, np.int32)           # result: positions 0..k-1
    elif pattern == "int_min":
        x = np.full(n, I32_MIN, np.int32)
    elif pattern == "ascending":
        x = np.arange(n, dtype=np.int32)
    elif pattern == "descending":
        x = np.arange(n, 0, -1).astype(np.int32)
    else:
        x = np.zeros(n, np.int32)
        x[::97] = 5
        x[n // 3] = 9
    for k in (1, 20, 100, 128):
        check(ltk, x, k)


def test_float_specials(ltk):
    n = 1_000_003
    rng = np.random.default_rng(5)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1e-42, -1e-42, 1.0,
                         -1.0, 3.4e38, -3.4e38], np.float32)
    x = specials[rng.integers(0, specials.size, size=n)]
    bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF],
                    dtype=np.uint32).view(np.float32)   # NaNs of both signs
    x[rng.integers(0, n, size=50)] = bits[rng.integers(0, 4, size=50)]
    for k in (1, 20, 64, 128):
        check(ltk, x, k)
    # without NaNs: +0 before -0 once only zeros remain near the top
    z = np.where(rng.random(n) < 0.5, np.float32(0.0),
                 np.float32(-0.0)).astype(np.float32)
    z[7] = np.float32(-1.0)
    check(ltk, z, 20)


@pytest.mark.parametrize("grid", [1, 2, 7, 64, 255, 512, 1024])
def test_grid_sweep(ltk, grid):
    x = synth.fill(34, 2_000_003)
    y = synth.fill(35, 2_000_003, 0, 100)
    try:
        ltk.set_grid(grid)
        for k in (1, 20, 100):
            check(ltk, x, k)
            check(ltk, y, k)
    finally:
        ltk.set_grid(0)


@pytest.mark.parametrize("k", [33, 100, 128])
def test_stage2_bound_with_fewer_blocks_than_k(ltk, k):
    # With fewer block lists than k, stage 2 bounds the result by the k-th
    # largest of the lists' first ceil(k / G) keys; grids on both sides.
    x = synth.fill(36, 500_003)
    y = synth.fill(37, 500_003, 0, 100)
    try:
        for grid in (1, 7, k - 1, k, k + 1, 122):
            ltk.set_grid(grid)
            check(ltk, x, k)
            check(ltk, y, k)
    finally:
        ltk.set_grid(0)


@pytest.mark.parametrize("order", ["ascending", "descending"])
def test_monotone_input_over_many_tiles(ltk, order):
    # Several tiles per workgroup, the last examined first; with ties, so
    # that positions decide among equal values.
    n = 6_000_011
    x = np.sort(synth.fill(42, n, 0, 50_000))
    if order == "descending":
        x = x[::-1].copy()
    for k in (1, 20, 64, 100, 128):
        check(ltk, x, k)


@pytest.mark.parametrize("copies", [300, 20_000])
def test_ties_below_a_unique_maximum(ltk, copies):
    n = 4_000_037
    x = synth.fill(800 + copies, n, -10**6, 10**6)
    idx = np.unique(synth.fill(900 + copies, copies, 0, n).astype(np.int64))
    x[idx] = 10**6 + 3
    x[n // 3] = 10**6 + 9
    for k in (20, 100):
        check(ltk, x, k)


def test_repeated_calls_and_two_streams(ltk):
    import torch
    xs = [synth.fill(60 + i, 1_000_000 + 977 * i, 0, 1000) for i in range(4)]
    ds = [dev(x) for x in xs]
    want = [oracle.topk_kv(x, 20) for x in xs]
    torch.cuda.synchronize()  # inputs were written on the default stream
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        for i, d in enumerate(ds):
            st = s1 if (i + rep) % 2 else s2
            with torch.cuda.stream(st):
                outs.append((i, ltk.topk_kv(d, 20)))
    torch.cuda.synchronize()
    for i, (v, ix) in outs:
        assert np.array_equal(ix.cpu().numpy(), want[i][1])
        assert np.array_equal(v.cpu().numpy(), want[i][0])


def test_values_agree_with_plain_topk(ltk):
    x = synth.workload("full_1e6")
    xd = dev(x)
    v, _ = ltk.topk_kv(xd, 50)
    assert np.array_equal(v.cpu().numpy(), ltk.topk(xd, 50).cpu().numpy())
