"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every workload is integer, so the bar is bit-exact equality.  Small cases
compare with the sort-based oracle element by element; the 1e9-element case,
too large to sort in a test, is checked with the oracle's linear top-k
characterisation and the oracle's int64 sum.
"""
import os

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
    """Device copy of x, optionally starting `offset` int32s past a 16-byte
    boundary (to exercise the unaligned head)."""
    import torch
    buf = torch.empty(x.size + 4, dtype=torch.int32, device="cuda")
    view = buf[offset:offset + x.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return view


def check_topk(ltk, x, k, offset=0):
    got = ltk.topk(dev(x, offset), k).cpu().numpy()
    want = oracle.topk(x, k)
    assert np.array_equal(got, want), (x.size, k, offset, got[:8], want[:8])


def check_reduce(ltk, x, offset=0):
    xd = dev(x, offset)
    for name, op in ltk.OPS.items():
        got = int(ltk.reduce(xd, op).cpu()[0])
        assert got == oracle.reduce(x, op), (name, x.size, offset)


# ------------------------------------------------------------- workloads
def test_full_1e6_topk20_and_reductions(ltk):
    x = synth.workload("full_1e6")
    check_topk(ltk, x, 20)
    check_reduce(ltk, x)


def test_pm1000_2p26_reductions(ltk):
    x = synth.workload("pm1000_2p26")
    check_reduce(ltk, x)


def test_full_1e8_topk20(ltk):
    x = synth.workload("full_1e8")
    check_topk(ltk, x, 20)


@pytest.mark.parametrize("variant", [None, "sorted", "equal"])
def test_dup1000_1e7_topk100(ltk, variant):
    x = synth.workload("dup1000_1e7", variant)
    check_topk(ltk, x, 100)


def test_full_1e9_topk20_and_sum(ltk):
    import torch
    x = synth.workload("full_1e9")
    xd = torch.from_numpy(x).to("cuda")
    got = ltk.topk(xd, 20).cpu().numpy()
    s = int(ltk.reduce(xd, ltk.SUM).cpu()[0])
    del xd
    torch.cuda.empty_cache()
    assert oracle.check_topk(x, 20, got) == 0, got
    assert s == oracle.reduce(x, oracle.SUM)


# ------------------------------------------------------------- edge cases
SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 4095, 4096, 4097,
         3 * 4096 + 17, 65536 + 3, (1 << 20) - 1, (1 << 20) + 1,
         517 * 4096 + 1029]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_sizes_and_misalignment(ltk, n, offset):
    x = synth.fill(1000 + n, n)
    for k in sorted({1, min(n, 7), min(n, 20), min(n, 128)}):
        check_topk(ltk, x, k, offset)
    check_reduce(ltk, x, offset)


@pytest.mark.parametrize("k", [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65,
                               100, 127, 128])
def test_every_list_capacity(ltk, k):
    x = synth.fill(77, 300_001)
    check_topk(ltk, x, k)
    y = synth.fill(78, 300_001, 0, 50)    # heavy duplicates
    check_topk(ltk, y, k)


@pytest.mark.parametrize("n", [1, 5, 64, 100, 128])
def test_k_equals_n(ltk, n):
    x = synth.fill(5 + n, n, -3, 7)
    check_topk(ltk, x, min(n, 128))


@pytest.mark.parametrize("pattern", ["int_min", "int_max", "alternating",
                                     "descending", "ascending", "top_ties",
                                     "all_but_one_min", "zeros"])
def test_special_values(ltk, pattern):
    n = 200_003
    if pattern == "int_min":
        x = np.full(n, I32_MIN, np.int32)
    elif pattern == "int_max":
        x = np.full(n, I32_MAX, np.int32)
    elif pattern == "alternating":
        x = np.where(np.arange(n) % 2 == 0, I32_MIN, I32_MAX).astype(np.int32)
    elif pattern == "descending":
        x = np.arange(n, 0, -1).astype(np.int32)
    elif pattern == "ascending":
        x = np.arange(-n // 2, n - n // 2).astype(np.int32)
    elif pattern == "top_ties":
        x = synth.fill(9, n, -10**6, 10**6)
        x[::1000] = 10**6 + 5        # ~200 copies of the maximum
    elif pattern == "all_but_one_min":
        x = np.full(n, I32_MIN, np.int32)
        x[n // 2] = 7
    else:
        x = np.zeros(n, np.int32)
    for k in (1, 20, 100, 128):
        check_topk(ltk, x, k)
    check_reduce(ltk, x)


@pytest.mark.parametrize("copies", [300, 2_000, 20_000])
@pytest.mark.parametrize("k", [20, 32])
def test_ties_below_a_unique_maximum(ltk, copies, k):
    # One maximum, then `copies` equal values just below it, scattered over
    # the whole input: the certified bound lands on the tied value, so the
    # merge of the block candidates sees about `copies` survivors (a few
    # hundred, a few thousand, or more than fit on chip).
    n = 4_000_037
    x = synth.fill(600 + copies, n, -10**6, 10**6)
    idx = np.unique(synth.fill(700 + copies, copies, 0, n).astype(np.int64))
    x[idx] = 10**6 + 3
    x[n // 3] = 10**6 + 9
    check_topk(ltk, x, k)
    check_topk(ltk, x, 100)


@pytest.mark.parametrize("run", [1, 9, 300])
@pytest.mark.parametrize("k", [25, 64, 100, 128])
def test_top_values_in_runs(ltk, run, k):
    # The largest values sit in runs of `run` consecutive elements, so the
    # few workgroups whose tiles hold a run have many survivors each: more
    # than stage 2 reads first from a candidate list (eight), which sends
    # it back for the rest of those lists.  Runs of 1 are the plain case.
    n = 4_000_037
    x = synth.fill(800 + run, n, -10**6, 10**6)
    nruns = (300 + run - 1) // run
    starts = np.sort(synth.fill(900 + run, nruns, 0, n - run)).astype(np.int64)
    top = 10**6 + 1 + synth.fill(950 + run, nruns * run, 0, 10**5)
    for i, s0 in enumerate(starts):
        x[s0:s0 + run] = top[i * run:(i + 1) * run]
    check_topk(ltk, x, k)
    x[starts[0]:starts[0] + run] = 10**6 + 2 * 10**5    # ties at the top
    check_topk(ltk, x, k)


@pytest.mark.parametrize("order", ["ascending", "descending"])
def test_monotone_input_over_many_tiles(ltk, order):
    # Each workgroup streams several tiles, its last one first: on monotone
    # input the first tile it examines holds its largest (ascending) or its
    # smallest (descending) values.
    n = 6_000_011
    x = np.sort(synth.fill(41, n))
    if order == "descending":
        x = x[::-1].copy()
    for k in (1, 20, 64, 100, 128):
        check_topk(ltk, x, k)


def test_sum_exceeds_int32(ltk):
    x = np.full(3_000_000, I32_MAX, np.int32)
    check_reduce(ltk, x)
    y = np.full(3_000_000, I32_MIN, np.int32)
    check_reduce(ltk, y)


def test_reduce_empty_gives_identity(ltk):
    import torch
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    assert int(ltk.reduce(e, ltk.SUM).cpu()[0]) == 0
    assert int(ltk.reduce(e, ltk.MAX).cpu()[0]) == I32_MIN
    assert int(ltk.reduce(e, ltk.MIN).cpu()[0]) == I32_MAX


# ------------------------------------------------------------- robustness
@pytest.mark.parametrize("grid", [1, 2, 7, 64, 255, 512, 1024])
def test_grid_sweep_gives_identical_results(ltk, grid):
    x = synth.fill(31, 2_000_003)
    y = synth.fill(32, 2_000_003, 0, 100)
    try:
        ltk.set_grid(grid)
        for k in (1, 20, 100):
            check_topk(ltk, x, k)
            check_topk(ltk, y, k)
        check_reduce(ltk, x)
    finally:
        ltk.set_grid(0)


@pytest.mark.parametrize("k", [33, 100, 128])
def test_stage2_bound_with_fewer_than_256_blocks(ltk, k):
    # Stage 2 bounds the k-th largest by the group maxima of the blocks;
    # with fewer than 256 blocks some groups are empty, and with fewer than
    # k non-empty groups only INT_MIN is certified.  Grids on both sides.
    x = synth.fill(33, 1_000_003)
    y = synth.fill(34, 1_000_003, 0, 100)
    try:
        for grid in (k - 1, k, k + 1, 200, 244):
            ltk.set_grid(grid)
            check_topk(ltk, x, k)
            check_topk(ltk, y, k)
    finally:
        ltk.set_grid(0)


def test_repeated_calls_and_two_streams(ltk):
    import torch
    xs = [synth.fill(40 + i, 1_000_000 + 977 * i) for i in range(4)]
    ds = [dev(x) for x in xs]
    want = [oracle.topk(x, 20) for x in xs]
    sums = [oracle.reduce(x, oracle.SUM) for x in xs]
    torch.cuda.synchronize()  # inputs were written on the default stream
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        for i, d in enumerate(ds):
            st = s1 if (i + rep) % 2 else s2
            with torch.cuda.stream(st):
                outs.append((i, ltk.topk(d, 20), ltk.reduce(d, ltk.SUM)))
    torch.cuda.synchronize()
    for i, t, s in outs:
        assert np.array_equal(t.cpu().numpy(), want[i])
        assert int(s.cpu()[0]) == sums[i]


def test_k_limits(ltk):
    """k up to 128 takes the register lists, 129 .. 16384 radix selection;
    above that the call is unsupported, and k > n is invalid."""
    xs = synth.fill(1, 20000)
    x = dev(xs)
    assert np.array_equal(ltk.topk(x, 129).cpu().numpy(), oracle.topk(xs, 129))
    with pytest.raises(ltk.LibtopkError) as e:
        ltk.topk(x, ltk.MAX_K_SELECT + 1)
    assert e.value.status == ltk.ERR_UNSUPPORTED
    with pytest.raises(ltk.LibtopkError) as e:
        ltk.topk(dev(xs[:1000]), 1001)
    assert e.value.status == ltk.ERR_INVALID
