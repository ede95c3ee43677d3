"""GPU parity for the one-pass statistics (reduce_stats_i32) against the CPU
oracle: count, sum, max, min and the exact 128-bit sum of squares must all
be bit-exact.  Covers every workload, sizes around the tile boundaries with
misaligned starts, extremes whose sum of squares needs more than 64 bits,
the empty input, a grid sweep, streams, and agreement with reduce_i32.
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
    buf = torch.empty(x.size + 4, dtype=torch.int32, device="cuda")
    view = buf[offset:offset + x.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return view


def check_stats(ltk, x, offset=0):
    got = ltk.unpack_stats(ltk.stats(dev(x, offset)))
    want = oracle.stats(x)
    assert got == want, (x.size, offset, got, want)
    return got


@pytest.mark.parametrize("name,variant", [
    ("full_1e6", None), ("pm1000_2p26", None), ("full_1e8", None),
    ("dup1000_1e7", None), ("dup1000_1e7", "sorted"),
    ("dup1000_1e7", "equal")])
def test_workloads(ltk, name, variant):
    x = synth.workload(name, variant)
    st = check_stats(ltk, x)
    # the population variance is non-negative and zero only for equal data
    num = st["count"] * st["sumsq"] - st["sum"] ** 2
    assert num >= 0
    assert (num == 0) == (st["max"] == st["min"])


def test_full_1e9(ltk):
    import torch
    x = synth.workload("full_1e9")
    xd = torch.from_numpy(x).to("cuda")
    got = ltk.unpack_stats(ltk.stats(xd))
    del xd
    torch.cuda.empty_cache()
    assert got == oracle.stats(x)
    assert got["sumsq"] >= 2 ** 64   # the high word is in use


SIZES = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 4095, 4096, 4097,
         3 * 4096 + 17, 65536 + 3, (1 << 20) - 1, (1 << 20) + 1,
         517 * 4096 + 1029]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_sizes_and_misalignment(ltk, n, offset):
    check_stats(ltk, synth.fill(2000 + n, n), offset)


def test_empty_gives_identities(ltk):
    import torch
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    assert ltk.unpack_stats(ltk.stats(e)) == {
        "count": 0, "sum": 0, "max": I32_MIN, "min": I32_MAX, "sumsq": 0}


@pytest.mark.parametrize("pattern", ["int_min", "int_max", "alternating",
                                     "zeros", "one_big"])
def test_extremes(ltk, pattern):
    n = 3_000_007
    if pattern == "int_min":
        x = np.full(n, I32_MIN, np.int32)        # sum of squares ~ 2^83.5
    elif pattern == "int_max":
        x = np.full(n, I32_MAX, np.int32)
    elif pattern == "alternating":
        x = np.where(np.arange(n) % 2 == 0, I32_MIN, I32_MAX).astype(np.int32)
    elif pattern == "zeros":
        x = np.zeros(n, np.int32)
    else:
        x = np.zeros(n, np.int32)
        x[n // 2] = I32_MIN
    got = check_stats(ltk, x)
    if pattern == "int_min":
        assert got["sumsq"] == n * 2 ** 62


@pytest.mark.parametrize("grid", [1, 2, 7, 64, 255, 512, 1024])
def test_grid_sweep(ltk, grid):
    x = synth.fill(33, 2_000_003)
    try:
        ltk.set_grid(grid)
        check_stats(ltk, x)
        check_stats(ltk, x, 3)
    finally:
        ltk.set_grid(0)


def test_agrees_with_single_reductions(ltk):
    x = synth.workload("pm1000_2p26")
    xd = dev(x)
    st = ltk.unpack_stats(ltk.stats(xd))
    for key, op in [("sum", ltk.SUM), ("max", ltk.MAX), ("min", ltk.MIN)]:
        assert st[key] == int(ltk.reduce(xd, op).cpu()[0])


def test_repeated_calls_and_two_streams(ltk):
    import torch
    xs = [synth.fill(50 + i, 1_000_000 + 1237 * i) for i in range(4)]
    ds = [dev(x) for x in xs]
    want = [oracle.stats(x) for x in xs]
    torch.cuda.synchronize()  # inputs were written on the default stream
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        for i, d in enumerate(ds):
            st = s1 if (i + rep) % 2 else s2
            with torch.cuda.stream(st):
                outs.append((i, ltk.stats(d)))
    torch.cuda.synchronize()
    for i, t in outs:
        assert ltk.unpack_stats(t) == want[i]
