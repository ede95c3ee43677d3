"""GPU parity for histogram_i32 and for topk_i32 with k above 128 (radix
selection), through the C ABI, against the CPU oracle.

Both are integer results, so the bar is bit-exact equality.  Histograms
cover per-wave (<= 256 bins) and per-workgroup (more bins) layouts, bin
widths from 1 to 2^31, ranges at both ends of int32, values outside every
bin, hot bins (all-equal data), sizes around the tile boundaries with
misaligned starts, n = 0, repeated calls and two streams (the device
counters clean themselves).  Top-k by radix selection covers k from 129 to
16384, ties at the k-th value, sorted and all-equal inputs, selection that
stops after the first digit (the whole bucket is needed), k = n, and the
1e8 workload.  At 2^24 elements (the sampled path starts at 2^18), inputs
built around the sampled positions drive each way through it: the one-workgroup
finish with and without copies of the threshold, a copy too large for it,
a copy too large for the candidate buffer, and a sample whose threshold is
too high; and the finish's placement by the first digit against its sort,
with distinct values and with ties, around k = 4096.
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


def check_hist(ltk, x, lo, shift, nbins, offset=0):
    got = ltk.histogram(dev(x, offset), lo, shift, nbins).cpu().numpy()
    want = oracle.histogram(x, lo, shift, nbins)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError("n=%d lo=%d shift=%d nbins=%d offset=%d: %d bins "
                             "differ, first %d: %d vs %d"
                             % (x.size, lo, shift, nbins, offset, bad.size,
                                bad[0], got[bad[0]], want[bad[0]]))


def check_topk(ltk, x, k, offset=0):
    got = ltk.topk(dev(x, offset), k).cpu().numpy()
    want = oracle.topk(x, k)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError("n=%d k=%d offset=%d: %d differ, first at %d: "
                             "%d vs %d" % (x.size, k, offset, bad.size, bad[0],
                                           got[bad[0]], want[bad[0]]))


# ------------------------------------------------------------ histograms
def test_pm1000_every_value_its_bin(ltk):
    x = synth.workload("pm1000_2p26")
    check_hist(ltk, x, -1000, 0, 2001)
    check_hist(ltk, x, -1000, 3, 251)
    check_hist(ltk, x, -500, 0, 256)   # part of the range only


def test_full_1e8_top_bits(ltk):
    x = synth.workload("full_1e8")
    check_hist(ltk, x, I32_MIN, 20, 4096)
    check_hist(ltk, x, I32_MIN, 24, 256)


def test_dup1000_and_pixels(ltk, rng):
    x = synth.workload("dup1000_1e7")
    check_hist(ltk, x, 0, 0, 1000)
    check_hist(ltk, synth.workload("dup1000_1e7", "sorted"), 0, 2, 250)
    pixels = rng.integers(0, 256, size=3_000_000).astype(np.int32)
    check_hist(ltk, pixels, 0, 0, 256)
    check_hist(ltk, pixels, 0, 4, 16)


def test_full_1e9_top_byte(ltk):
    import torch
    x = synth.workload("full_1e9")
    xd = torch.from_numpy(x).to("cuda")
    got = ltk.histogram(xd, I32_MIN, 24, 256).cpu().numpy()
    del xd
    torch.cuda.empty_cache()
    assert np.array_equal(got, oracle.histogram(x, I32_MIN, 24, 256))
    assert int(got.sum()) == x.size


SIZES = [0, 1, 3, 4, 5, 255, 256, 257, 4095, 4096, 4097, 8191, 8192, 12289,
         65536 + 3, 1_000_003]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_sizes_and_offsets(ltk, rng, n, offset):
    x = rng.integers(-3000, 3000, size=n).astype(np.int32)
    check_hist(ltk, x, -2048, 4, 256, offset)
    check_hist(ltk, x, -2500, 0, 4096, offset)


@pytest.mark.parametrize("lo,shift,nbins", [
    (0, 0, 1), (I32_MIN, 31, 2), (I32_MIN, 31, 1), (I32_MAX, 0, 1),
    (I32_MAX, 5, 7), (-1, 31, 1), (I32_MIN, 0, 4096), (I32_MIN + 5, 28, 17),
    (0, 31, 1), (-7, 1, 257), (123, 9, 255)])
def test_ranges_and_widths(ltk, rng, lo, shift, nbins):
    x = rng.integers(I32_MIN, I32_MAX, size=500_000, dtype=np.int64,
                     endpoint=True).astype(np.int32)
    x[:6] = [I32_MIN, I32_MAX, 0, -1, lo, I32_MIN + 1]
    check_hist(ltk, x, lo, shift, nbins)
    small = rng.integers(-20, 20, size=70_000).astype(np.int32)
    check_hist(ltk, small, lo, shift, nbins)


@pytest.mark.parametrize("nbins", [1, 256, 4096])
def test_hot_bins(ltk, nbins):
    for v in (0, 7, I32_MIN, I32_MAX):
        x = np.full(2_000_003, v, np.int32)
        check_hist(ltk, x, min(v, 0), 0 if nbins > 1 else 31, nbins)
    alt = np.tile(np.array([3, 250], np.int32), 600_000)
    check_hist(ltk, alt, 0, 0, nbins)
    # A whole wave's elements in one bin add with one atomic; below the
    # range they add nowhere.
    check_hist(ltk, np.full(1_000_003, -7, np.int32), 0, 0, nbins)
    runs = np.repeat(np.arange(40, dtype=np.int32), 50_000)
    check_hist(ltk, runs, 0, 2, nbins)


@pytest.mark.parametrize("grid", [1, 7, 64, 1024])
def test_histogram_grid_setting(ltk, rng, grid):
    x = rng.integers(-10_000, 10_000, size=2_000_000).astype(np.int32)
    try:
        ltk.set_grid(grid)
        check_hist(ltk, x, -10_000, 3, 2500)
        check_hist(ltk, x, -128, 0, 256)
    finally:
        ltk.set_grid(0)


def test_histogram_repeated_calls_on_two_streams(ltk, rng):
    import torch
    xs = [rng.integers(-500, 500, size=3_000_000).astype(np.int32)
          for _ in range(2)]
    ds = [dev(x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for x, d, s in zip(xs, ds, streams):
            with torch.cuda.stream(s):
                outs.append((x, ltk.histogram(d, -500, 2, 250)))
    torch.cuda.synchronize()
    for x, o in outs:
        assert np.array_equal(o.cpu().numpy(),
                              oracle.histogram(x, -500, 2, 250))


# ------------------------------------------------------ top-k for large k
@pytest.mark.parametrize("k", [129, 200, 1000, 4096, 16384])
def test_full_1e6_large_k(ltk, k):
    x = synth.workload("full_1e6")
    check_topk(ltk, x, k)
    check_topk(ltk, x[:777_777], k, offset=3)


@pytest.mark.parametrize("variant", [None, "sorted", "equal"])
@pytest.mark.parametrize("k", [129, 5000, 16384])
def test_dup1000_large_k(ltk, variant, k):
    x = synth.workload("dup1000_1e7", variant)
    check_topk(ltk, x, k)


def test_full_1e8_large_k(ltk):
    x = synth.workload("full_1e8")
    check_topk(ltk, x, 1000)
    check_topk(ltk, x, 16384)


@pytest.mark.parametrize("k", [129, 1000, 16384])
def test_large_k_edges(ltk, rng, k):
    # k = n, and n just above k
    for n in (k, k + 1, k + 4097):
        check_topk(ltk, rng.integers(-50, 50, size=n).astype(np.int32), k)
    for v in (I32_MIN, I32_MAX, 0):
        check_topk(ltk, np.full(3 * k + 11, v, np.int32), k)
    alt = np.tile(np.array([I32_MIN, I32_MAX], np.int32), 2 * k)
    check_topk(ltk, alt, k)
    # exactly k values above the rest: selection stops after the first
    # digit, since the whole bucket is needed
    x = rng.integers(-1000, 1000, size=300_000).astype(np.int32)
    x[rng.choice(x.size, size=k, replace=False)] = 2 ** 30
    check_topk(ltk, x, k)
    # the k-th value tied many times over
    y = rng.integers(0, 1 << 20, size=500_000).astype(np.int32)
    y[: 3 * k] = 1 << 19
    check_topk(ltk, y, k)


@pytest.mark.parametrize("grid", [1, 7, 1024])
def test_large_k_grid_setting(ltk, rng, grid):
    x = rng.integers(I32_MIN, I32_MAX, size=2_000_000, dtype=np.int64,
                     endpoint=True).astype(np.int32)
    try:
        ltk.set_grid(grid)
        check_topk(ltk, x, 3000)
    finally:
        ltk.set_grid(0)


def test_large_k_repeated_and_mixed_with_small_k(ltk, rng):
    """The selection state, counters and tickets are reused call after call,
    between calls of the other paths on the same stream."""
    x = rng.integers(I32_MIN, I32_MAX, size=1_500_000, dtype=np.int64,
                     endpoint=True).astype(np.int32)
    d = dev(x)
    for k in (1000, 20, 129, 128, 16384, 5):
        assert np.array_equal(ltk.topk(d, k).cpu().numpy(), oracle.topk(x, k))
        h = ltk.histogram(d, I32_MIN, 22, 1024).cpu().numpy()
        assert np.array_equal(h, oracle.histogram(x, I32_MIN, 22, 1024))


# ------------------------------------------- the sampled path (n = 2^24)
# From 2^18 elements on, a strided sample of 16-byte vectors (16, 32 or
# 64 thousand of them, by k) sets a threshold t and a filter pass copies
# the values above t.  With an aligned input of n = 2^24 the sample reads
# elements s i .. s i + 3 with a stride s of 1024, 512 or 256, all within
# the positions 256 i .. 256 i + 3, so the cases below can steer what the
# sample sees and send the call down each of its ways: the one-workgroup
# finish (with and without copies of t), the selection passes over the
# copy, and the passes over the input when the copy is too large or the
# sample claims too much.
N_SAMPLED = 2 ** 24
SPACING = 256


def sampled_positions():
    """Every position a sample of an aligned 2^24 input may read."""
    base = np.arange(N_SAMPLED // SPACING, dtype=np.int64) * SPACING
    return (base[:, None] + np.arange(4)[None, :]).ravel()


def unsampled_choice(rng, count):
    """count distinct positions that no sample reads."""
    free = SPACING - 4
    pos = rng.choice(N_SAMPLED // SPACING * free, size=count, replace=False)
    return (pos // free) * SPACING + 4 + (pos % free)


@pytest.mark.parametrize("k", [129, 1000, 16384])
def test_sampled_all_equal(ltk, k):
    # gt = 0 above t and every value equal to it: k copies of t
    for v in (0, -7, I32_MIN, I32_MAX):
        check_topk(ltk, np.full(N_SAMPLED, v, np.int32), k)


@pytest.mark.parametrize("k", [129, 1000, 16384])
def test_sampled_few_above_a_sea(ltk, rng, k):
    # fewer than k values above t = 5: all of them, then copies of 5
    x = np.full(N_SAMPLED, 5, np.int32)
    pos = unsampled_choice(rng, 100)
    x[pos] = 10 + np.arange(100, dtype=np.int32)
    check_topk(ltk, x, k)


@pytest.mark.parametrize("k", [1000, 16384])
def test_sampled_copy_between_finish_and_buffer(ltk, rng, k):
    # the sample sees only zeros, t = 0, and 2M values lie above it: too
    # many for one workgroup, few enough for the candidate buffer
    x = np.zeros(N_SAMPLED, np.int32)
    pos = unsampled_choice(rng, 2_000_000)
    x[pos] = rng.integers(1, 2 ** 31 - 1, size=pos.size, dtype=np.int64)
    check_topk(ltk, x, k)


def test_sampled_copy_beyond_buffer(ltk, rng):
    # 5M values above t = 0: more than the candidate buffer holds, so the
    # selection passes read the input
    x = np.zeros(N_SAMPLED, np.int32)
    pos = unsampled_choice(rng, 5_000_000)
    x[pos] = rng.integers(1, 1_000_000, size=pos.size)
    check_topk(ltk, x, 1000)
    check_topk(ltk, x, 16384)


@pytest.mark.parametrize("k", [1000, 16384])
def test_sampled_threshold_too_high(ltk, rng, k):
    # the sample sees only large values, the rest of the input is small:
    # fewer than k values reach t, so the passes read the input
    x = rng.integers(-1_000_000, 1_000_000, size=N_SAMPLED).astype(np.int32)
    sp = sampled_positions()
    x[sp] = 1_000_000_000 + rng.permutation(sp.size).astype(np.int32)
    check_topk(ltk, x, k)


def test_sampled_misaligned_and_ties(ltk, rng):
    # a misaligned start moves the sample; ties at the k-th value
    x = rng.integers(0, 1 << 16, size=N_SAMPLED + 12345).astype(np.int32)
    check_topk(ltk, x, 5000, offset=1)
    check_topk(ltk, x, 16384, offset=3)


@pytest.mark.parametrize("hi", [None, 2 ** 24, 2 ** 20])
@pytest.mark.parametrize("k", [129, 1000, 4096, 4097])
def test_sampled_placement_and_ties(ltk, rng, hi, k):
    # The one-workgroup finish places the result by its first digit's
    # counts when k <= 4096 and no bin is crowded, and sorts otherwise:
    # distinct values, occasional ties and heavy ties, around k = 4096.
    if hi is None:
        x = rng.integers(I32_MIN, I32_MAX, size=N_SAMPLED, dtype=np.int64,
                         endpoint=True).astype(np.int32)
    else:
        x = rng.integers(0, hi, size=N_SAMPLED).astype(np.int32)
    check_topk(ltk, x, k)


@pytest.mark.parametrize("span", [2 ** 20, 2 ** 18])
@pytest.mark.parametrize("k", [200, 4096])
def test_sampled_placement_with_equal_values(ltk, rng, span, k):
    # Values just below INT32_MAX, each about n / span times: the copy's
    # bins each hold one value many times over (about 16 times: placed by
    # the first digit; about 64: sorted instead).
    x = (I32_MAX - rng.integers(0, span, size=N_SAMPLED)).astype(np.int32)
    check_topk(ltk, x, k)


@pytest.mark.parametrize("n,k", [(2 ** 18 - 1, 1000), (2 ** 18, 1000),
                                 (2 ** 18 + 5, 129), (300_000, 16384),
                                 (600_000, 5000), (1_000_000, 16384),
                                 (3_000_000, 4096), (3_000_000, 5000),
                                 (6_000_000, 16384), (100_000, 5000),
                                 (200_000, 16384), (2 ** 18 - 1, 2000)])
def test_sampling_thresholds(ltk, rng, n, k):
    # Around the sizes where the sampled path takes over from the digit
    # passes (2^18, and about 334 k for large k): both ways agree with the
    # oracle, with distinct values and with ties, aligned or not.
    x = rng.integers(I32_MIN, I32_MAX, size=n, dtype=np.int64,
                     endpoint=True).astype(np.int32)
    check_topk(ltk, x, k)
    check_topk(ltk, x[: n - 7], k, offset=2)
    ties = rng.integers(0, 5000, size=n).astype(np.int32)
    check_topk(ltk, ties, k)
