"""GPU parity of the segmented top-k (topk_segmented_i32) against the
oracle, bit-exact: values, INT32_MIN padding and counts.

Segments of every class the library handles differently: empty, shorter
than k, short (one wave, up to 4096 elements; each register bucket and its
edges), medium (one workgroup streams the segment, up to 2^18 elements)
and huge (cut into up to 1024 parts merged by a stage 2); misaligned
starts and a misaligned array; ties; every list capacity; scratch growth
and reuse; two streams; scrambled tickets and counters.
"""
import numpy as np
import pytest

import oracle
import synth
import top_selection_two_amd as ltk

pytestmark = pytest.mark.gpu

I32_MIN = -(2 ** 31)


def _dev(a, offset=0):
    import torch
    a = np.ascontiguousarray(a)
    buf = torch.empty(a.size + 4, dtype=torch.from_numpy(a[:0]).dtype,
                      device="cuda")
    view = buf[offset:offset + a.size]
    view.copy_(torch.from_numpy(a))
    return view


def check(x, offsets, k, offset=0, with_counts=True):
    offsets = np.asarray(offsets, dtype=np.int64)
    xd = _dev(x, offset)
    od = _dev(offsets)
    out, cnt = ltk.topk_segmented(xd, od, k, with_counts=with_counts)
    want, wcnt = oracle.topk_segmented(x, offsets, k)
    got = out.cpu().numpy()
    bad = np.nonzero((got != want).any(axis=1))[0] if got.size else []
    assert len(bad) == 0, ("segments differ", bad[:5], np.diff(offsets)[bad[:5]],
                           got[bad[:1]], want[bad[:1]])
    if with_counts:
        assert np.array_equal(cnt.cpu().numpy(), wcnt)
    return got


def cuts_from_lengths(lengths, start=0):
    return np.concatenate([[start], start + np.cumsum(lengths)]).astype(
        np.int64)


def test_hand_example():
    x = np.array([5, 1, 9, 9, 3, 7, 2], np.int32)
    got = check(x, [0, 3, 3, 7], 2)
    assert got.tolist() == [[9, 5], [I32_MIN, I32_MIN], [9, 7]]


@pytest.mark.parametrize("k", [1, 7, 20, 64, 100, 128])
def test_mixed_lengths(k):
    rng = np.random.default_rng(100 + k)
    lengths = np.concatenate([
        rng.integers(0, 8, 50),                       # empty and tiny
        rng.integers(1, 4097, 300),                   # short
        [255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049,
         4095, 4096, 4097, 4098],                     # bucket edges
        rng.integers(4097, 40_000, 40),               # medium
        [131_071, 131_072, 131_073],                  # medium / huge edge
        [262_143, 262_144, 262_145],                  # one / two units
        [700_001, 2_500_003],                         # huge
    ]).astype(np.int64)
    rng.shuffle(lengths)
    offsets = cuts_from_lengths(lengths, start=3)
    x = synth.fill(7 + k, int(offsets[-1]) + 5)
    print("mixed k=%d nseg=%d n=%d" % (k, lengths.size, x.size), flush=True)
    check(x, offsets, k)


@pytest.mark.parametrize("k", [1, 20, 100, 128])
def test_many_short_segments(k):
    # An average length below 1024 takes the lean short kernel, which lists
    # segments of 1025 .. 4096 elements for one wave each of the long
    # kernel; a few medium and huge ones ride along.
    rng = np.random.default_rng(200 + k)
    lengths = np.concatenate([
        rng.integers(0, 100, 30_000),                 # tiny (and empty)
        rng.integers(100, 1025, 2_000),               # short
        [1024, 1025, 2048, 2049, 4096, 4097],         # mid-length edges
        rng.integers(1025, 4097, 300),                # mid-length
        rng.integers(4097, 100_000, 5),               # medium
        [300_001],                                    # huge
    ]).astype(np.int64)
    rng.shuffle(lengths)
    offsets = cuts_from_lengths(lengths, start=1)
    x = synth.fill(50 + k, int(offsets[-1]) + 3)
    assert x.size < 1024 * lengths.size  # the lean kernel
    print("many short k=%d nseg=%d n=%d" % (k, lengths.size, x.size), flush=True)
    check(x, offsets, k)
    # ties: few distinct values, and one value throughout
    check(synth.fill(60 + k, x.size, 0, 7), offsets, k)
    check(np.full(x.size, -5, np.int32), offsets, k, with_counts=False)


@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_misaligned_array_and_starts(offset):
    rng = np.random.default_rng(offset)
    lengths = rng.choice([3, 100, 4096, 4097, 9000, 300_000], size=40)
    offsets = cuts_from_lengths(lengths, start=int(rng.integers(0, 4)))
    x = synth.fill(50 + offset, int(offsets[-1]) + 3)
    check(x, offsets, 20, offset=offset)


def test_one_huge_segment_is_the_whole_top_k():
    x = synth.workload("full_1e8")[:30_000_000]
    got = check(x, [0, x.size], 50)
    assert np.array_equal(got[0], oracle.topk(x, 50))


def test_full_1e8_one_segment_and_inner_segment():
    # 1e8 elements in one segment: about a thousand parts merged by one
    # stage 2; and the same array with a huge segment inside short ones.
    x = synth.workload("full_1e8")
    got = check(x, [0, x.size], 20)
    assert np.array_equal(got[0], oracle.topk(x, 20))
    offs = [0, 10, 4000, 4000 + 97_000_000, x.size - 7, x.size]
    check(x, offs, 128)


@pytest.mark.parametrize("variant", [None, "sorted", "equal"])
def test_heavy_ties(variant):
    x = synth.workload("dup1000_1e7", variant, n=3_000_000)
    rng = np.random.default_rng(9)
    lengths = rng.choice([1, 50, 3000, 4096, 20_000, 300_000, 1_000_000],
                         size=12)
    offsets = cuts_from_lengths(lengths)
    offsets = offsets[offsets <= x.size]
    check(x, offsets, 100)


def test_equal_rows_match_batched():
    x = synth.fill(3, 97 * 1024)
    offsets = np.arange(98, dtype=np.int64) * 1024
    got = check(x, offsets, 20)
    assert np.array_equal(got, oracle.topk_batched(x.reshape(97, 1024), 20))


def test_many_tiny_segments():
    rng = np.random.default_rng(4)
    lengths = rng.integers(0, 40, 200_000)
    offsets = cuts_from_lengths(lengths)
    x = synth.fill(4, int(offsets[-1]))
    check(x, offsets, 16)
    check(x, offsets, 1)


def test_all_empty_and_no_elements():
    x = synth.fill(5, 1000)
    check(x, [17] * 40, 5)
    check(np.zeros(0, np.int32), [0, 0, 0], 3)


def test_without_counts():
    x = synth.fill(6, 500_000)
    check(x, [0, 10, 5000, 400_000, 500_000], 30, with_counts=False)


def test_int32_min_values_and_counts():
    x = np.full(10_000, I32_MIN, np.int32)
    x[5000] = 3
    got = check(x, [0, 2, 5001, 10_000], 4)
    assert got[1].tolist()[:2] == [3, I32_MIN]


def test_scratch_growth_and_two_streams():
    import torch
    small = synth.fill(8, 100_000)
    big = synth.fill(9, 6_000_000)
    for x, offs in ((small, [0, 50_000, 100_000]),
                    (big, [0, 1, 5_000_000, 6_000_000]),
                    (small, [0, 99_999, 100_000])):
        check(x, offs, 33)
    s1 = torch.cuda.Stream()
    s2 = torch.cuda.Stream()
    xd = _dev(big)
    od = _dev(np.array([0, 2_000_000, 2_000_100, 6_000_000], np.int64))
    want, _ = oracle.topk_segmented(big, [0, 2_000_000, 2_000_100, 6_000_000],
                                    64)
    outs = []
    for st in (s1, s2, s1, s2):
        with torch.cuda.stream(st):
            outs.append(ltk.topk_segmented(xd, od, 64)[0])
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy(), want)


def test_after_scramble():
    x = synth.fill(10, 3_000_000)
    offs = [0, 100, 5_000, 300_000, 2_900_000, 3_000_000]
    check(x, offs, 20)          # the segmented scratch exists now
    for seed in (3, 0xABCDEF, 2 ** 62 + 1):
        ltk.debug_scramble(0, seed)
        check(x, offs, 20)


def test_rejects_invalid_arguments():
    import torch
    x = torch.zeros(100, dtype=torch.int32, device="cuda")
    o = torch.tensor([0, 50, 100], dtype=torch.int64, device="cuda")
    out = torch.empty(2 * 129, dtype=torch.int32, device="cuda")
    assert ltk.topk_segmented_raw(x.data_ptr(), 100, o.data_ptr(), 2, 129,
                                  out.data_ptr()) == ltk.ERR_UNSUPPORTED
    assert ltk.topk_segmented_raw(x.data_ptr(), 100, o.data_ptr(), 2, 0,
                                  out.data_ptr()) == ltk.ERR_INVALID
    assert ltk.topk_segmented_raw(x.data_ptr(), 100, o.data_ptr() + 4, 2, 5,
                                  out.data_ptr()) == ltk.ERR_INVALID
    assert ltk.topk_segmented_raw(x.data_ptr(), 100, o.data_ptr(), 2, 5,
                                  x.data_ptr()) == ltk.ERR_INVALID
