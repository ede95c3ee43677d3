"""Pins for the CPU oracle, each independent of the oracle's own code.

The oracle's top-k is "sort, take the last k backwards"; its reductions are
plain loops.  The pins below come from elsewhere: the worked example printed
on the reduction page, closed forms, exhaustive brute force with a different
algorithm (repeated max extraction, Python big-int sums), invariants of the
top-k multiset, and a sort-free linear characterisation.  The last test
compiles deliberately broken copies of oracle.cpp and checks that the same
battery rejects every one of them.
"""
import itertools
import os
import re
import shutil

import numpy as np
import pytest

import oracle
from oracle import MAX, MIN, SUM

I32_MIN = -(2 ** 31)
I32_MAX = 2 ** 31 - 1
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def brute_topk(xs, k):
    """Repeated max extraction (O(nk)); shares nothing with a sort."""
    pool = list(xs)
    out = []
    for _ in range(k):
        j = max(range(len(pool)), key=lambda i: pool[i])
        out.append(pool.pop(j))
    return out


def read_kv(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = vals
    return d


# ---------------------------------------------------------------- battery
def pin_worked_example(o):
    g = read_kv("reduce_worked_example.txt")
    xs = np.array([int(v) for v in g["input"]], dtype=np.int32)
    assert g["op"] == ["sum"]
    assert o.reduce(xs, SUM) == int(g["output"][0]) == 36
    # closed forms of the same input
    assert o.reduce(xs, MAX) == 8
    assert o.reduce(xs, MIN) == 1
    assert list(o.topk(xs, 3)) == [8, 7, 6]
    assert list(o.topk(xs, 8)) == [8, 7, 6, 5, 4, 3, 2, 1]


def pin_all_ones(o):
    g = read_kv("reduce_all_ones_2p24.txt")
    n = int(g["n"][0])
    xs = np.full(n, int(g["value"][0]), dtype=np.int32)
    assert o.reduce(xs, SUM) == int(g["sum"][0]) == n
    assert o.reduce(xs, MAX) == int(g["max"][0])
    assert o.reduce(xs, MIN) == int(g["min"][0])
    assert list(o.topk(xs, 20)) == [1] * 20


def pin_exhaustive_small(o):
    alphabet = [I32_MIN, -1, 0, 1, I32_MAX]
    for n in range(1, 6):
        for xs in itertools.product(alphabet, repeat=n):
            a = np.array(xs, dtype=np.int32)
            assert o.reduce(a, SUM) == sum(xs)
            assert o.reduce(a, MAX) == max(xs)
            assert o.reduce(a, MIN) == min(xs)
            for k in range(1, n + 1):
                assert list(o.topk(a, k)) == brute_topk(xs, k), (xs, k)


def pin_empty_identities(o):
    e = np.zeros(0, dtype=np.int32)
    assert o.reduce(e, SUM) == 0
    assert o.reduce(e, MAX) == I32_MIN
    assert o.reduce(e, MIN) == I32_MAX


def pin_int64_sum(o):
    # sums far outside int32: an int32 accumulator would wrap
    for v, n in [(I32_MAX, 1000), (I32_MIN, 1000), (I32_MAX, 3)]:
        a = np.full(n, v, dtype=np.int32)
        assert o.reduce(a, SUM) == v * n
    a = np.array([I32_MAX, 1], dtype=np.int32)
    assert o.reduce(a, SUM) == 2 ** 31


def pin_closed_forms(o, rng):
    for n in [1, 2, 7, 100, 1000, 4099]:
        perm = rng.permutation(n).astype(np.int32)
        assert o.reduce(perm, SUM) == n * (n - 1) // 2
        assert o.reduce(perm, MAX) == n - 1
        assert o.reduce(perm, MIN) == 0
        for k in sorted({1, min(n, 3), min(n, 20), n}):
            assert list(o.topk(perm, k)) == list(range(n - 1, n - 1 - k, -1))
    # symmetric range sums to zero; all-negative input exercises max's start
    sym = np.arange(-5000, 5001, dtype=np.int32)
    rng.shuffle(sym)
    assert o.reduce(sym, SUM) == 0
    neg = np.arange(-100, -1, dtype=np.int32)
    assert o.reduce(neg, MAX) == -2
    assert list(o.topk(neg, 3)) == [-2, -3, -4]
    pos = np.arange(5, 100, dtype=np.int32)
    assert o.reduce(pos, MIN) == 5
    # ascending input -> last k reversed; all-equal -> k copies
    asc = np.arange(-50, 50, dtype=np.int32)
    assert list(o.topk(asc, 10)) == list(range(49, 39, -1))
    eq = np.full(77, -9, dtype=np.int32)
    assert list(o.topk(eq, 40)) == [-9] * 40


def pin_invariants(o, rng):
    for trial in range(40):
        n = int(rng.integers(1, 3000))
        hi = int(rng.choice([3, 50, 2 ** 31]))
        a = rng.integers(-hi, hi, size=n, dtype=np.int64).astype(np.int32)
        k = int(rng.integers(1, min(n, 130) + 1))
        t = o.topk(a, k)
        assert t.size == k
        assert all(t[i] >= t[i + 1] for i in range(k - 1))
        # multiset containment, with multiplicity
        vals, cnt = np.unique(a, return_counts=True)
        have = dict(zip(vals.tolist(), cnt.tolist()))
        tv, tc = np.unique(t, return_counts=True)
        for v, c in zip(tv.tolist(), tc.tolist()):
            assert have.get(v, 0) >= c
        # every excluded element is <= the k-th output
        assert int((a > t[-1]).sum()) == int((t > t[-1]).sum())
        # duplicates kept with multiplicity
        assert int((t == t[-1]).sum()) == min(have[int(t[-1])],
                                                k - int((t > t[-1]).sum()))
        # cross-op identities
        assert t[0] == o.reduce(a, MAX)
        full = o.topk(a, n)
        assert int(full.astype(np.int64).sum()) == o.reduce(a, SUM)
        assert full[-1] == o.reduce(a, MIN)
        # permutation invariance
        b = a.copy()
        rng.shuffle(b)
        assert list(o.topk(b, k)) == list(t)
        assert o.reduce(b, SUM) == o.reduce(a, SUM)
        # the linear characterisation accepts the result
        assert o.check_topk(a, k, t) == 0


def pin_checker_rejects(o, rng):
    a = rng.integers(-1000, 1000, size=5000).astype(np.int32)
    a[:7] = 999  # plant duplicates at the top
    k = 12
    t = o.topk(a, k)
    assert o.check_topk(a, k, t) == 0
    bad = t.copy()
    bad[[0, 5]] = bad[[5, 0]]
    if bad[0] != t[0]:
        assert o.check_topk(a, k, bad) == 1           # order broken
    bad = t.copy()
    bad[-1] = t[-1] - 1                               # a smaller value
    assert o.check_topk(a, k, bad) != 0
    bad = t.copy()
    bad[0] = 1000                                     # value not in input
    assert o.check_topk(a, k, bad) != 0
    dup = np.array([5, 5, 5, 1, 0], dtype=np.int32)
    assert o.check_topk(dup, 3, [5, 5, 5]) == 0
    assert o.check_topk(dup, 3, [5, 5, 1]) == 3       # a duplicate dropped
    assert o.check_topk(dup, 4, [5, 5, 5, 5]) == 2    # multiplicity exceeded
    assert o.check_topk(dup, 2, [5, 1]) != 0


def pin_stats(o, rng):
    """Statistics (count, sum, max, min, sum of squares), pinned by the
    page's worked example, closed forms, Python big-int brute force, values
    beyond 64 bits, and invariants."""
    g = read_kv("reduce_worked_example.txt")
    xs = np.array([int(v) for v in g["input"]], dtype=np.int32)
    st = o.stats(xs)
    # [1..8]: sum from the page; sum of squares n(n+1)(2n+1)/6 = 204
    assert st == {"count": 8, "sum": int(g["output"][0]), "max": 8, "min": 1,
                  "sumsq": 204}
    e = o.stats(np.zeros(0, dtype=np.int32))
    assert e == {"count": 0, "sum": 0, "max": I32_MIN, "min": I32_MAX,
                 "sumsq": 0}
    alphabet = [I32_MIN, -1, 0, 1, I32_MAX]
    for n in range(1, 5):
        for t in itertools.product(alphabet, repeat=n):
            st = o.stats(np.array(t, dtype=np.int32))
            assert st == {"count": n, "sum": sum(t), "max": max(t),
                          "min": min(t), "sumsq": sum(v * v for v in t)}, t
    for n in [1, 2, 10, 1000, 4099]:
        perm = rng.permutation(n).astype(np.int32)
        st = o.stats(perm)
        assert st["sumsq"] == (n - 1) * n * (2 * n - 1) // 6
        assert st["sum"] == n * (n - 1) // 2
    # beyond 64 bits: (-2^31)^2 = 2^62, so four of them already overflow
    assert o.stats(np.full(1000, I32_MIN, np.int32))["sumsq"] == 1000 * 2 ** 62
    assert o.stats(np.full(7, I32_MAX, np.int32))["sumsq"] == 7 * I32_MAX ** 2
    for trial in range(20):
        n = int(rng.integers(1, 5000))
        a = rng.integers(I32_MIN + 1, I32_MAX, size=n, dtype=np.int64)
        a = a.astype(np.int32)
        st = o.stats(a)
        ref = [int(v) for v in a.tolist()]
        assert st["sumsq"] == sum(v * v for v in ref)
        # cross-op with the single reductions
        assert st["sum"] == o.reduce(a, SUM)
        assert st["max"] == o.reduce(a, MAX)
        assert st["min"] == o.reduce(a, MIN)
        # permutation and negation invariance (no INT_MIN in a)
        b = a.copy()
        rng.shuffle(b)
        assert o.stats(b) == st
        neg = o.stats(-a)
        assert neg["sumsq"] == st["sumsq"] and neg["sum"] == -st["sum"]
        assert neg["max"] == -st["min"] and neg["min"] == -st["max"]
        # population variance is non-negative: n * sumsq >= sum^2
        assert n * st["sumsq"] >= st["sum"] ** 2
    eq = o.stats(np.full(50, -12345, np.int32))
    assert 50 * eq["sumsq"] == eq["sum"] ** 2   # zero variance


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def pin_topk_kv(o, rng):
    """Key-value top-k: hand examples of the tie rule (value descending,
    then position ascending), Python brute force with a different sort,
    agreement with the value-only top-k, and float order pinned by Python's
    own float comparison (-0 below +0, NaNs at the two ends)."""
    x = np.array([5, 7, 7, 3, 7], np.int32)
    v, i = o.topk_kv(x, 2)
    assert list(v) == [7, 7] and list(i) == [1, 2]
    v, i = o.topk_kv(x, 5)
    assert list(v) == [7, 7, 7, 5, 3] and list(i) == [1, 2, 4, 0, 3]
    v, i = o.topk_kv(np.full(50, -4, np.int32), 10)
    assert list(v) == [-4] * 10 and list(i) == list(range(10))
    v, i = o.topk_kv(np.arange(100, dtype=np.int32), 3)
    assert list(v) == [99, 98, 97] and list(i) == [99, 98, 97]
    for trial in range(60):
        n = int(rng.integers(1, 300))
        hi = int(rng.choice([2, 10, 2 ** 31]))
        a = rng.integers(-hi, hi, size=n, dtype=np.int64).astype(np.int32)
        k = int(rng.integers(1, n + 1))
        want = sorted(range(n), key=lambda j: (-int(a[j]), j))[:k]
        v, i = o.topk_kv(a, k)
        assert list(i) == want, (a, k)
        assert list(v) == [int(a[j]) for j in want]
        assert list(v) == list(o.topk(a, k))
    # floats: numerical order, +0 before -0, ties by position
    specials = [0.0, -0.0, np.inf, -np.inf, 1.5, -1.5, 1e-40, -1e-40,
                3.4e38, -3.4e38, 1.0, 1.0]
    for trial in range(40):
        n = int(rng.integers(1, 200))
        a = rng.choice(specials + list(rng.normal(size=8)), size=n)
        a = a.astype(np.float32)
        k = int(rng.integers(1, n + 1))

        def key(j):
            f = float(a[j])
            return (-f, 1 if (f == 0.0 and np.signbit(a[j])) else 0, j)
        want = sorted(range(n), key=key)[:k]
        v, i = o.topk_kv(a, k)
        assert list(i) == want, (a, k)
        assert v.view(np.uint32).tolist() == a[want].view(np.uint32).tolist()
    # NaNs: a positive NaN ranks above +inf, a negative one below -inf
    pnan, nnan = _f32(0x7FC00000), _f32(0xFFC00000)
    a = np.array([1.0, nnan, np.inf, pnan, -np.inf], np.float32)
    v, i = o.topk_kv(a, 5)
    assert list(i) == [3, 2, 0, 4, 1]


def np_topk_rows(x, k):
    """numpy's own sort along rows, read backwards: a library routine that
    shares nothing with the oracle's std::sort."""
    return np.sort(np.asarray(x, dtype=np.int64), axis=1)[:, ::-1][:, :k]


def pin_topk_batched(o, rng):
    """Per-row top-k: a hand example, numpy's sort along rows, exhaustive
    brute force on tiny matrices, and the row stride: columns past `cols`
    (filled with INT32_MAX here) must never reach the result."""
    x = np.array([[3, 1, 2], [9, 9, 0]], np.int32)
    assert o.topk_batched(x, 2).tolist() == [[3, 2], [9, 9]]
    assert o.topk_batched(x, 3).tolist() == [[3, 2, 1], [9, 9, 0]]
    assert o.topk_batched(x, 1, cols=2).tolist() == [[3], [9]]
    assert o.topk_batched(np.zeros((0, 4), np.int32), 2).shape == (0, 2)
    alphabet = [I32_MIN, -1, 0, I32_MAX]
    for cols in (1, 2, 3):
        for flat in itertools.product(alphabet, repeat=2 * cols):
            a = np.array(flat, np.int32).reshape(2, cols)
            for k in range(1, cols + 1):
                got = o.topk_batched(a, k).tolist()
                assert got == [brute_topk(a[0], k), brute_topk(a[1], k)]
    for trial in range(40):
        rows = int(rng.integers(1, 40))
        cols = int(rng.integers(1, 300))
        pad = int(rng.integers(0, 5))
        hi = int(rng.choice([3, 1000, 2 ** 31]))
        a = rng.integers(-hi, hi, size=(rows, cols), dtype=np.int64)
        a = a.astype(np.int32)
        k = int(rng.integers(1, cols + 1))
        want = np_topk_rows(a, k)
        assert (o.topk_batched(a, k) == want).all()
        wide = np.full((rows, cols + pad), I32_MAX, np.int32)
        wide[:, :cols] = a
        assert (o.topk_batched(wide, k, cols=cols) == want).all()


def pin_topk_merge(o, rng):
    """Merging top-k lists: hand examples, and the two-stage lemma itself
    (the top-k of the union of every shard's top-k is the top-k of the
    whole), with numpy's sort on both sides; a list out of order is
    refused."""
    lists = np.array([[9, 5, 1], [7, 6, 2]], np.int32)
    assert o.topk_merge(lists, 3).tolist() == [9, 7, 6]
    assert o.topk_merge(lists, 6).tolist() == [9, 7, 6, 5, 2, 1]
    assert o.topk_merge(np.array([[5, 5], [5, 4]], np.int32), 3).tolist() \
        == [5, 5, 5]
    assert o.topk_merge(np.array([[4], [8], [-3]], np.int32), 3).tolist() \
        == [8, 4, -3]
    refused = False
    try:
        o.topk_merge(np.array([[3, 1], [1, 2]], np.int32), 1)
    except ValueError:
        refused = True
    assert refused, "a list out of order must be refused"
    for trial in range(40):
        m = int(rng.integers(1, 30))
        size = int(rng.integers(1, 200))
        k = int(rng.integers(1, min(size, 128) + 1))
        hi = int(rng.choice([3, 1000, 2 ** 31]))
        shards = rng.integers(-hi, hi, size=(m, size), dtype=np.int64)
        shards = shards.astype(np.int32)
        tops = np_topk_rows(shards, k).astype(np.int32)
        want = np.sort(shards.ravel().astype(np.int64))[::-1][:k]
        assert o.topk_merge(tops, k).tolist() == want.tolist()
        kk = int(rng.integers(1, m * k + 1))
        whole = np.sort(tops.ravel().astype(np.int64))[::-1][:kk]
        assert o.topk_merge(tops, kk).tolist() == whole.tolist()


def pin_histogram(o, rng):
    """Histogram: hand examples, numpy's own histogram with integer bin
    edges (a library routine sharing nothing with the oracle's loop),
    closed forms over permutations, the extremes of int32, and brute force
    over tiny inputs."""
    x = np.array([0, 1, 1, 2, 255, 256, -1, 7, 7, 7], np.int32)
    assert o.histogram(x, 0, 0, 256)[[0, 1, 2, 7, 255]].tolist() == \
        [1, 2, 1, 3, 1]
    assert o.histogram(x, 0, 0, 256).sum() == 8        # -1 and 256 fall out
    assert o.histogram(x, 0, 3, 2).tolist() == [7, 0]  # [0, 8) and [8, 16)
    assert o.histogram(x, -1, 8, 2).tolist() == [8, 2]  # [-1, 255), [255, 511)
    assert o.histogram(np.zeros(0, np.int32), 0, 0, 4).tolist() == [0] * 4
    full = np.array([I32_MIN, -1, 0, I32_MAX], np.int32)
    assert o.histogram(full, I32_MIN, 31, 2).tolist() == [2, 2]
    assert o.histogram(full, I32_MAX, 0, 1).tolist() == [1]
    assert o.histogram(full, I32_MIN, 0, 1).tolist() == [1]
    for trial in range(40):
        n = int(rng.integers(0, 3000))
        spread = int(rng.choice([10, 1000, 2 ** 31]))
        a = rng.integers(-spread, spread, size=n, dtype=np.int64)
        a = a.astype(np.int32)
        lo = int(rng.integers(-spread, spread))
        shift = int(rng.integers(0, 24))
        nbins = int(rng.integers(1, 5000))
        edges = lo + (np.arange(nbins + 1, dtype=np.float64) * 2.0 ** shift)
        want, _ = np.histogram(a.astype(np.float64), bins=edges - 0.5)
        assert o.histogram(a, lo, shift, nbins).tolist() == want.tolist()
    for s in (0, 3, 10):
        n = 5000
        perm = rng.permutation(n).astype(np.int32)
        h = o.histogram(perm, 0, s, (n >> s) + 2)
        w = 1 << s
        assert h[: n // w].tolist() == [w] * (n // w)
        assert h.sum() == n
    for xs in itertools.product([I32_MIN, -3, 0, 5, I32_MAX], repeat=3):
        a = np.array(xs, np.int32)
        for lo, shift, nbins in ((-4, 1, 5), (I32_MIN, 30, 4), (0, 0, 6)):
            want = [sum(1 for v in xs
                        if lo + b * 2 ** shift <= v < lo + (b + 1) * 2 ** shift)
                    for b in range(nbins)]
            assert o.histogram(a, lo, shift, nbins).tolist() == want


def pin_topk_segmented(o, rng):
    """Segmented top-k: a hand example (empty and short segments, padding
    and counts), repeated max extraction per segment over random
    segmentations (brute force sharing nothing with a sort), numpy's sort
    per segment on larger ones, equal segments against per-row top-k, one
    segment against the whole array's top-k, and the two-stage lemma (the
    top-k of the union of the segments' lists is the top-k of the whole);
    offsets out of order are refused."""
    x = np.array([5, 1, 9, 9, 3, 7, 2], np.int32)
    out, cnt = o.topk_segmented(x, [0, 3, 3, 7], 2)
    assert out.tolist() == [[9, 5], [I32_MIN, I32_MIN], [9, 7]]
    assert cnt.tolist() == [2, 0, 2]
    out, cnt = o.topk_segmented(x, [1, 2, 6], 3)     # [1] and [9, 9, 3, 7]
    assert out.tolist() == [[1, I32_MIN, I32_MIN], [9, 9, 7]]
    assert cnt.tolist() == [1, 3]
    out, cnt = o.topk_segmented(np.array([I32_MIN, 4], np.int32), [0, 1, 2], 2)
    assert out.tolist() == [[I32_MIN, I32_MIN], [4, I32_MIN]]
    assert cnt.tolist() == [1, 1]
    out, cnt = o.topk_segmented(x, [4], 5)            # no segments
    assert out.shape == (0, 5) and cnt.size == 0
    for bad in ([0, 5, 3], [-1, 2], [0, 8]):
        refused = False
        try:
            o.topk_segmented(x, bad, 1)
        except ValueError:
            refused = True
        assert refused, "offsets %s must be refused" % bad
    for trial in range(60):
        n = int(rng.integers(0, 40))
        hi = int(rng.choice([2, 5, 2 ** 31]))
        a = rng.integers(-hi, hi, size=n, dtype=np.int64).astype(np.int32)
        nseg = int(rng.integers(0, 8))
        cuts = np.sort(rng.integers(0, n + 1, size=nseg + 1))
        k = int(rng.integers(1, 8))
        out, cnt = o.topk_segmented(a, cuts, k)
        for s in range(nseg):
            seg = a[cuts[s]:cuts[s + 1]].tolist()
            m = min(k, len(seg))
            assert out[s].tolist() == brute_topk(seg, m) + [I32_MIN] * (k - m)
            assert cnt[s] == m
    for trial in range(20):
        n = int(rng.integers(1, 20000))
        a = rng.integers(-2 ** 31, 2 ** 31, size=n, dtype=np.int64)
        a = a.astype(np.int32)
        nseg = int(rng.integers(1, 60))
        cuts = np.sort(rng.integers(0, n + 1, size=nseg + 1))
        k = int(rng.integers(1, 129))
        out, cnt = o.topk_segmented(a, cuts, k)
        for s in range(nseg):
            seg = np.sort(a[cuts[s]:cuts[s + 1]].astype(np.int64))[::-1][:k]
            assert out[s, :seg.size].tolist() == seg.tolist()
            assert (out[s, seg.size:] == I32_MIN).all()
        live = out[out > I32_MIN]
        whole = np.sort(a[cuts[0]:cuts[-1]].astype(np.int64))[::-1][:k]
        assert np.sort(live.astype(np.int64))[::-1][:whole.size][
            :np.count_nonzero(whole > I32_MIN)].tolist() == \
            whole[whole > I32_MIN].tolist()
    rows = rng.integers(-1000, 1000, size=(7, 90), dtype=np.int64)
    rows = rows.astype(np.int32)
    out, cnt = o.topk_segmented(rows.ravel(), np.arange(8) * 90, 13)
    assert (out == np_topk_rows(rows, 13)).all() and (cnt == 13).all()
    a = rng.integers(-2 ** 31, 2 ** 31, size=5000, dtype=np.int64)
    a = a.astype(np.int32)
    out, cnt = o.topk_segmented(a, [0, 5000], 40)
    assert out[0].tolist() == np.sort(a.astype(np.int64))[::-1][:40].tolist()


BATTERY = [pin_worked_example, pin_all_ones, pin_exhaustive_small,
           pin_empty_identities, pin_int64_sum, pin_closed_forms,
           pin_invariants, pin_checker_rejects, pin_stats, pin_topk_kv,
           pin_topk_batched, pin_topk_merge, pin_histogram,
           pin_topk_segmented]


def run_battery(o, seed=7):
    for pin in BATTERY:
        args = (o,) if pin.__code__.co_argcount == 1 else (
            o, np.random.default_rng(seed))
        pin(*args)


# ---------------------------------------------------------------- tests
@pytest.mark.parametrize("pin", BATTERY, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    o = oracle.default()
    if pin.__code__.co_argcount == 1:
        pin(o)
    else:
        pin(o, np.random.default_rng(7))


def test_oracle_rejects_bad_arguments():
    o = oracle.default()
    a = np.arange(5, dtype=np.int32)
    for k in (0, -1, 6):
        with pytest.raises(ValueError):
            o.topk(a, k)
    with pytest.raises(ValueError):
        o.reduce(a, 3)


# Plausible mistakes, each planted in a private copy of oracle.cpp.  The
# battery must reject every mutant; if one survived, the pins would not be
# able to tell that mistake from the correct oracle.
MUTANTS = {
    "int32_sum_accumulator": (r"int64_t s = 0;", "int32_t s = 0;"),
    "ascending_output": (r"out\[i\] = v\[\(size_t\)\(n - 1 - i\)\];",
                         "out[i] = v[(size_t)i];"),
    "duplicates_dropped": (
        r"std::sort\(v.begin\(\), v.end\(\)\);",
        "std::sort(v.begin(), v.end()); v.erase(std::unique(v.begin(), "
        "v.end()), v.end()); v.insert(v.begin(), (size_t)n - v.size(), "
        "INT32_MIN);"),
    "max_starts_at_zero": (r"int32_t m = INT32_MIN;", "int32_t m = 0;"),
    "min_starts_at_zero": (r"int32_t m = INT32_MAX;", "int32_t m = 0;"),
    "sum_skips_last": (r"for \(int64_t i = 0; i < n; \+\+i\)\n            s \+=",
                       "for (int64_t i = 0; i + 1 < n; ++i)\n            s +="),
    "wrong_identity_sum": (r"int64_t s = 0;", "int64_t s = 1;"),
    "checker_counts_ties_as_above": (r"if \(x > t\)\n            \+\+above_in;",
                                     "if (x >= t)\n            ++above_in;"),
    "checker_ignores_multiplicity": (r"if \(want\[d\] > have\[d\]\)",
                                     "if (have[d] == 0)"),
    "topk_off_by_one": (r"out\[i\] = v\[\(size_t\)\(n - 1 - i\)\];",
                        "out[i] = v[(size_t)(n - 1 - (i > 0 ? i - 1 : 0))];"),
    "sumsq_in_64_bits": (r"unsigned __int128 sq = 0;", "uint64_t sq = 0;"),
    "sumsq_of_abs": (r"sq \+= \(unsigned __int128\)\(uint64_t\)\(x \* x\);",
                     "sq += (unsigned __int128)(uint64_t)(x < 0 ? -x : x);"),
    "sumsq_skips_first": (r"sq \+= \(unsigned __int128\)",
                          "if (i > 0) sq += (unsigned __int128)"),
    "stats_max_starts_at_zero": (r"int32_t mx = INT32_MIN, mn = INT32_MAX;",
                                 "int32_t mx = 0, mn = INT32_MAX;"),
    "stats_min_starts_at_zero": (r"int32_t mx = INT32_MIN, mn = INT32_MAX;",
                                 "int32_t mx = INT32_MIN, mn = 0;"),
    "kv_ties_by_larger_index": (
        r"std::stable_sort\(pos.begin\(\), pos.end\(\),\n\s*\[in\]\(int64_t a, int64_t b\) \{ return in\[a\] > in\[b\]; \}\);",
        "std::sort(pos.begin(), pos.end(), [in](int64_t a, int64_t b) "
        "{ return in[a] > in[b] || (in[a] == in[b] && a > b); });"),
    "kv_index_off_by_one": (r"out_i\[i\] = pos\[\(size_t\)i\];\n        out_v\[i\] = in",
                            "out_i[i] = pos[(size_t)i] + (i > 0);\n        out_v[i] = in"),
    "kv_float_raw_bits": (r"key\[\(size_t\)i\] = \(b & 0x80000000u\) \? ~b : \(b \| 0x80000000u\);",
                          "key[(size_t)i] = b;"),
    "kv_float_sign_only": (r"key\[\(size_t\)i\] = \(b & 0x80000000u\) \? ~b : \(b \| 0x80000000u\);",
                           "key[(size_t)i] = b ^ 0x80000000u;"),
    "batched_ignores_row_stride": (r"const int32_t \*row = in \+ r \* ld;",
                                   "const int32_t *row = in + r * cols;"),
    "batched_reads_past_cols": (
        r"std::vector<int32_t> v\(row, row \+ cols\);",
        "std::vector<int32_t> v(row, row + cols + (cols < ld ? 1 : 0));"),
    "batched_rows_shifted": (r"out\[r \* k \+ i\] = v",
                             "out[(r + 1 < rows ? r + 1 : r) * k + i] = v"),
    "merge_drops_last_list": (
        r"std::vector<int32_t> v\(lists, lists \+ total\);",
        "std::vector<int32_t> v(lists, lists + total); if (m > 1) for "
        "(int32_t i = 0; i < len; ++i) v[(size_t)(total - len + i)] = "
        "INT32_MIN;"),
    "merge_accepts_unsorted": (r"return -2;", "(void)0;"),
    "merge_ascending": (r"out\[i\] = v\[\(size_t\)\(total - 1 - i\)\];",
                        "out[i] = v[(size_t)(total - k + i)];"),
    "segmented_end_past_segment": (
        r"std::vector<int32_t> v\(in \+ a, in \+ b\);",
        "std::vector<int32_t> v(in + a, in + (b < n ? b + 1 : b));"),
    "segmented_skips_first": (
        r"std::vector<int32_t> v\(in \+ a, in \+ b\);",
        "std::vector<int32_t> v(in + (a < b ? a + 1 : a), in + b);"),
    "segmented_pads_with_zero": (r"out\[s \* k \+ i\] = INT32_MIN;",
                                 "out[s * k + i] = 0;"),
    "segmented_counts_length": (r"counts\[s\] = \(int32_t\)have;",
                                "counts[s] = (int32_t)len;"),
    "segmented_ascending": (r"out\[s \* k \+ i\] = v\[\(size_t\)\(len - 1 - i\)\];",
                            "out[s * k + i] = v[(size_t)(len - have + i)];"),
    "segmented_drops_last_segment": (r"for \(int64_t s = 0; s < nseg; \+\+s\) \{\n        const int64_t a",
                                     "for (int64_t s = 0; s < nseg; ++s) {\n        if (s == nseg - 1 && s > 0) { for (int32_t i = 0; i < k; ++i) out[s * k + i] = INT32_MIN; if (counts) counts[s] = 0; continue; }\n        const int64_t a"),
    "histogram_off_by_one_bin": (r"const int64_t b = d / width;",
                                 "const int64_t b = (d + 1) / width;"),
    "histogram_keeps_last_edge": (r"if \(b < nbins\)\n            \+\+out\[b\];",
                                  "if (b <= nbins - 1 || d == nbins * width)\n"
                                  "            ++out[b < nbins ? b : nbins - 1];"),
    "histogram_wraps_in_32_bits": (
        r"const int64_t d = \(int64_t\)in\[i\] - \(int64_t\)lo;",
        "const int64_t d = (int32_t)((uint32_t)in[i] - (uint32_t)lo);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_battery_rejects_mutant(name, tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__),
                            "oracle.cpp")).read()
    pat, rep = MUTANTS[name]
    mutated, count = re.subn(pat, rep, src, count=1)
    assert count == 1, "mutation pattern %s no longer matches" % name
    so = oracle.compile_oracle_source(mutated, str(tmp_path / "mut.so"))
    o = oracle.Oracle(so)
    with pytest.raises(AssertionError):
        run_battery(o)
