/*
 * CPU oracle for the two-stage reduction / Top-K path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library, and it is plain single-threaded C++ built by
 * g++.
 *
 * Sources (the pages the method is taken from):
 *   [TopK]   "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计"
 *            (CUDA optimisation in practice: shared memory and reduction
 *            design through the TopK problem).
 *   [Reduce] "CUDA归约优化完全指南：从入门到精通"
 *            (A complete guide to CUDA reduction optimisation).
 *
 * Every result here has a plain definition, so the oracle is that definition
 * written out, with a library sort as its one primitive:
 *
 *   oracle_topk_i32   the k largest values of the input in descending order,
 *                     duplicates kept with their multiplicity ([TopK] §1: the
 *                     20 largest of 1e8 values; §2.1: each thread keeps its
 *                     list in descending order and thread 0 writes the
 *                     block's list out in that order; §2.2: the GPU result
 *                     must be identical to the CPU's; §5.2: duplicate
 *                     elements must be handled).  Definition: sort a copy
 *                     ascending, read the last k backwards.
 *
 *   oracle_reduce_i32 folding the array with a binary operator ([Reduce],
 *                     "Basic concepts": a reduction combines all elements
 *                     with one binary operation into a single result; the
 *                     worked example sums [1..8] to 36).  Sum is accumulated
 *                     in int64 so that it cannot overflow for n <= 2^32
 *                     (the page's own int accumulator would); max and min
 *                     start from the int32 extremes and are returned
 *                     sign-extended to int64.
 *
 *   oracle_stats_i32  the statistics of one array in one call: count, sum,
 *                     max, min and the sum of squares, from which mean and
 *                     (population) variance follow ([TopK] §6: the same
 *                     two-stage reduction serves large-scale statistics
 *                     such as the mean and the variance; [Reduce], "Basic
 *                     concepts": each of these is a fold of the array with
 *                     one binary operator).  Definition: four independent
 *                     folds, each written out; the sum of squares is
 *                     accumulated exactly in unsigned 128-bit arithmetic
 *                     (x^2 <= 2^62, so n <= 2^32 elements stay below 2^94).
 *
 *   oracle_topk_kv_i32, oracle_topk_kv_f32
 *                     the k largest values together with their positions
 *                     in the input ([TopK] §6: the reduction keeps a
 *                     candidate list of items ordered by their score;
 *                     "GPU基数排序优化：10亿级数据处理与性能调优" §8: key-value
 *                     pairs, and floating-point keys through a suitable bit
 *                     transform).  With indices the answer is no longer
 *                     unique under ties, so a rule is fixed: order by value,
 *                     descending, and among equal values by index,
 *                     ascending (the earlier element first).  Definition: a
 *                     stable sort of the positions by value, descending,
 *                     then the first k.  Float scores are ordered by the
 *                     usual order-preserving map of their bits to unsigned
 *                     integers (negative: all bits flipped; otherwise the
 *                     sign bit set), which agrees with numerical order on
 *                     numbers and puts -0 below +0, positive NaNs above
 *                     +infinity and negative NaNs below -infinity.
 *
 *   oracle_topk_batched_i32
 *                     the top-k of every row of a row-major matrix: rows
 *                     r = 0..rows-1 of `cols` values each, row r starting
 *                     at in[r * ld] ([TopK] §6: the two-stage pattern is a
 *                     building block, for instance candidate selection per
 *                     user in a recommender).  Definition: for each row,
 *                     the row's top-k exactly as oracle_topk_i32 defines
 *                     it, written to out[r * k .. r * k + k).  Elements
 *                     between cols and ld of a row are not part of it.
 *
 *   oracle_topk_merge_i32
 *                     merging several top-k results into one ([TopK] §6:
 *                     several TopK results merged again; §2.2: stage 2
 *                     merges the per-block top-k lists into the final
 *                     one).  Input: m lists of `len` values each, row-major
 *                     and contiguous, each in descending order (as the
 *                     top-k calls write them).  Result: the k largest
 *                     values of the union of the lists, descending --
 *                     by definition, sort all m * len values and read the
 *                     last k backwards.  A list that is not in descending
 *                     order is a caller error, reported as such.
 *
 *   oracle_topk_segmented_i32
 *                     the top-k of every segment of one array, segments of
 *                     different lengths given by offsets ([TopK] §6: the
 *                     two-stage pattern as a building block, for instance
 *                     candidate selection per user, whose candidate lists
 *                     differ in length; several TopK results merged
 *                     again).  Segment s is in[offsets[s] .. offsets[s+1]),
 *                     with 0 <= offsets[0] <= ... <= offsets[nseg] <= n.
 *                     Definition: for each segment, sort a copy ascending
 *                     and read its last min(k, len) values backwards into
 *                     out[s * k ..]; a segment shorter than k has all its
 *                     values there, the remaining slots hold INT32_MIN,
 *                     and counts[s] = min(k, len) tells them apart from
 *                     real INT32_MIN values.  Offsets out of order are a
 *                     caller error, reported as such.
 *
 *   oracle_histogram_i32
 *                     counts of the values falling into equal-width bins
 *                     ([TopK] §6: histogram computation as a use of the
 *                     two-stage reduction; "GPU基数排序优化：10亿级数据处理与
 *                     性能调优" §3.3: per-warp histograms merged at the end).
 *                     Bin b covers the integers lo + b * 2^shift up to
 *                     lo + (b + 1) * 2^shift - 1; values outside all nbins
 *                     bins are not counted.  Definition: one loop over the
 *                     input, each value's bin found by subtracting lo (in
 *                     64-bit arithmetic, so nothing wraps) and dividing by
 *                     the bin width.
 *
 *   oracle_check_topk a second, sort-free characterisation of the top-k
 *                     multiset, linear in n.  It is used to check results
 *                     at sizes where sorting is too slow, and as an
 *                     independent pin for oracle_topk_i32.  A candidate o of
 *                     length k is the top-k of `in` iff
 *                       (1) o is non-increasing;
 *                       (2) every value occurs in o at most as often as in
 *                           `in`;
 *                       (3) #{x in in : x > o[k-1]} == #{i : o[i] > o[k-1]}.
 *                     (1)-(3) force o's elements above t = o[k-1] to be
 *                     exactly the input's elements above t, and the rest of
 *                     o to be copies of t that the input holds.
 *
 * Values are compared as signed int32 throughout.
 */
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

extern "C" {

/* Returns 0 on success, -1 on invalid arguments (null pointers, n < 0,
 * k < 1, k > n).  out receives k values, largest first. */
int oracle_topk_i32(const int32_t *in, int64_t n, int32_t k, int32_t *out)
{
    if (!in || !out || n < 0 || k < 1 || (int64_t)k > n)
        return -1;
    std::vector<int32_t> v(in, in + n);
    std::sort(v.begin(), v.end());
    for (int32_t i = 0; i < k; ++i)
        out[i] = v[(size_t)(n - 1 - i)];
    return 0;
}

/* op: 0 = sum (int64), 1 = max, 2 = min.  n == 0 yields the operator's
 * identity: 0, INT32_MIN, INT32_MAX.  Returns 0, or -1 on invalid
 * arguments. */
int oracle_reduce_i32(const int32_t *in, int64_t n, int32_t op, int64_t *out)
{
    if (!out || n < 0 || (n > 0 && !in) || op < 0 || op > 2)
        return -1;
    if (op == 0) {
        int64_t s = 0;
        for (int64_t i = 0; i < n; ++i)
            s += (int64_t)in[i];
        *out = s;
    } else if (op == 1) {
        int32_t m = INT32_MIN;
        for (int64_t i = 0; i < n; ++i)
            if (in[i] > m)
                m = in[i];
        *out = (int64_t)m;
    } else {
        int32_t m = INT32_MAX;
        for (int64_t i = 0; i < n; ++i)
            if (in[i] < m)
                m = in[i];
        *out = (int64_t)m;
    }
    return 0;
}

/* out[0] = n; out[1] = sum (int64); out[2] = max and out[3] = min,
 * sign-extended (INT32_MIN and INT32_MAX when n == 0); out[4] and out[5] =
 * the low and high 64 bits of the sum of squares, an unsigned 128-bit
 * integer.  Returns 0, or -1 on invalid arguments. */
int oracle_stats_i32(const int32_t *in, int64_t n, int64_t *out)
{
    if (!out || n < 0 || (n > 0 && !in))
        return -1;
    int64_t s = 0;
    int32_t mx = INT32_MIN, mn = INT32_MAX;
    unsigned __int128 sq = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t x = in[i];
        s += x;
        if (in[i] > mx)
            mx = in[i];
        if (in[i] < mn)
            mn = in[i];
        sq += (unsigned __int128)(uint64_t)(x * x);
    }
    out[0] = n;
    out[1] = s;
    out[2] = (int64_t)mx;
    out[3] = (int64_t)mn;
    out[4] = (int64_t)(uint64_t)sq;
    out[5] = (int64_t)(uint64_t)(sq >> 64);
    return 0;
}

/* out_v[i], out_i[i] for i < k: the value and the position of the i-th
 * element in the order (value descending, position ascending).  Returns 0,
 * or -1 on invalid arguments (null pointers, n < 0, k < 1, k > n). */
int oracle_topk_kv_i32(const int32_t *in, int64_t n, int32_t k,
                       int32_t *out_v, int64_t *out_i)
{
    if (!in || !out_v || !out_i || n < 0 || k < 1 || (int64_t)k > n)
        return -1;
    std::vector<int64_t> pos((size_t)n);
    for (int64_t i = 0; i < n; ++i)
        pos[(size_t)i] = i;
    std::stable_sort(pos.begin(), pos.end(),
                     [in](int64_t a, int64_t b) { return in[a] > in[b]; });
    for (int32_t i = 0; i < k; ++i) {
        out_i[i] = pos[(size_t)i];
        out_v[i] = in[pos[(size_t)i]];
    }
    return 0;
}

/* The same for float scores, ordered through their bit patterns (see
 * above); out_v receives the input's own bits. */
int oracle_topk_kv_f32(const float *in, int64_t n, int32_t k, float *out_v,
                       int64_t *out_i)
{
    if (!in || !out_v || !out_i || n < 0 || k < 1 || (int64_t)k > n)
        return -1;
    std::vector<uint32_t> key((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b;
        std::memcpy(&b, &in[i], sizeof b);
        key[(size_t)i] = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
    std::vector<int64_t> pos((size_t)n);
    for (int64_t i = 0; i < n; ++i)
        pos[(size_t)i] = i;
    std::stable_sort(pos.begin(), pos.end(), [&key](int64_t a, int64_t b) {
        return key[(size_t)a] > key[(size_t)b];
    });
    for (int32_t i = 0; i < k; ++i) {
        out_i[i] = pos[(size_t)i];
        std::memcpy(&out_v[i], &in[pos[(size_t)i]], sizeof(float));
    }
    return 0;
}

/* Returns 0 if cand[0..k) is exactly the top-k of in[0..n) in descending
 * order; 1, 2 or 3 naming the first condition above that fails; -1 on
 * invalid arguments. */
int oracle_check_topk(const int32_t *in, int64_t n, int32_t k,
                      const int32_t *cand)
{
    if (!in || !cand || n < 0 || k < 1 || (int64_t)k > n)
        return -1;
    for (int32_t i = 1; i < k; ++i)
        if (cand[i] > cand[i - 1])
            return 1;
    const int32_t t = cand[k - 1];

    /* distinct values of cand (already sorted descending) and their counts */
    std::vector<int32_t> val;
    std::vector<int64_t> want;
    for (int32_t i = 0; i < k; ++i) {
        if (val.empty() || val.back() != cand[i]) {
            val.push_back(cand[i]);
            want.push_back(0);
        }
        ++want.back();
    }
    std::vector<int64_t> have(val.size(), 0);

    int64_t above_in = 0;
    for (int64_t j = 0; j < n; ++j) {
        const int32_t x = in[j];
        if (x < t)
            continue;
        if (x > t)
            ++above_in;
        /* val is descending: find x by binary search */
        size_t lo = 0, hi = val.size();
        while (lo < hi) {
            size_t mid = (lo + hi) / 2;
            if (val[mid] > x)
                lo = mid + 1;
            else
                hi = mid;
        }
        if (lo < val.size() && val[lo] == x)
            ++have[lo];
    }
    for (size_t d = 0; d < val.size(); ++d)
        if (want[d] > have[d])
            return 2;
    int64_t above_cand = 0;
    for (int32_t i = 0; i < k; ++i)
        if (cand[i] > t)
            ++above_cand;
    if (above_in != above_cand)
        return 3;
    return 0;
}

/* out[r * k + i], i < k: the i-th largest value of row r, which is
 * in[r * ld .. r * ld + cols).  Returns 0, or -1 on invalid arguments
 * (null pointers, rows < 0, cols < 1, ld < cols, k < 1, k > cols). */
int oracle_topk_batched_i32(const int32_t *in, int64_t rows, int64_t cols,
                            int64_t ld, int32_t k, int32_t *out)
{
    if (!in || !out || rows < 0 || cols < 1 || ld < cols || k < 1 ||
        (int64_t)k > cols)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t *row = in + r * ld;
        std::vector<int32_t> v(row, row + cols);
        std::sort(v.begin(), v.end());
        for (int32_t i = 0; i < k; ++i)
            out[r * k + i] = v[(size_t)(cols - 1 - i)];
    }
    return 0;
}

/* out[0..k): the k largest of the m * len values of lists[], descending.
 * Returns 0; -1 on invalid arguments (null pointers, m < 1, len < 1,
 * k < 1, k > m * len); -2 if some list is not in descending order. */
int oracle_topk_merge_i32(const int32_t *lists, int64_t m, int32_t len,
                          int32_t k, int32_t *out)
{
    if (!lists || !out || m < 1 || len < 1 || k < 1 ||
        (int64_t)k > m * (int64_t)len)
        return -1;
    for (int64_t j = 0; j < m; ++j)
        for (int32_t i = 1; i < len; ++i)
            if (lists[j * len + i] > lists[j * len + i - 1])
                return -2;
    const int64_t total = m * (int64_t)len;
    std::vector<int32_t> v(lists, lists + total);
    std::sort(v.begin(), v.end());
    for (int32_t i = 0; i < k; ++i)
        out[i] = v[(size_t)(total - 1 - i)];
    return 0;
}

/* out[s * k + i], i < min(k, len_s): the i-th largest value of segment s,
 * which is in[offsets[s] .. offsets[s + 1]); out[s * k + i] = INT32_MIN for
 * len_s <= i < k; counts[s] = min(k, len_s) (counts may be NULL).  Returns
 * 0; -1 on invalid arguments (null pointers, n < 0, nseg < 0, k < 1); -2 if
 * the offsets are not non-decreasing within [0, n]. */
int oracle_topk_segmented_i32(const int32_t *in, int64_t n,
                              const int64_t *offsets, int64_t nseg,
                              int32_t k, int32_t *out, int32_t *counts)
{
    if (!offsets || n < 0 || nseg < 0 || k < 1 || (nseg > 0 && !out) ||
        (n > 0 && !in))
        return -1;
    if (offsets[0] < 0 || offsets[nseg] > n)
        return -2;
    for (int64_t s = 0; s < nseg; ++s)
        if (offsets[s + 1] < offsets[s])
            return -2;
    for (int64_t s = 0; s < nseg; ++s) {
        const int64_t a = offsets[s], b = offsets[s + 1];
        std::vector<int32_t> v(in + a, in + b);
        std::sort(v.begin(), v.end());
        const int64_t len = b - a;
        const int64_t have = len < (int64_t)k ? len : (int64_t)k;
        for (int64_t i = 0; i < have; ++i)
            out[s * k + i] = v[(size_t)(len - 1 - i)];
        for (int64_t i = have; i < k; ++i)
            out[s * k + i] = INT32_MIN;
        if (counts)
            counts[s] = (int32_t)have;
    }
    return 0;
}

/* out[b] for b < nbins: how many values v of in[0..n) have
 * lo + b * 2^shift <= v < lo + (b + 1) * 2^shift.  Returns 0, or -1 on
 * invalid arguments (null pointers, n < 0, shift outside 0..31, nbins < 1). */
int oracle_histogram_i32(const int32_t *in, int64_t n, int32_t lo,
                         int32_t shift, int32_t nbins, int64_t *out)
{
    if (!out || n < 0 || (n > 0 && !in) || shift < 0 || shift > 31 ||
        nbins < 1)
        return -1;
    const int64_t width = (int64_t)1 << shift;
    for (int32_t b = 0; b < nbins; ++b)
        out[b] = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t d = (int64_t)in[i] - (int64_t)lo;
        if (d < 0)
            continue;
        const int64_t b = d / width;
        if (b < nbins)
            ++out[b];
    }
    return 0;
}

} /* extern "C" */
