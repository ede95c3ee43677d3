/*
 * libtopk — two-stage parallel reduction and Top-K selection over int32
 * arrays on AMD Instinct MI355X (gfx950).  C ABI, no C++ or PyTorch types.
 *
 * Sources (the pages the method is taken from):
 *   [TopK]   "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计"
 *            (CUDA optimisation in practice: shared memory and reduction
 *            design through the TopK problem)
 *   [Reduce] "CUDA归约优化完全指南：从入门到精通"
 *            (A complete guide to CUDA reduction optimisation)
 *
 * Common conventions
 * ------------------
 *  - `in`, `out` and `out_i64` are DEVICE pointers on the calling thread's
 *    current HIP device.  They are owned by the caller; the library never
 *    frees or retains them.  `in` must be 4-byte aligned (16-byte alignment
 *    takes the fastest path; otherwise up to three leading elements are
 *    peeled).  `in` and the output must not overlap.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Both calls are
 *    asynchronous and stream-ordered: they return once the work is enqueued
 *    and never synchronise the host.  The result is valid once the stream
 *    reaches the call; `in` must stay alive and unmodified until then.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is launched and the output is untouched.  Launch and
 *    allocation failures are reported as LIBTOPK_ERR_HIP / _NOMEM; a fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - The library owns a small scratch area per (device, stream), about
 *    1.6 MiB: per-block candidates (1.5 MiB, int32 and key-value), partial
 *    results, histogram counters and tickets; the first topk_i32 call with
 *    k > LIBTOPK_MAX_K on the pair adds a 16 MiB candidate buffer (and
 *    64 KiB for sample lists).  It is
 *    allocated by the
 *    first call on that pair (so do that first call before capturing the
 *    stream into a HIP graph), kept for reuse, and freed by
 *    libtopk_release() or at process exit.  No per-call clearing is
 *    enqueued: the words that the workgroups of one launch count into
 *    (completion tickets, histogram counters) carry that launch's epoch,
 *    so no result depends on what an earlier call, finished or not, left
 *    in the scratch.
 *  - Calls on different streams may run concurrently.  Thread-safe.
 *  - No C++ exception crosses this interface.  The library prints nothing
 *    unless LIBTOPK_DEBUG is set in the environment (then HIP failures are
 *    described on stderr).
 */
#ifndef LIBTOPK_H
#define LIBTOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layout-compatible with HIP's hipStream_t (a pointer to struct
 * ihipStream_t); callers may pass a hipStream_t directly. */
struct ihipStream_t;
typedef struct ihipStream_t *libtopk_stream_t;

/* Status codes returned by every entry point. */
enum {
    LIBTOPK_OK = 0,
    LIBTOPK_ERR_INVALID = 1,     /* bad pointer, size, k or op            */
    LIBTOPK_ERR_UNSUPPORTED = 2, /* k above the call's supported maximum  */
    LIBTOPK_ERR_NOMEM = 3,       /* scratch allocation failed             */
    LIBTOPK_ERR_HIP = 4          /* no device, or a HIP call / launch failed */
};

/* Reduction operators for reduce_i32. */
enum { LIBTOPK_SUM = 0, LIBTOPK_MAX = 1, LIBTOPK_MIN = 2 };

/* Largest k of every top-k entry point (the register-list path). */
#define LIBTOPK_MAX_K 128

/* Largest k of topk_i32, which takes k above LIBTOPK_MAX_K through radix
 * selection. */
#define LIBTOPK_MAX_K_SELECT 16384

/* Most bins of histogram_i32. */
#define LIBTOPK_MAX_BINS 4096

/*
 * topk_i32 — the k largest values of in[0..n), written to out[0..k) in
 * descending order, duplicates kept with their multiplicity.
 *
 * Operation: [TopK] §1 (find the 20 largest of 1e8 values) and §2 (the
 * two-stage design: §2.1 each thread keeps a descending local top-k list
 * over a grid-stride share of the input, and the block merges the lists;
 * §2.2 a second, single-block stage merges the per-block candidates; the
 * result must be identical to the CPU's).  For k <= LIBTOPK_MAX_K both
 * stages run in one launch: the last workgroup to finish stage 1 performs
 * stage 2.  Larger k, up to LIBTOPK_MAX_K_SELECT, goes through radix
 * selection ("GPU基数排序优化：10亿级数据处理与性能调优" §3.2–3.3: 8-bit digit
 * histograms kept per warp in shared memory): four digit passes find the
 * k-th largest value, a gather pass collects the values above it, and one
 * workgroup sorts the k results.  Once a digit leaves fewer than 2^22
 * candidates they are copied aside and the remaining passes read only
 * them.  From n = 2^18 on (when n is large enough for k), a sample first
 * fixes a threshold and a filter pass copies the values above it aside;
 * when that copy is small (the usual case) one workgroup selects the
 * top-k from it, the digit passes return at once, and the input is read
 * once.  Six stream-ordered launches, eight on sampled inputs.
 *
 *   in   device, int32[n], read once (k <= LIBTOPK_MAX_K)
 *   n    number of elements, 1 <= n <= 2^32
 *   k    1 <= k <= min(n, LIBTOPK_MAX_K_SELECT)
 *   out  device, int32[k], written in full
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer, n out of
 * range, k < 1 or k > n; LIBTOPK_ERR_UNSUPPORTED for
 * k > LIBTOPK_MAX_K_SELECT.
 */
int topk_i32(const int32_t *in, int64_t n, int32_t k, int32_t *out,
             libtopk_stream_t stream);

/* Bytes of the fixed device array behind topk_i32_noalloc (528 KiB). */
#define LIBTOPK_NOALLOC_SCRATCH_BYTES 540672

/*
 * topk_i32_noalloc — topk_i32 for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  Same operation, arguments, output and errors as
 * topk_i32 for k <= LIBTOPK_MAX_K (one launch), but the call never
 * allocates: no hipMalloc, hipFree or allocating library routine.  Its
 * scratch (stage-1 candidates, block maxima and completion tickets) is a
 * fixed array of LIBTOPK_NOALLOC_SCRATCH_BYTES in the library's device
 * memory, one per device, held until the process ends; it is sized for
 * every k <= LIBTOPK_MAX_K and every n <= 2^32.  The first call on a device
 * looks up the array's address and clears its tickets with a small kernel
 * on `stream` (no allocation).
 *
 * Every call on one device shares that device's array, which keeps the
 * last call's contents: calls that overlap on one device (different
 * streams, or different host threads) race and give wrong results; order
 * them on one stream or otherwise.
 *
 *   in, n, out, stream   as for topk_i32
 *   k    1 <= k <= min(n, LIBTOPK_MAX_K)
 *
 * Errors: as topk_i32; k > LIBTOPK_MAX_K returns LIBTOPK_ERR_UNSUPPORTED
 * (radix selection needs megabytes of candidate space, not in the array).
 */
int topk_i32_noalloc(const int32_t *in, int64_t n, int32_t k, int32_t *out,
                     libtopk_stream_t stream);

/*
 * reduce_i32 — fold in[0..n) with one operator into a single int64.
 *
 * Operation: [Reduce] "Basic concepts" (a reduction combines every element
 * through one binary operation into one result; the worked example sums
 * [1..8] to 36) and the "complete multi-level reduction" driver (a first
 * pass leaves one partial per block, a further pass combines them).  Here
 * exactly two stages run in one launch: per-block partials, then the last
 * workgroup to finish combines them.
 *
 *   in       device, int32[n] (may be NULL when n == 0)
 *   n        0 <= n <= 2^32
 *   op       LIBTOPK_SUM: exact int64 sum (cannot overflow for n <= 2^32);
 *            LIBTOPK_MAX / LIBTOPK_MIN: the extreme value, sign-extended.
 *            n == 0 yields the identity: 0, INT32_MIN or INT32_MAX.
 *   out_i64  device, int64[1]
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer, n out of
 * range or an unknown op.
 */
int reduce_i32(const int32_t *in, int64_t n, int32_t op, int64_t *out_i64,
               libtopk_stream_t stream);

/*
 * topk_kv_i32 / topk_kv_f32 — the k largest elements of in[0..n) with their
 * positions: out_values[i] and out_indices[i] for i < k, ordered by value,
 * descending, and among equal values by position, ascending (the earlier
 * element first), so the result is unique.
 *
 * Operation: [TopK] §6 (the reduction keeps a candidate list of items
 * ordered by their score) with [TopK] §2's two stages, and "GPU基数排序优化：
 * 10亿级数据处理与性能调优" §8 (key-value pairs carried together; float keys
 * through a bit transform).  Float order: the order-preserving map of the
 * bits to unsigned integers (negative: all bits flipped; otherwise the sign
 * bit set): numerical order on numbers, -0 below +0, positive NaNs above
 * +infinity, negative NaNs below -infinity.  One launch, as topk_i32.
 *
 *   in           device, int32[n] or float32[n], read once
 *   n            1 <= n < 2^32 (positions must fit 32 bits)
 *   k            1 <= k <= min(n, LIBTOPK_MAX_K)
 *   out_values   device, int32[k] / float32[k] (the input's own bits)
 *   out_indices  device, int64[k], positions in [0, n)
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer (out_indices
 * 8-byte aligned), n out of range, k < 1 or k > n, or overlapping buffers;
 * LIBTOPK_ERR_UNSUPPORTED for k > LIBTOPK_MAX_K.
 */
int topk_kv_i32(const int32_t *in, int64_t n, int32_t k, int32_t *out_values,
                int64_t *out_indices, libtopk_stream_t stream);
int topk_kv_f32(const float *in, int64_t n, int32_t k, float *out_values,
                int64_t *out_indices, libtopk_stream_t stream);

/*
 * reduce_stats_i32 — count, sum, max, min and sum of squares of in[0..n),
 * all from one read of the data.
 *
 * Operation: [TopK] §6 (the two-stage reduction also serves large-scale
 * statistics such as the mean and the variance) and [Reduce] "Basic
 * concepts" (each statistic is a fold through one binary operator).  Mean
 * and population variance follow from the result: sum / count and
 * (count * sumsq - sum^2) / count^2.  Two stages in one launch, as
 * reduce_i32.
 *
 *   in       device, int32[n] (may be NULL when n == 0)
 *   n        0 <= n <= 2^32
 *   out      device, int64[6], written in full:
 *              out[0]  count = n
 *              out[1]  exact sum (int64; cannot overflow for n <= 2^32)
 *              out[2]  max, sign-extended (INT32_MIN when n == 0)
 *              out[3]  min, sign-extended (INT32_MAX when n == 0)
 *              out[4]  sum of squares, low 64 bits  } one unsigned 128-bit
 *              out[5]  sum of squares, high 64 bits } integer, exact
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer (out must be
 * 8-byte aligned), n out of range, or overlapping in and out.
 */
int reduce_stats_i32(const int32_t *in, int64_t n, int64_t *out,
                     libtopk_stream_t stream);

/*
 * topk_batched_i32 — the top-k of every row of a row-major int32 matrix:
 * out[r * k + i], i < k, is the i-th largest value of row r, which is
 * in[r * ld .. r * ld + cols); each row's k values in descending order,
 * duplicates kept.
 *
 * Operation: [TopK] §6 (the two-stage pattern as a building block, e.g.
 * candidate selection per user in a recommender) with [TopK] §2's two
 * stages per row.  Long rows get several workgroups each and the last of a
 * row's workgroups merges its candidates; rows of up to 4096 elements are
 * handled one wave per row.
 *
 *   in    device, int32, rows of `cols` elements `ld` elements apart;
 *         elements between cols and ld of a row are never read
 *   rows  0 <= rows (0: nothing is enqueued and LIBTOPK_OK is returned
 *         once cols, ld and k are valid; in and out may then be NULL)
 *   cols  1 <= cols <= 2^32
 *   ld    row stride in elements, ld >= cols (any value: rows need not be
 *         16-byte aligned)
 *   k     1 <= k <= min(cols, LIBTOPK_MAX_K)
 *   out   device, int32[rows * k], written in full
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer, rows < 0,
 * cols or ld out of range, k < 1 or k > cols, an input span beyond 2^60
 * elements, or overlapping input and output; LIBTOPK_ERR_UNSUPPORTED for
 * k > LIBTOPK_MAX_K.
 */
int topk_batched_i32(const int32_t *in, int64_t rows, int64_t cols,
                     int64_t ld, int32_t k, int32_t *out,
                     libtopk_stream_t stream);

/*
 * topk_merge_i32 — merge several top-k results: the k largest values of the
 * union of m lists, written to out[0..k) in descending order.
 *
 * Operation: [TopK] §6 (several TopK results merged again) and §2.2 (the
 * second stage merges per-block top-k lists into the final one).  Only the
 * first min(len, k) entries of a list are read, plus what the merge needs
 * to bound the result.  Typical inputs: the outputs of topk_i32 on shards
 * of one array (the merge of the shards' top-k lists is the top-k of the
 * whole), or the rows written by topk_batched_i32.
 *
 *   lists  device, int32[m * len], list j at lists + j * len; every list
 *          MUST be in descending order (as the top-k calls write them).
 *          The library does not check this; on a list out of order the
 *          result is unspecified (nothing is read outside lists[]).
 *   m      1 <= m <= 2^20 lists
 *   len    entries per list, len >= 1
 *   k      1 <= k <= min(m * len, LIBTOPK_MAX_K)
 *   out    device, int32[k], written in full
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer, m or len
 * out of range, k < 1 or k > m * len, or overlapping lists and out;
 * LIBTOPK_ERR_UNSUPPORTED for k > LIBTOPK_MAX_K.
 */
int topk_merge_i32(const int32_t *lists, int64_t m, int32_t len, int32_t k,
                   int32_t *out, libtopk_stream_t stream);

/*
 * topk_segmented_i32 — the top-k of every segment of one array, segments
 * of any lengths given by offsets: segment s is
 * in[offsets[s] .. offsets[s + 1]), and out[s * k + i], i < min(k, len_s),
 * is its i-th largest value (descending, duplicates kept).  A segment
 * shorter than k (empty included) fills the rest of its k slots with
 * INT32_MIN; counts[s] = min(k, len_s) tells that padding from real
 * INT32_MIN values.
 *
 * Operation: [TopK] §6 (the two-stage pattern as a building block, e.g.
 * candidate selection per user, whose candidate lists differ in length;
 * several TopK results merged again) with [TopK] §2's two stages per
 * segment.  Two launches on `stream`: one wave per segment finishes
 * segments of up to 4096 elements in registers and plans the rest on the
 * device; persistent workgroups then stream the longer segments (a
 * segment above 2^16 elements in up to 1024 parts, whose candidates the
 * last part to finish merges).
 *
 *   in       device, int32[n] (may be NULL when n == 0)
 *   n        elements of in, 0 <= n <= 2^32
 *   offsets  device, int64[nseg + 1], 8-byte aligned; the caller promises
 *            0 <= offsets[0] <= offsets[1] <= ... <= offsets[nseg] <= n.
 *            The library does not check this (the offsets live on the
 *            device); with offsets that break it the results are
 *            unspecified, but nothing outside in[0..n), out and counts is
 *            read or written.
 *   nseg     0 <= nseg < 2^31 (0: nothing is enqueued, LIBTOPK_OK once k
 *            is valid; the pointers may then be NULL)
 *   k        1 <= k <= LIBTOPK_MAX_K
 *   out      device, int32[nseg * k], written in full
 *   counts   device, int32[nseg], or NULL when not wanted
 *
 * Scratch: besides the per-stream area, about 0.6 KiB per 1,000 elements
 * of n (lists and the parts' candidates), allocated on the first call with
 * a larger n on the stream (which then synchronises the stream once).
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer, n or nseg
 * out of range, k < 1, or overlapping buffers; LIBTOPK_ERR_UNSUPPORTED for
 * k > LIBTOPK_MAX_K.
 */
int topk_segmented_i32(const int32_t *in, int64_t n, const int64_t *offsets,
                       int64_t nseg, int32_t k, int32_t *out, int32_t *counts,
                       libtopk_stream_t stream);

/*
 * histogram_i32 — counts of the values of in[0..n) in nbins equal bins:
 * out[b] = the number of elements v with
 *     lo + b * 2^shift <= v <= lo + (b + 1) * 2^shift - 1
 * (bounds taken in exact integer arithmetic); values outside all bins are
 * not counted.
 *
 * Operation: [TopK] §6 (histogram computation as a use of the two-stage
 * reduction) and "GPU基数排序优化：10亿级数据处理与性能调优" §3.3 (one
 * shared-memory histogram per warp, merged at the end, rather than global
 * atomics per element).  One launch: per-wave histograms in LDS, per-block
 * totals added into device counters, and the last workgroup to finish
 * writes the result and clears the counters.
 *
 *   in     device, int32[n] (may be NULL when n == 0)
 *   n      0 <= n <= 2^32
 *   lo     the first bin's lowest value (any int32)
 *   shift  bin width 2^shift, 0 <= shift <= 31
 *   nbins  1 <= nbins <= LIBTOPK_MAX_BINS
 *   out    device, int64[nbins], 8-byte aligned, written in full
 *
 * Errors: LIBTOPK_ERR_INVALID for a NULL or misaligned pointer, n, shift
 * or nbins out of range, or overlapping in and out.
 */
int histogram_i32(const int32_t *in, int64_t n, int32_t lo, int32_t shift,
                  int32_t nbins, int64_t *out, libtopk_stream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char *libtopk_strerror(int status);

/* LIBTOPK_MAX_K. */
int libtopk_max_k(void);

/*
 * Number of stage-1 workgroups for later calls in this process: 0 restores
 * the automatic choice, otherwise 1..1024.  Results never depend on it (the
 * tests sweep it); it exists for tuning.  Returns LIBTOPK_ERR_INVALID for a
 * value outside 0..1024.
 */
int libtopk_set_grid(int32_t blocks);

/*
 * Workgroups that a topk_i32 call of size n (k <= LIBTOPK_MAX_K) would
 * launch under the current setting (reporting and traffic accounting; no
 * device work).  Returns 0 for n < 1.  With no grid set, the other calls
 * choose their own counts: reductions, statistics and selection for
 * k > LIBTOPK_MAX_K launch at most one workgroup per compute unit,
 * histograms at most two, all of them fewer on small inputs, and key-value
 * calls whose kernel fits only one workgroup per compute unit (k > 64) at
 * most one per unit.
 */
int32_t libtopk_grid_for(int64_t n);

/*
 * Test hook: overwrite, on `stream`, the completion tickets and histogram
 * counters that later calls will use with pseudo-random nonzero words
 * derived from `seed` -- which == 0: those of the scratch of calls on
 * `stream` (allocated first if need be), with the counters and tickets of
 * the segmented top-k once it has run there; which == 1: the tickets of the
 * fixed array of topk_i32_noalloc on the current device.  These words are
 * tagged with each launch's epoch, so no later result may depend on what
 * they held; tests use this to check that.  They index no memory, so any
 * value is safe.  Returns LIBTOPK_ERR_INVALID for another `which`.
 */
int libtopk_debug_scramble(libtopk_stream_t stream, int32_t which,
                           uint64_t seed);

/*
 * Free every cached scratch area after synchronising the devices that own
 * them.  The next call allocates afresh.  Must not race with other calls.
 */
void libtopk_release(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBTOPK_H */
