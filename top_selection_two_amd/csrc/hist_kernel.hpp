// Histograms over int32, and top-k for large k by radix selection built on
// the same histograms.
//
// Sources:
//   [TopK]  "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计" §6
//           (histogram computation as a use of the two-stage reduction) and
//           §2 (per-block partial results, merged by a final stage).
//   [Radix] "GPU基数排序优化：10亿级数据处理与性能调优" §3.2 (8-bit digits,
//           four passes for 32-bit keys) and §3.3 (one shared-memory
//           histogram per warp, updated with atomics and merged at the end,
//           instead of global atomics per element).
//
// gfx950 design.  The input streams through the same round-robin tiles and
// register double buffer as the reductions (non-temporal 16-byte loads).
// Each element's bin is found with 32-bit arithmetic and counted with an
// LDS atomic into the wave's own copy of the histogram (up to 256 bins;
// larger histograms use one copy per workgroup).  At the end each
// workgroup adds its nonzero bins into 64-bit device counters (global
// atomics, one per bin and workgroup rather than one per element), and the
// last workgroup to finish (ticket) hands the counters on and clears them,
// so no memset is ever enqueued.
//
// Radix selection of the k-th largest value g ([Radix] §3.2's digits, used
// for selection instead of sorting): pass p counts digit p (bits
// 31 - 8p .. 24 - 8p of the order-preserving biased value) over the
// elements whose higher digits equal the prefix chosen so far (the
// bucket); the last workgroup picks the digit holding the k-th largest and
// updates the prefix.  After four passes the prefix is g.  Everything
// between passes is decided on the device, from a state the last
// workgroup writes:
//  * once a pass leaves a bucket of fewer than kCandCap elements, the next
//    pass over the input also splits it: values above the bucket go
//    straight to the output (they are all in the top-k), the bucket's
//    values to a candidate buffer, and the remaining passes read only
//    that buffer;
//  * if every element of the chosen bucket is needed, selection stops
//    early (later passes return at once).
// A gather pass then appends what is still missing (values above the final
// bucket, or the whole bucket when selection stopped early) from the input
// or the candidate buffer, copies of g fill the rest, and one workgroup
// sorts the k values in LDS.
#pragma once

#include "wave.hpp"

namespace ltk {

constexpr int kMaxBins = 4096;     // histogram_i32
constexpr int kWaveHistBins = 256; // per-wave copies up to this many bins
constexpr int kDigitBins = 256;
constexpr int kMaxKSelect = 16384; // largest k of the radix-select path

constexpr int kCandCap = 1 << 22;  // candidate buffer, elements

// Selection state in device memory, written by the last workgroup of each
// pass and read by every workgroup of the next.
struct RadixState {
  unsigned prefix;  // biased high digits chosen so far
  unsigned mask;    // the bits they cover
  int kleft;        // top-k elements still to be found inside the bucket
  int done;         // every element of the bucket is in the top-k
  int bucket;       // elements in the bucket (exact when < kCandCap)
  int src;          // 0: passes read the input; 1: the candidate buffer
  int split;        // the next pass over the input splits the bucket off
  unsigned gcount;  // values appended to the output so far
  unsigned ccount;  // values appended to the candidate buffer
  int guess;        // top digit the first pass copies from (sample kernel)
};

// histogram_i32: bins of width 2^shift from lo.
struct HistParams {
  const int* in;
  int64_t n, head, ntiles, covered;
  int grid;
  int lo, shift, nbins;
  int64_t* out;             // [nbins]
  unsigned long long* acc;  // [kMaxBins] device counters, zero between calls
  unsigned* ticket;
};

// One digit pass of radix selection, or the gather.
struct SelectParams {
  const int* in;
  int64_t n, head, ntiles, covered;
  int grid;
  int dshift;   // the digit's lowest bit
  int first;    // the first pass: start from an empty prefix, kleft = k
  int use_guess;  // the first pass also copies values whose top digit is
                  // >= the sampled guess to the candidate buffer
  int k;
  RadixState* st;
  int* cand;    // [kCandCap] candidate buffer
  int* out;     // [k]
  unsigned long long* acc;  // [256] device counters, zero between calls
  unsigned* ticket;
};

// Inclusive prefix sum over the wave (row shifts within 16-lane rows, then
// the two row broadcasts); lanes without a source add 0.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Visit every element this workgroup owns: its round-robin tiles through
// two alternating register buffers (both always filled, so each tile's
// wait is for that tile alone), as fv(v4i) per 16-byte vector; then, in
// the last workgroup, the unaligned head and the tail, kBlock at a time,
// as fe(x, ok), where lanes past the end pass (INT_MIN, false) so that fe
// may use wave-wide votes.
template <int U, class FV, class FE>
__device__ __forceinline__ void for_each_vector(const int* in, int64_t n,
                                                int64_t head, int64_t ntiles,
                                                int64_t covered, int grid,
                                                int blk, FV&& fv, FE&& fe) {
  auto tile = [&](const v4i (&d)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) fv(d[u]);
  };
  const v4i* __restrict__ body = reinterpret_cast<const v4i*>(in + head);
  const int64_t cnt = tiles_of(ntiles, blk, grid);
  if (cnt > 0) {
    v4i A[U], B[U];
    load_tile<U>(body, blk, grid, cnt, 0, A);
    sched_fence();
    load_tile<U>(body, blk, grid, cnt, 1, B);
    sched_fence();
    int64_t i = 0;
#pragma nounroll
    for (; i + 2 <= cnt; i += 2) {
      ready(A);
      tile(A);
      sched_fence();
      load_tile<U>(body, blk, grid, cnt, i + 2, A);
      sched_fence();
      ready(B);
      tile(B);
      sched_fence();
      load_tile<U>(body, blk, grid, cnt, i + 3, B);
      sched_fence();
    }
    if (i < cnt) tile(A);
  }
  if (blk == grid - 1) {
    const int64_t left = n - covered;
    for (int64_t base = 0; base < left; base += kBlock) {
      const int64_t i = base + threadIdx.x;
      const bool ok = i < left;
      fe(ok ? in[i < head ? i : covered + i] : kI32Min, ok);
    }
  }
}

// The same with f(x, true) for every element of the tiles too.
template <int U, class F>
__device__ __forceinline__ void for_each_element(const int* in, int64_t n,
                                                 int64_t head, int64_t ntiles,
                                                 int64_t covered, int grid,
                                                 F&& f) {
  for_each_vector<U>(
      in, n, head, ntiles, covered, grid, (int)blockIdx.x,
      [&](const v4i& d) __attribute__((always_inline)) {
        f(d.x, true);
        f(d.y, true);
        f(d.z, true);
        f(d.w, true);
      },
      f);
}

// Device counters are kept in kAccCopies interleaved copies when the
// histogram is small enough: workgroup b adds into copy b % kAccCopies, so
// each counter address sees an eighth of the workgroups' atomics (they
// serialise at the L2), and the last workgroup sums the copies.
constexpr int kAccCopies = 8;

__device__ __forceinline__ int acc_copies(int nbins) {
  return nbins * kAccCopies <= kMaxBins ? kAccCopies : 1;
}

// Add this workgroup's nonzero count for bin b.
__device__ __forceinline__ void acc_add(unsigned long long* acc, int nbins,
                                        int b, unsigned c) {
  if (!c) return;
  const int copies = acc_copies(nbins);
  const int copy = copies > 1 ? (int)(blockIdx.x % kAccCopies) : 0;
  atomicAdd(acc + copy * nbins + b, (unsigned long long)c);
}

// Read bin b summed over the copies and clear it (last workgroup only).
// All copies are loaded before any is used, so the device-coherent loads
// overlap.
__device__ __forceinline__ unsigned long long acc_take(unsigned long long* acc,
                                                       int nbins, int b) {
  if (acc_copies(nbins) == 1) {
    const unsigned long long t = ld_agent(acc + b);
    st_agent(acc + b, 0ull);
    return t;
  }
  unsigned long long v[kAccCopies];
#pragma unroll
  for (int j = 0; j < kAccCopies; ++j) v[j] = ld_agent(acc + j * nbins + b);
  unsigned long long t = 0;
#pragma unroll
  for (int j = 0; j < kAccCopies; ++j) {
    t += v[j];
    st_agent(acc + j * nbins + b, 0ull);
  }
  return t;
}

template <int U>
__global__ __launch_bounds__(kBlock) void hist_kernel(HistParams p) {
  __shared__ unsigned h[kMaxBins];
  __shared__ int is_last;
  const int w = threadIdx.x / kWave;
  const int lo = p.lo, nb = p.nbins;
  const unsigned shift = (unsigned)p.shift;
  // Per-wave copies kWaveHistBins apart when they fit (fewer same-address
  // collisions), else one copy for the workgroup; clear what is used.
  const bool per_wave = nb <= kWaveHistBins;
  const int used = per_wave ? kWaves * kWaveHistBins : nb;
  for (int i = threadIdx.x; i < used; i += kBlock) h[i] = 0u;
  __syncthreads();
  unsigned* hw = per_wave ? h + w * kWaveHistBins : h;

  for_each_element<U>(p.in, p.n, p.head, p.ntiles, p.covered, p.grid,
                      [&](int x, bool ok) __attribute__((always_inline)) {
                        // x >= lo makes x - lo exact in 32 unsigned bits.
                        const unsigned d = ((unsigned)x - (unsigned)lo) >> shift;
                        if (ok && x >= lo && d < (unsigned)nb)
                          atomicAdd(&hw[d], 1u);
                      });
  __syncthreads();

  // This workgroup's counts into the device counters.
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    unsigned c = h[b];
    if (per_wave) {
#pragma unroll
      for (int j = 1; j < kWaves; ++j) c += h[j * kWaveHistBins + b];
    }
    acc_add(p.acc, nb, b, c);
  }

  if (!last_to_finish(p.ticket, p.grid, &is_last)) return;
  for (int b = threadIdx.x; b < nb; b += kBlock)
    p.out[b] = (int64_t)acc_take(p.acc, nb, b);
  if (threadIdx.x == 0) st_agent(p.ticket, 0u);
}

// Append the lanes where q holds to dst at a device counter (one atomic per
// wave); positions at or past cap are dropped (they never occur while the
// selection state is sound: the bound only guards the buffers).
__device__ __forceinline__ void append(bool q, int x, unsigned* counter,
                                       int* dst, unsigned cap) {
  const uint64_t b = ballot(q);
  if (b == 0) return;
  unsigned base = 0;
  if (lane() == 0) base = atomicAdd(counter, (unsigned)popc(b));
  base = uni(base);
  const unsigned pos = base + (unsigned)lanes_below(b);
  if (q && pos < cap) dst[pos] = x;
}

// Workgroups that take part in a pass: all of them over the input; over
// the candidate buffer (16-byte aligned, no head peel) only as many as it
// has tiles (at least one).  The others return before the ticket.
template <int U>
__device__ __forceinline__ int pass_grid(const SelectParams& p,
                                         const RadixState& s) {
  if (s.src == 0) return p.grid;
  const int64_t ntiles = (int64_t)s.bucket / ((int64_t)kBlock * U * 4);
  return (int)min((int64_t)p.grid, max(ntiles, (int64_t)1));
}

// The elements a selection pass reads: the input, or the candidate buffer
// (`bucket` elements), spread over pass_grid workgroups.
template <int U, class F>
__device__ __forceinline__ void for_each_source(const SelectParams& p,
                                                const RadixState& s, int grid,
                                                F&& f) {
  if (s.src == 0) {
    for_each_element<U>(p.in, p.n, p.head, p.ntiles, p.covered, grid, f);
  } else {
    const int64_t n = s.bucket;
    const int64_t ntiles = n / ((int64_t)kBlock * U * 4);
    for_each_element<U>(p.cand, n, 0, ntiles, ntiles * kBlock * U * 4, grid,
                        f);
  }
}

// A wave's LDS staging area for the values a split copies to the
// candidate buffer: the wave appends with ballots (no atomics) and copies a
// whole batch out with one device atomic when the area is nearly full and
// at the end, so the shared counter sees about one atomic per wave instead
// of one per wave and element slot.
constexpr int kStage = 512;

struct Stager {
  int* buf;        // this wave's kStage LDS slots
  int cnt;         // wave-uniform fill level
  unsigned* counter;
  int* dst;
  unsigned cap;    // dst slots; positions past it are dropped (a guard)
  __device__ __forceinline__ void flush() {
    if (cnt == 0) return;
    unsigned base = 0;
    if (lane() == 0) base = atomicAdd(counter, (unsigned)cnt);
    base = uni(base);
    __builtin_amdgcn_wave_barrier();
    for (int i = lane(); i < cnt; i += kWave) {
      const unsigned pos = base + (unsigned)i;
      if (pos < cap) dst[pos] = buf[i];
    }
    __builtin_amdgcn_wave_barrier();
    cnt = 0;
  }
  __device__ __forceinline__ void put(bool q, int x) {
    const uint64_t b = ballot(q);
    if (b == 0) return;
    if (q) buf[cnt + lanes_below(b)] = x;
    cnt += popc(b);
    if (cnt > kStage - kWave) flush();
  }
};

template <int U>
__global__ __launch_bounds__(kBlock) void select_pass_kernel(SelectParams p) {
  __shared__ unsigned h[kWaves * kDigitBins];
  __shared__ int stage[kWaves][kStage];
  __shared__ int scan[kWaves];
  __shared__ int is_last;
  const int w = threadIdx.x / kWave;

  RadixState s;
  if (p.first) {
    s.prefix = 0u;
    s.mask = 0u;
    s.kleft = p.k;
    s.done = 0;
    s.bucket = 0;
    s.src = 0;
    s.split = 0;
    s.gcount = 0u;
    s.ccount = 0u;
  } else {
    s = *p.st;
    if (s.done) return;  // selection already finished: nothing to count
  }
  const bool split = s.split && s.src == 0;
  const int grid = pass_grid<U>(p, s);
  if ((int)blockIdx.x >= grid) return;
  // First pass with a sampled guess: copy every value whose top digit is
  // at or above it (a superset of the top-k when the guess is at most the
  // digit the pass selects, which the last workgroup checks).
  const bool pre = p.first && p.use_guess;
  const unsigned guess = pre ? (unsigned)p.st->guess : 256u;
  for (int i = threadIdx.x; i < kWaves * kDigitBins; i += kBlock) h[i] = 0u;
  __syncthreads();
  unsigned* hw = h + w * kDigitBins;
  const unsigned prefix = s.prefix, mask = s.mask;
  const unsigned dshift = (unsigned)p.dshift;

  Stager stg{stage[w], 0, &p.st->ccount, p.cand, (unsigned)kCandCap};
  if (pre) {
    // Every element counts in the first pass; copies are rare, so one vote
    // per 16-byte vector decides whether its four values need a look.
    auto one = [&](int x, bool ok) __attribute__((always_inline)) {
      const unsigned u = bias(x);
      if (ok) atomicAdd(&hw[u >> 24], 1u);
      stg.put(ok && (u >> 24) >= guess, x);
    };
    for_each_vector<U>(
        p.in, p.n, p.head, p.ntiles, p.covered, grid, (int)blockIdx.x,
        [&](const v4i& d) __attribute__((always_inline)) {
          atomicAdd(&hw[bias(d.x) >> 24], 1u);
          atomicAdd(&hw[bias(d.y) >> 24], 1u);
          atomicAdd(&hw[bias(d.z) >> 24], 1u);
          atomicAdd(&hw[bias(d.w) >> 24], 1u);
          const int m = max(max(d.x, d.y), max(d.z, d.w));
          if (ballot((bias(m) >> 24) >= guess) == 0) return;
          stg.put((bias(d.x) >> 24) >= guess, d.x);
          stg.put((bias(d.y) >> 24) >= guess, d.y);
          stg.put((bias(d.z) >> 24) >= guess, d.z);
          stg.put((bias(d.w) >> 24) >= guess, d.w);
        },
        one);
  }
  if (!pre) {
    for_each_source<U>(p, s, grid, [&](int x, bool ok)
                                       __attribute__((always_inline)) {
      const unsigned u = bias(x);
      const unsigned key = u & mask;
      // One vote guards the rest: most elements lie below the bucket.
      const bool ge = ok && key >= prefix;
      if (ballot(ge) == 0) return;
      const bool in_bucket = ge && key == prefix;
      if (in_bucket) atomicAdd(&hw[(u >> dshift) & (kDigitBins - 1)], 1u);
      if (split) {
        // Values above the bucket are few (fewer than k): direct appends.
        append(ge && key > prefix, x, &p.st->gcount, p.out, (unsigned)p.k);
        stg.put(in_bucket, x);
      }
    });
  }
  if (split || pre) stg.flush();
  __syncthreads();
  for (int b = threadIdx.x; b < kDigitBins; b += kBlock) {
    unsigned c = h[b];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) c += h[j * kDigitBins + b];
    acc_add(p.acc, kDigitBins, b, c);
  }

  if (!last_to_finish(p.ticket, grid, &is_last)) return;

  // Pick the digit holding the k-th largest: thread t looks at bin 255 - t,
  // so an inclusive prefix sum over threads is the count of the bucket's
  // elements at or above that bin.  Counts are capped at kCandCap, which
  // keeps the sums in 32 bits and leaves every comparison with kleft
  // (<= 16384) unchanged: the first bin whose capped sum reaches kleft is
  // reached by exact counts.
  const int t = threadIdx.x;
  const int b = kDigitBins - 1 - t;
  const unsigned long long raw = acc_take(p.acc, kDigitBins, b);
  const int c = raw > (unsigned long long)kCandCap ? kCandCap : (int)raw;
  const int incl_w = wave_scan_incl(c);
  if (lane() == kWave - 1) scan[w] = incl_w;
  __syncthreads();
  int incl = incl_w;
  for (int j = 0; j < w; ++j) incl += scan[j];
  const int above = incl - c;
  if (incl >= s.kleft && above < s.kleft) {
    RadixState n = s;
    n.prefix = prefix | ((unsigned)b << dshift);
    n.mask = mask | ((unsigned)(kDigitBins - 1) << dshift);
    n.kleft = s.kleft - above;
    n.done = c == n.kleft;  // the whole bucket is needed
    if (split) n.src = 1;   // later passes read the candidate buffer
    // The candidate buffer holds the bucket chosen before this pass; it
    // keeps that size (its elements are filtered by prefix from now on).
    n.bucket = split || s.src == 1 ? s.bucket : c;
    if (pre) {
      // The copy holds every value of top digit >= guess; it covers the
      // top-k if the chosen digit is >= guess, and is whole if it fit.
      const unsigned copied = ld_agent(&p.st->ccount);
      if ((unsigned)b >= guess && copied <= (unsigned)kCandCap) {
        n.src = 1;
        n.bucket = (int)copied;
      }
    }
    n.split = !n.done && n.src == 0 && c < kCandCap;
    // gcount and ccount are left as the pass's appends made them (both
    // start at 0 with the first pass; only one pass ever splits).
    p.st->prefix = n.prefix;
    p.st->mask = n.mask;
    p.st->kleft = n.kleft;
    p.st->done = n.done;
    p.st->bucket = n.bucket;
    p.st->src = n.src;
    p.st->split = n.split;
    if (p.first) {
      p.st->gcount = 0u;
      p.st->ccount = 0u;
    }
  }
  if (t == 0) st_agent(p.ticket, 0u);
}

// The sampled guess of the first digit for top-k with large n: S values
// spread evenly over the input (U 16-byte vectors per thread, `stride`
// vectors apart) are counted by top digit, and the last workgroup picks the
// largest digit d such that at least `need` sampled values have a top digit
// >= d (need covers k scaled to the sample with a wide margin).  The guess
// only decides what the first pass copies aside; a wrong guess costs time,
// never correctness.
struct SampleParams {
  const v4i* body;   // the 16-byte-aligned body of the input
  int64_t nvec;      // vectors in it
  int64_t stride;    // vectors between consecutive samples
  int need;
  RadixState* st;
  unsigned long long* acc;  // [256] device counters, zero between calls
  unsigned* ticket;
  int grid;
};

template <int U>
__global__ __launch_bounds__(kBlock) void sample_kernel(SampleParams p) {
  __shared__ unsigned h[kWaves * kDigitBins];
  __shared__ int scan[kWaves];
  __shared__ int is_last;
  const int w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kWaves * kDigitBins; i += kBlock) h[i] = 0u;
  __syncthreads();
  unsigned* hw = h + w * kDigitBins;
  const int64_t first =
      ((int64_t)blockIdx.x * kBlock + threadIdx.x) * U;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (first + u) * p.stride;
    if (v < p.nvec) {
      const v4i d = __builtin_nontemporal_load(p.body + v);
      atomicAdd(&hw[bias(d.x) >> 24], 1u);
      atomicAdd(&hw[bias(d.y) >> 24], 1u);
      atomicAdd(&hw[bias(d.z) >> 24], 1u);
      atomicAdd(&hw[bias(d.w) >> 24], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kDigitBins; b += kBlock) {
    unsigned c = h[b];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) c += h[j * kDigitBins + b];
    acc_add(p.acc, kDigitBins, b, c);
  }
  if (!last_to_finish(p.ticket, p.grid, &is_last)) return;
  // Suffix counts over digits, as in the selection passes.
  const int t = threadIdx.x;
  const int b = kDigitBins - 1 - t;
  const unsigned long long raw = acc_take(p.acc, kDigitBins, b);
  const int c = raw > (unsigned long long)kCandCap ? kCandCap : (int)raw;
  const int incl_w = wave_scan_incl(c);
  if (lane() == kWave - 1) scan[w] = incl_w;
  __syncthreads();
  int incl = incl_w;
  for (int j = 0; j < w; ++j) incl += scan[j];
  // The largest digit whose suffix reaches `need`; digit 0 if none does.
  if ((incl >= p.need && incl - c < p.need) || (b == 0 && incl < p.need))
    p.st->guess = b;
  if (t == 0) {
    p.st->ccount = 0u;
    st_agent(p.ticket, 0u);
  }
}

// Append what the top-k still misses -- the values above the final bucket
// (and, when selection stopped early, the bucket itself) -- from the input
// or the candidate buffer; the last workgroup fills the remaining slots
// with copies of g.  Order is arbitrary here; the sort kernel follows.
template <int U>
__global__ __launch_bounds__(kBlock) void gather_kernel(SelectParams p) {
  __shared__ int stage[kWaves][kStage];
  __shared__ int is_last;
  const RadixState s = *p.st;
  const int w = threadIdx.x / kWave;
  // Staged like the split's copies: one device atomic per wave and batch.
  const int grid = pass_grid<U>(p, s);
  if ((int)blockIdx.x >= grid) return;
  Stager stg{stage[w], 0, &p.st->gcount, p.out, (unsigned)p.k};
  for_each_source<U>(p, s, grid, [&](int x, bool ok)
                                     __attribute__((always_inline)) {
    const unsigned key = bias(x) & s.mask;
    stg.put(ok && (key > s.prefix || (s.done && key == s.prefix)), x);
  });
  stg.flush();
  if (!last_to_finish(p.ticket, grid, &is_last)) return;
  if (!s.done) {
    const int g = unbias(s.prefix);
    for (int j = p.k - s.kleft + (int)threadIdx.x; j < p.k; j += kBlock)
      p.out[j] = g;
  }
  if (threadIdx.x == 0) st_agent(p.ticket, 0u);
}

// Sort out[0..k) (k <= kMaxKSelect) descending in one workgroup of 1024
// threads: a bitonic network over m = k rounded up to a power of two (at
// least 1024; padding INT_MIN).  Thread t holds elements t + 1024 j,
// j < V = m / 1024, in registers, so a compare-exchange step of distance
// d costs: d < 64, a lane exchange inside the wave; d >= 1024, a swap
// between two of the thread's registers; 64 <= d < 1024, a round trip
// through LDS with two barriers (only these need the workgroup).
constexpr int kSortThreads = 1024;

template <int V>
__device__ __forceinline__ void sort_desc_block(int* out, int k, int* lds) {
  constexpr int m = V * kSortThreads;
  const int t = threadIdx.x;
  int v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j * kSortThreads + t;
    v[j] = i < k ? out[i] : kI32Min;
  }
  // Keep the max at position i of a pair when i is the lower index of a
  // pair in a run sorted descending, or the upper in an ascending one.
  auto keep_max = [](int i, int d, int size) __attribute__((always_inline)) {
    return ((i & d) == 0) == ((i & size) == 0);
  };
  for (int size = 2; size <= m; size <<= 1) {
    for (int d = size >> 1; d > 0; d >>= 1) {
      if (d >= kSortThreads) {
#pragma unroll
        for (int js = 1; js < V; js <<= 1) {
          if (d == js * kSortThreads) {
#pragma unroll
            for (int j = 0; j < V; ++j) {
              if ((j & js) == 0) {
                const int i = j * kSortThreads + t;
                const int a = v[j], b = v[j | js];
                const bool desc = (i & size) == 0;
                v[j] = desc ? max(a, b) : min(a, b);
                v[j | js] = desc ? min(a, b) : max(a, b);
              }
            }
          }
        }
      } else if (d >= kWave) {
#pragma unroll
        for (int j = 0; j < V; ++j) lds[j * kSortThreads + t] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int i = j * kSortThreads + t;
          const int o = lds[i ^ d];
          v[j] = keep_max(i, d, size) ? max(v[j], o) : min(v[j], o);
        }
        __syncthreads();
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int i = j * kSortThreads + t;
          const int o = __shfl_xor(v[j], d, kWave);
          v[j] = keep_max(i, d, size) ? max(v[j], o) : min(v[j], o);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j * kSortThreads + t;
    if (i < k) out[i] = v[j];
  }
}

__global__ __launch_bounds__(kSortThreads) void sort_desc_kernel(int* out,
                                                                 int k) {
  __shared__ int lds[kMaxKSelect];
  if (k <= kSortThreads) sort_desc_block<1>(out, k, lds);
  else if (k <= 2 * kSortThreads) sort_desc_block<2>(out, k, lds);
  else if (k <= 4 * kSortThreads) sort_desc_block<4>(out, k, lds);
  else if (k <= 8 * kSortThreads) sort_desc_block<8>(out, k, lds);
  else sort_desc_block<16>(out, k, lds);
}

}  // namespace ltk
