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
// for selection instead of sorting): pass p histograms digit p (bits
// 31 - 8p .. 24 - 8p of the order-preserving biased value) over the
// elements whose higher digits equal the prefix chosen so far; the last
// workgroup picks the digit holding the k-th largest and updates the
// prefix.  After four passes the prefix is g.  If a pass finds that every
// element of the chosen bucket is needed, selection stops early.  A gather
// pass then appends the elements above the bucket (and, when stopped
// early, the bucket itself) to the output; copies of g fill the rest, and
// one workgroup sorts the k values in LDS.
#pragma once

#include "wave.hpp"

namespace ltk {

constexpr int kMaxBins = 4096;     // histogram_i32
constexpr int kWaveHistBins = 256; // per-wave copies up to this many bins
constexpr int kDigitBins = 256;
constexpr int kMaxKSelect = 16384; // largest k of the radix-select path

// Selection state in device memory, written by the last workgroup of each
// pass and read by every workgroup of the next.
struct RadixState {
  unsigned prefix;  // biased high digits chosen so far
  unsigned mask;    // the bits they cover
  int kleft;        // top-k elements still to be found inside the bucket
  int done;         // every element of the bucket is in the top-k
  unsigned gcount;  // elements appended by the gather pass
};

struct HistParams {
  const int* in;
  int64_t n, head, ntiles, covered;
  int grid;
  // histogram_i32: bins of width 2^shift from lo
  int lo, shift, nbins;
  int64_t* out;  // [nbins]
  // radix selection: digit at bit `dshift`; the first pass starts from an
  // empty prefix and kleft = k instead of reading the state
  RadixState* st;
  int dshift, first, k;
  unsigned long long* acc;  // [kMaxBins] device counters, zero between calls
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

// Call f(x, true) for every element this workgroup owns: its round-robin
// tiles through two alternating register buffers (both always filled, so
// each tile's wait is for that tile alone), then, in the last workgroup,
// the unaligned head and the tail, kBlock at a time, where lanes past the
// end call f(INT_MIN, false) so that f may use wave-wide votes.
template <int U, class F>
__device__ __forceinline__ void for_each_element(const int* in, int64_t n,
                                                 int64_t head, int64_t ntiles,
                                                 int64_t covered, int grid,
                                                 F&& f) {
  const int blk = blockIdx.x;
  auto tile = [&](const v4i (&d)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f(d[u].x, true);
      f(d[u].y, true);
      f(d[u].z, true);
      f(d[u].w, true);
    }
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
      f(ok ? in[i < head ? i : covered + i] : kI32Min, ok);
    }
  }
}

// The bin of x, or -1 when x is not counted.
template <bool DIGIT>
struct Binner {
  int lo;
  unsigned shift, nbins;    // range bins
  unsigned prefix, mask;    // digit bins: elements in the bucket only
  __device__ __forceinline__ int operator()(int x) const {
    if (DIGIT) {
      const unsigned u = bias(x);
      return (u & mask) == prefix ? (int)((u >> shift) & (kDigitBins - 1))
                                  : -1;
    }
    // x >= lo makes x - lo exact in 32 unsigned bits.
    const unsigned d = ((unsigned)x - (unsigned)lo) >> shift;
    return (x >= lo && d < nbins) ? (int)d : -1;
  }
};

template <int U, bool DIGIT>
__global__ __launch_bounds__(kBlock) void hist_kernel(HistParams p) {
  __shared__ unsigned h[kMaxBins];
  __shared__ int scan[kWaves];
  __shared__ int is_last;
  const int w = threadIdx.x / kWave;

  Binner<DIGIT> bin;
  int kleft = p.k;
  if (DIGIT) {
    unsigned prefix = 0u, mask = 0u;
    if (!p.first) {
      const RadixState s = *p.st;
      if (s.done) return;  // selection already finished: nothing to count
      prefix = s.prefix;
      mask = s.mask;
      kleft = s.kleft;
    }
    bin.prefix = prefix;
    bin.mask = mask;
    bin.shift = (unsigned)p.dshift;
  } else {
    bin.lo = p.lo;
    bin.shift = (unsigned)p.shift;
    bin.nbins = (unsigned)p.nbins;
  }
  const int nb = DIGIT ? kDigitBins : p.nbins;
  // Per-wave copies when they fit (fewer same-address collisions), else one.
  // The copies sit kWaveHistBins apart: clear all of them.
  const bool per_wave = nb <= kWaveHistBins;
  const int used = per_wave ? kWaves * kWaveHistBins : nb;
  for (int i = threadIdx.x; i < used; i += kBlock) h[i] = 0u;
  __syncthreads();
  unsigned* hw = per_wave ? h + w * kWaveHistBins : h;

  for_each_element<U>(p.in, p.n, p.head, p.ntiles, p.covered, p.grid,
                      [&](int x, bool ok) __attribute__((always_inline)) {
                        const int b = bin(x);
                        if (ok && b >= 0) atomicAdd(&hw[b], 1u);
                      });
  __syncthreads();

  // This workgroup's counts into the device counters.
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    unsigned c = h[b];
    if (per_wave) {
#pragma unroll
      for (int j = 1; j < kWaves; ++j) c += h[j * kWaveHistBins + b];
    }
    if (c) atomicAdd(p.acc + b, (unsigned long long)c);
  }

  if (!last_to_finish(p.ticket, p.grid, &is_last)) return;

  if (!DIGIT) {
    for (int b = threadIdx.x; b < nb; b += kBlock) {
      p.out[b] = (int64_t)ld_agent(p.acc + b);
      st_agent(p.acc + b, 0ull);
    }
    if (threadIdx.x == 0) st_agent(p.ticket, 0u);
    return;
  }

  // Pick the digit holding the k-th largest: thread t looks at bin 255 - t,
  // so an inclusive prefix sum over threads is the count of the bucket's
  // elements at or above that bin.  Counts are capped at 2^20 (> any k),
  // which keeps the sums in 32 bits and leaves every comparison with kleft
  // unchanged: the first bin whose capped sum reaches kleft is reached by
  // exact counts.
  const int t = threadIdx.x;
  const int b = kDigitBins - 1 - t;
  const unsigned long long raw = ld_agent(p.acc + b);
  st_agent(p.acc + b, 0ull);
  const int c = raw > (1ull << 20) ? (1 << 20) : (int)raw;
  const int incl_w = wave_scan_incl(c);
  if (lane() == kWave - 1) scan[w] = incl_w;
  __syncthreads();
  int incl = incl_w;
  for (int j = 0; j < w; ++j) incl += scan[j];
  const int above = incl - c;
  if (incl >= kleft && above < kleft) {
    RadixState s;
    s.prefix = bin.prefix | ((unsigned)b << p.dshift);
    s.mask = bin.mask | ((unsigned)(kDigitBins - 1) << p.dshift);
    s.kleft = kleft - above;
    s.done = c == s.kleft;  // the whole bucket is needed
    s.gcount = 0u;
    *p.st = s;
  }
  if (t == 0) st_agent(p.ticket, 0u);
}

struct GatherParams {
  const int* in;
  int64_t n, head, ntiles, covered;
  int grid, k;
  RadixState* st;
  int* out;  // [k]
  unsigned* ticket;
};

// Append the elements of the top-k that lie above the final bucket (and,
// when selection stopped early, the bucket itself) to out; the last
// workgroup fills the remaining slots with copies of g.  Order is
// arbitrary here; the sort kernel follows.
template <int U>
__global__ __launch_bounds__(kBlock) void gather_kernel(GatherParams p) {
  __shared__ int is_last;
  const RadixState s = *p.st;
  for_each_element<U>(
      p.in, p.n, p.head, p.ntiles, p.covered, p.grid,
      [&](int x, bool ok) __attribute__((always_inline)) {
        const unsigned key = bias(x) & s.mask;
        const bool q = ok && (key > s.prefix || (s.done && key == s.prefix));
        const uint64_t b = ballot(q);
        if (b == 0) return;
        unsigned base = 0;
        if (lane() == 0) base = atomicAdd(&p.st->gcount, (unsigned)popc(b));
        base = uni(base);
        // Exactly k - kleft values pass (k when stopped early); the bound
        // only guards the output against a selection state gone wrong.
        const unsigned pos = base + (unsigned)lanes_below(b);
        if (q && pos < (unsigned)p.k) p.out[pos] = x;
      });
  if (!last_to_finish(p.ticket, p.grid, &is_last)) return;
  if (!s.done) {
    const int g = unbias(s.prefix);
    for (int j = p.k - s.kleft + (int)threadIdx.x; j < p.k; j += kBlock)
      p.out[j] = g;
  }
  if (threadIdx.x == 0) st_agent(p.ticket, 0u);
}

// Sort out[0..k) (k <= kMaxKSelect) descending in one workgroup: the values
// go to LDS padded with INT_MIN to a power of two, a bitonic network runs
// over them with a barrier per step, and they are written back.
constexpr int kSortThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void sort_desc_kernel(int* out,
                                                                 int k) {
  __shared__ int s[kMaxKSelect];
  int m = 1;
  while (m < k) m <<= 1;
  for (int i = threadIdx.x; i < m; i += kSortThreads)
    s[i] = i < k ? out[i] : kI32Min;
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < m / 2; i += kSortThreads) {
        // The i-th pair: lower index a (bit `stride` clear), partner a + stride.
        const int a = 2 * i - (i & (stride - 1));
        const int b2 = a + stride;
        const int x = s[a], y = s[b2];
        const bool desc = (a & size) == 0;
        if (desc ? x < y : x > y) {
          s[a] = y;
          s[b2] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < k; i += kSortThreads) out[i] = s[i];
}

}  // namespace ltk
