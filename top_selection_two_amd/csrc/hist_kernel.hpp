// Histograms over int32, and the streaming helpers the radix selection
// (select_kernel.hpp) shares with them.
//
// Sources:
//   [TopK]  "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计" §6
//           (histogram computation as a use of the two-stage reduction) and
//           §2 (per-block partial results, merged by a final stage).
//   [Radix] "GPU基数排序优化：10亿级数据处理与性能调优" §3.3 (one shared-memory
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
// last workgroup to finish (ticket) hands the counters on and arms them for
// the next launch; the counters are tagged with the launch's epoch, so no
// memset is ever enqueued and no stale count is ever added in.
#pragma once

#include "wave.hpp"

namespace ltk {

constexpr int kMaxBins = 4096;     // histogram_i32
constexpr int kWaveHistBins = 256; // per-wave copies up to this many bins
constexpr int kDigitBins = 256;

// histogram_i32: bins of width 2^shift from lo.
struct HistParams {
  const int* in;
  int64_t n, head, ntiles, covered;
  int grid;
  int lo, shift, nbins;
  int64_t* out;             // [nbins]
  uint64_t* acc;            // [kMaxBins] epoch-tagged device counters
  uint64_t* ticket;
  uint32_t epoch;           // this launch's (see Tagged)
};

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
    visit_rest<kBlock * U * 4>(in, n, head, covered,
                               [&](int x, int64_t, bool ok)
                                   __attribute__((always_inline)) {
                                     fe(x, ok);
                                   });
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

// Device counters carry the launch's epoch tag (see Tagged): a counter left
// at any value by an earlier launch, finished or not, counts as zero, and
// the last workgroup arms every counter it reads for the next epoch instead
// of clearing it.  A count is at most n <= 2^32, so 33 bits hold it.
typedef Tagged<33> BinCount;

// Add this workgroup's nonzero count for bin b.
__device__ __forceinline__ void acc_add(uint64_t* acc, int nbins, int b,
                                        unsigned c, uint32_t epoch) {
  if (!c) return;
  const int copies = acc_copies(nbins);
  const int copy = copies > 1 ? (int)(blockIdx.x % kAccCopies) : 0;
  BinCount::add(acc + copy * nbins + b, c, epoch);
}

// Read bin b summed over the copies and arm it for the next epoch (last
// workgroup only).  All copies are loaded before any is used, so the
// device-coherent loads overlap.
__device__ __forceinline__ uint64_t acc_take(uint64_t* acc, int nbins, int b,
                                             uint32_t epoch) {
  const uint64_t next = BinCount::armed(epoch + 1u);
  if (acc_copies(nbins) == 1) {
    const uint64_t t = BinCount::count(ld_agent(acc + b), epoch);
    st_agent(acc + b, next);
    return t;
  }
  uint64_t v[kAccCopies];
#pragma unroll
  for (int j = 0; j < kAccCopies; ++j) v[j] = ld_agent(acc + j * nbins + b);
  uint64_t t = 0;
#pragma unroll
  for (int j = 0; j < kAccCopies; ++j) {
    t += BinCount::count(v[j], epoch);
    st_agent(acc + j * nbins + b, next);
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

  // An element's bin, or nb and more when it has none (x >= lo makes
  // x - lo exact in 32 unsigned bits).
  auto bin_of = [&](int x) __attribute__((always_inline)) -> unsigned {
    return x >= lo ? ((unsigned)x - (unsigned)lo) >> shift : 0xffffffffu;
  };
  // Same-address LDS atomics serialise, so a wave whose 256 elements of
  // one vector slot all share a bin adds 256 with one atomic (a histogram
  // of 1e8 equal values, or of values that all fall into one bin, took
  // 333 us with an atomic per element, against 61 us for spread values).
  // The check costs spread values about 2 % (60.7 -> 62.0 us); checking
  // only every 16th slot until one passes cost more (63.5 us).
  for_each_vector<U>(
      p.in, p.n, p.head, p.ntiles, p.covered, p.grid, (int)blockIdx.x,
      [&](const v4i& v) __attribute__((always_inline)) {
        const unsigned b0 = bin_of(v.x), b1 = bin_of(v.y), b2 = bin_of(v.z),
                       b3 = bin_of(v.w);
        const unsigned bu = (unsigned)uni((int)b0);
        // Tiles keep every lane active.
        if (ballot((b0 == bu) & (b1 == bu) & (b2 == bu) & (b3 == bu)) == ~0ull) {
          if (lane() == 0 && bu < (unsigned)nb) atomicAdd(&hw[bu], 4u * kWave);
        } else {
          if (b0 < (unsigned)nb) atomicAdd(&hw[b0], 1u);
          if (b1 < (unsigned)nb) atomicAdd(&hw[b1], 1u);
          if (b2 < (unsigned)nb) atomicAdd(&hw[b2], 1u);
          if (b3 < (unsigned)nb) atomicAdd(&hw[b3], 1u);
        }
      },
      [&](int x, bool ok) __attribute__((always_inline)) {
        const unsigned d = bin_of(x);
        if (ok && d < (unsigned)nb) atomicAdd(&hw[d], 1u);
      });
  __syncthreads();

  // This workgroup's counts into the device counters.
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    unsigned c = h[b];
    if (per_wave) {
#pragma unroll
      for (int j = 1; j < kWaves; ++j) c += h[j * kWaveHistBins + b];
    }
    acc_add(p.acc, nb, b, c, p.epoch);
  }

  if (!last_to_finish(p.ticket, p.grid, p.epoch, &is_last)) return;
  for (int b = threadIdx.x; b < nb; b += kBlock)
    p.out[b] = (int64_t)acc_take(p.acc, nb, b, p.epoch);
}

}  // namespace ltk
