// Statistics of an int32 array in one pass: count, sum, max, min and the
// exact sum of squares (from which the mean and the variance follow), all
// from a single read of the data.
//
// Sources:
//   [TopK]   "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计", §6
//            (the same two-stage reduction serves large-scale statistics
//            such as the mean and the variance).
//   [Reduce] "CUDA归约优化完全指南：从入门到精通", "Basic concepts" (each
//            statistic is a fold through one binary operator), Level 2
//            (reduce while loading, several elements per thread), Level 4
//            (wave-level exchange for the last steps), and the "complete
//            multi-level reduction" driver (one partial per block, then a
//            pass over the partials).
//
// gfx950 design: the streaming of reduce_kernel (non-temporal 16-byte
// loads, tiles dealt round-robin, register double buffering), with four
// accumulators per lane instead of one.  Reading the array once for all
// four statistics costs what one reduction costs; four separate passes
// would read it four times.
//  * sum: int64 per lane (exact for n <= 2^32).
//  * max, min: int32 per lane.
//  * sum of squares: x^2 <= 2^62, so two squares fit an unsigned 64-bit
//    value; each pair is added with carry into a 128-bit lane accumulator.
//    n <= 2^32 squares sum to at most 2^94, so nothing can overflow.
// The last workgroup to finish folds the per-block partials (ticket
// counter; see last_to_finish), as in reduce_kernel.  No MFMA: nothing here
// is a dense contraction.
#pragma once

#include "wave.hpp"

namespace ltk {

struct StatsParams {
  const int* in;
  int64_t n;
  int64_t head;
  int64_t ntiles;
  int64_t covered;
  int grid;
  uint64_t* partials;  // [grid * 4]: sum, max:min, squares low, high
  uint64_t* ticket;    // completion counter (epoch-tagged, see Tagged)
  uint32_t epoch;      // this launch's
  int64_t* out;        // [6]: count, sum, max, min, squares low, high
};

// One lane's statistics.  The sum of squares is qhi * 2^64 + qlo.
struct StatsAcc {
  int64_t s;
  int mx, mn;
  uint64_t qlo;
  uint64_t qhi;
};

__device__ __forceinline__ StatsAcc stats_identity() {
  StatsAcc a;
  a.s = 0;
  a.mx = kI32Min;
  a.mn = kI32Max;
  a.qlo = 0;
  a.qhi = 0;
  return a;
}

// Add an unsigned 64-bit value to the 128-bit sum of squares.
__device__ __forceinline__ void add_sq(StatsAcc& a, uint64_t t) {
  uint64_t lo;
  const bool c = __builtin_add_overflow(a.qlo, t, &lo);
  a.qlo = lo;
  a.qhi += (uint64_t)c;
}

__device__ __forceinline__ uint64_t square(int x) {
  return (uint64_t)((int64_t)x * (int64_t)x);
}

__device__ __forceinline__ void stats_add1(StatsAcc& a, int x) {
  a.s += (int64_t)x;
  a.mx = max(a.mx, x);
  a.mn = min(a.mn, x);
  add_sq(a, square(x));
}

__device__ __forceinline__ void stats_add4(StatsAcc& a, v4i d) {
  a.s += ((int64_t)d.x + (int64_t)d.y) + ((int64_t)d.z + (int64_t)d.w);
  a.mx = max(max(a.mx, max(d.x, d.y)), max(d.z, d.w));
  a.mn = min(min(a.mn, min(d.x, d.y)), min(d.z, d.w));
  // Two squares (each <= 2^62) per 64-bit addend.
  add_sq(a, square(d.x) + square(d.y));
  add_sq(a, square(d.z) + square(d.w));
}

__device__ __forceinline__ void stats_combine(StatsAcc& a, const StatsAcc& b) {
  a.s += b.s;
  a.mx = max(a.mx, b.mx);
  a.mn = min(a.mn, b.mn);
  uint64_t lo;
  const bool c = __builtin_add_overflow(a.qlo, b.qlo, &lo);
  a.qlo = lo;
  a.qhi += b.qhi + (uint64_t)c;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const int lo = __shfl_xor((int)(uint32_t)v, o, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Butterfly over the wave; every lane ends with the wave's statistics.
__device__ __forceinline__ StatsAcc stats_wave(StatsAcc a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    StatsAcc b;
    b.s = (int64_t)shfl_xor_u64((uint64_t)a.s, o);
    b.mx = __shfl_xor(a.mx, o, kWave);
    b.mn = __shfl_xor(a.mn, o, kWave);
    b.qlo = shfl_xor_u64(a.qlo, o);
    b.qhi = shfl_xor_u64(a.qhi, o);
    stats_combine(a, b);
  }
  return a;
}

// A block's (or the grid's) statistics as four 64-bit words.
__device__ __forceinline__ void stats_pack(const StatsAcc& a, uint64_t w[4]) {
  w[0] = (uint64_t)a.s;
  w[1] = ((uint64_t)(uint32_t)a.mx << 32) | (uint32_t)a.mn;
  w[2] = a.qlo;
  w[3] = a.qhi;
}

__device__ __forceinline__ StatsAcc stats_unpack(const uint64_t w[4]) {
  StatsAcc a;
  a.s = (int64_t)w[0];
  a.mx = (int)(uint32_t)(w[1] >> 32);
  a.mn = (int)(uint32_t)w[1];
  a.qlo = w[2];
  a.qhi = w[3];
  return a;
}

template <int U>
__global__ __launch_bounds__(kBlock) void stats_kernel(StatsParams p) {
  __shared__ uint64_t red[kWaves][4];
  __shared__ int is_last;
  const int blk = blockIdx.x;
  const int w = threadIdx.x / kWave;

  StatsAcc acc = stats_identity();
  // Round-robin tiles, two alternating register buffers (see load_tile and
  // reduce_kernel: every path into the loop has the same loads pending).
  const v4i* __restrict__ body = reinterpret_cast<const v4i*>(p.in + p.head);
  const int64_t count = tiles_of(p.ntiles, blk, p.grid);
  if (count > 0) {
    v4i A[U], B[U];
    load_tile<U>(body, blk, p.grid, count, 0, A);
    sched_fence();
    load_tile<U>(body, blk, p.grid, count, 1, B);
    sched_fence();
    int64_t i = 0;
#pragma nounroll
    for (; i + 2 <= count; i += 2) {
      ready(A);
#pragma unroll
      for (int u = 0; u < U; ++u) stats_add4(acc, A[u]);
      pin(acc.s);
      pin(acc.qlo);
      sched_fence();
      load_tile<U>(body, blk, p.grid, count, i + 2, A);
      sched_fence();
      ready(B);
#pragma unroll
      for (int u = 0; u < U; ++u) stats_add4(acc, B[u]);
      pin(acc.s);
      pin(acc.qlo);
      sched_fence();
      load_tile<U>(body, blk, p.grid, count, i + 3, B);
      sched_fence();
    }
    if (i < count) {
#pragma unroll
      for (int u = 0; u < U; ++u) stats_add4(acc, A[u]);
    }
  }
  // The unaligned head and the tail after the last full tile.
  if (blk == p.grid - 1) {
    const int64_t left = p.n - p.covered;
    for (int64_t i = threadIdx.x; i < left; i += kBlock)
      stats_add1(acc, p.in[i < p.head ? i : p.covered + i]);
  }
  acc = stats_wave(acc);
  if (lane() == 0) stats_pack(acc, red[w]);
  __syncthreads();
  if (threadIdx.x == 0) {
    StatsAcc b = stats_unpack(red[0]);
#pragma unroll
    for (int j = 1; j < kWaves; ++j) stats_combine(b, stats_unpack(red[j]));
    uint64_t wds[4];
    stats_pack(b, wds);
#pragma unroll
    for (int j = 0; j < 4; ++j) st_agent(p.partials + 4 * (int64_t)blk + j, wds[j]);
  }

  if (!last_to_finish(p.ticket, p.grid, p.epoch, &is_last)) return;

  // Fold the per-block partials.
  StatsAcc g = stats_identity();
  for (int b = threadIdx.x; b < p.grid; b += kBlock) {
    uint64_t wds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wds[j] = ld_agent(p.partials + 4 * (int64_t)b + j);
    stats_combine(g, stats_unpack(wds));
  }
  g = stats_wave(g);
  __syncthreads();  // red[] is reused
  if (lane() == 0) stats_pack(g, red[w]);
  __syncthreads();
  if (threadIdx.x == 0) {
    StatsAcc r = stats_unpack(red[0]);
#pragma unroll
    for (int j = 1; j < kWaves; ++j) stats_combine(r, stats_unpack(red[j]));
    p.out[0] = p.n;
    p.out[1] = r.s;
    p.out[2] = (int64_t)r.mx;
    p.out[3] = (int64_t)r.mn;
    p.out[4] = (int64_t)r.qlo;
    p.out[5] = (int64_t)r.qhi;
  }
}

}  // namespace ltk
