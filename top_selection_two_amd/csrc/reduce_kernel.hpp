// Plain int32 reductions (sum into int64, max, min): the two-stage
// reduction with both stages in one launch.
//
// Sources:
//   [Reduce] "CUDA归约优化完全指南：从入门到精通": "Basic concepts" (fold
//            every element through one binary operator), Level 2 (reduce
//            while loading, several elements per thread), Level 4 (wave-level
//            exchange for the last steps), the non-power-of-two advice (pad
//            with the identity) and the "complete multi-level reduction"
//            driver (one partial per block, then a pass over the partials).
//
// gfx950 design: non-temporal 16-byte loads, U per lane per tile, tiles
// dealt round-robin to the workgroups and double-buffered in registers;
// lanes accumulate in registers (int64 for the sum,
// so it cannot overflow for n <= 2^32), the wave combines with cross-lane
// shuffles, four wave partials meet in LDS, and the last workgroup to
// finish (ticket counter; see last_to_finish) folds the per-block partials
// instead of a second launch.  No MFMA: nothing here is a dense
// contraction.
#pragma once

#include "wave.hpp"

namespace ltk {

enum { kOpSum = 0, kOpMax = 1, kOpMin = 2 };

struct ReduceParams {
  const int* in;
  int64_t n;
  int64_t head;
  int64_t ntiles;
  int64_t covered;
  int grid;
  int64_t* partials;  // [grid]
  uint64_t* ticket;   // completion counter (epoch-tagged, see Tagged)
  uint32_t epoch;     // this launch's
  int64_t* out;       // [1]
};

template <int OP>
struct Fold;

template <>
struct Fold<kOpSum> {
  typedef int64_t acc_t;
  __device__ static acc_t identity() { return 0; }
  __device__ static acc_t add(acc_t a, int x) { return a + (int64_t)x; }
  __device__ static acc_t add4(acc_t a, v4i d) {
    return a + ((int64_t)d.x + (int64_t)d.y) + ((int64_t)d.z + (int64_t)d.w);
  }
  __device__ static int64_t combine(int64_t a, int64_t b) { return a + b; }
  __device__ static int64_t wave(acc_t a) { return wave_sum(a); }
  __device__ static int64_t widen(acc_t a) { return a; }
};

template <>
struct Fold<kOpMax> {
  typedef int acc_t;
  __device__ static acc_t identity() { return kI32Min; }
  __device__ static acc_t add(acc_t a, int x) { return max(a, x); }
  __device__ static acc_t add4(acc_t a, v4i d) {
    return max(max(a, max(d.x, d.y)), max(d.z, d.w));
  }
  __device__ static int64_t combine(int64_t a, int64_t b) {
    return a > b ? a : b;
  }
  __device__ static int64_t wave(acc_t a) { return wave_max(a); }
  __device__ static int64_t widen(acc_t a) { return (int64_t)a; }
};

template <>
struct Fold<kOpMin> {
  typedef int acc_t;
  __device__ static acc_t identity() { return kI32Max; }
  __device__ static acc_t add(acc_t a, int x) { return min(a, x); }
  __device__ static acc_t add4(acc_t a, v4i d) {
    return min(min(a, min(d.x, d.y)), min(d.z, d.w));
  }
  __device__ static int64_t combine(int64_t a, int64_t b) {
    return a < b ? a : b;
  }
  __device__ static int64_t wave(acc_t a) { return wave_min(a); }
  __device__ static int64_t widen(acc_t a) { return (int64_t)a; }
};

template <int OP>
__device__ __forceinline__ int64_t wave_combine64(int64_t v) {
  if (OP == kOpSum) return wave_sum(v);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int lo = __shfl_xor((int)(uint32_t)v, o, kWave);
    const int hi = __shfl_xor((int)(v >> 32), o, kWave);
    v = Fold<OP>::combine(v, (int64_t)(((uint64_t)(uint32_t)hi << 32) |
                                       (uint32_t)lo));
  }
  return v;
}

template <int OP, int U>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceParams p) {
  typedef Fold<OP> F;
  __shared__ int64_t red[kWaves];
  __shared__ int is_last;
  const int blk = blockIdx.x;
  const int w = threadIdx.x / kWave;

  typename F::acc_t acc = F::identity();
  // Round-robin tiles, two alternating register buffers (see load_tile).
  const v4i* __restrict__ body = reinterpret_cast<const v4i*>(p.in + p.head);
  const int64_t count = tiles_of(p.ntiles, blk, p.grid);
  if (count > 0) {
    // Both buffers are filled unconditionally (the second load re-reads the
    // only tile when there is one), so every path into the loop has the
    // same loads pending in the same order, and the wait before each tile
    // is for that tile alone.
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
      for (int u = 0; u < U; ++u) acc = F::add4(acc, A[u]);
      pin(acc);
      sched_fence();
      load_tile<U>(body, blk, p.grid, count, i + 2, A);
      sched_fence();
      ready(B);
#pragma unroll
      for (int u = 0; u < U; ++u) acc = F::add4(acc, B[u]);
      pin(acc);
      sched_fence();
      load_tile<U>(body, blk, p.grid, count, i + 3, B);
      sched_fence();
    }
    if (i < count) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc = F::add4(acc, A[u]);
    }
  }
  if (blk == p.grid - 1) {
    const int64_t left = p.n - p.covered;
    for (int64_t i = threadIdx.x; i < left; i += kBlock)
      acc = F::add(acc, p.in[i < p.head ? i : p.covered + i]);
  }
  const int64_t wv = F::wave(acc);
  if (lane() == 0) red[w] = wv;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t b = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) b = F::combine(b, red[i]);
    st_agent(p.partials + blk, b);
  }

  if (!last_to_finish(p.ticket, p.grid, p.epoch, &is_last)) return;

  int64_t v = F::widen(F::identity());
  for (int i = threadIdx.x; i < p.grid; i += kBlock)
    v = F::combine(v, ld_agent(p.partials + i));
  v = wave_combine64<OP>(v);
  if (lane() == 0) red[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t r = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = F::combine(r, red[i]);
    *p.out = r;
  }
}

}  // namespace ltk
