// Top-K of every row of a matrix whose rows are short (at most 64 * V
// elements): one wave per row, the whole row held in registers.
//
// Sources:
//   [TopK] "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计"
//          §6 (the two-stage pattern as a building block, for instance
//          candidate selection per user in a recommender) and §2 (each
//          thread keeps its share of the row, a cross-thread step merges the
//          shares into the top-k, written in descending order).
//   [Reduce] "CUDA归约优化完全指南：从入门到精通", Level 4 (the final steps of
//          a reduction within one wave, without shared-memory barriers).
//
// gfx950 design.  A short row does not fill a workgroup, and a per-row
// workgroup merge (barriers, a hand-off) would cost more than reading the
// row, so each wave owns whole rows, visiting rows wave, wave + W, ... of
// the launch's W waves:
//  1. Lane l loads elements l, l + 64, l + 128, ... of the row: each load
//     instruction reads 256 consecutive bytes, and any row start and row
//     stride work (no alignment peel).
//  2. A certified bound T: for k <= 32, a lower bound on the k-th largest
//     of the 64 lane maxima (k lanes then hold an element >= T); for
//     larger k, a lower bound on the k-th largest element itself.  Both
//     come from a short bitwise radix search over ballot counts.
//  3. The elements >= T (about k to 2k of them on random data) are
//     compacted into the wave's LDS buffer, one ballot per register slot.
//  4. Up to 64 of them, one per lane, are sorted across the wave by a
//     bitonic network whose exchanges stay in registers (DPP and the
//     gfx950 row swaps); lanes 0..k-1 then hold the result in order.  More
//     candidates (up to 256) are ranked by counting instead (a 64-bit key:
//     biased value, then the complement of the buffer slot, so ranks are
//     distinct and equal values take consecutive ranks).
// Heavy ties (more candidates than the buffer holds) or a bound that
// certifies nothing (INT_MIN) take an exact path: radix selection of the
// k-th largest g over the registers, the elements above g ranked, then
// copies of g.  No MFMA: nothing here is a dense contraction.
#pragma once

#include "wave.hpp"

namespace ltk {

struct RowsParams {
  const int* in;
  int64_t rows;
  int64_t ld;  // elements between row starts
  int n;       // elements per row, 1 <= n <= 64 * V
  int k;       // 1 <= k <= min(n, kMaxK)
  int* out;    // [rows * k]
};

constexpr int kRowCap = 256;  // candidates per wave held in LDS

// One wave's LDS: kRowCap candidate slots, then one slot per lane that
// takes the compaction's stores with nothing to keep (and the ranking's
// padding reads).
struct RowsWaveLds {
  alignas(16) int buf[kRowCap + kWave];
};

// Rank each of the m (<= kRowCap) values in buf by counting and write those
// of rank < k to out.  Slots m .. m rounded up to 16 are first set to
// INT_MIN, whose keys never exceed a real one (a real INT_MIN sits in a
// lower slot).  Every lane reads the same 16 bytes at a time (an LDS
// broadcast); the reads stop at m rounded up to 4.
__device__ __forceinline__ void wave_rank_out(int* buf, int m, int k,
                                              int* out) {
  const int m16 = (m + 15) & ~15;
  if (m + lane() < m16) buf[m + lane()] = kI32Min;
  __builtin_amdgcn_wave_barrier();
  const v4i* q = reinterpret_cast<const v4i*>(buf);
  for (int i0 = 0; i0 < m; i0 += kWave) {
    const int i = i0 + lane();
    const int v = i < m ? buf[i] : kI32Min;
    const uint64_t ki = ((uint64_t)bias(v) << 32) | (uint32_t)~i;
    int r = 0;
    for (int j0 = 0; j0 < m; j0 += 4) {
      const v4i o4 = q[j0 / 4];
      const int o[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + e;
        r += (((uint64_t)bias(o[e]) << 32) | (uint32_t)~j) > ki;
      }
    }
    if (i < m && r < k) out[r] = v;
  }
}

// Sort buf[0..m) (m <= 64 R) descending across the wave, R values per
// lane, and write the first k to out.
template <int R>
__device__ __forceinline__ void sort_out(const int* buf, int m, int k,
                                         int* out) {
  int v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = j * kWave + lane();
    v[j] = i < m ? buf[i] : kI32Min;
  }
  wave_sort_desc_regs<R>(v);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = j * kWave + lane();
    if (i < k) out[i] = v[j];
  }
}

// Append the elements that pass (x[j] > t, or >= t) to buf, one ballot per
// register slot, at offsets from a wave-uniform count; nothing is kept
// past kRowCap.  Every lane stores in every slot, with no branch: a lane
// with nothing to keep (or past kRowCap) writes its own slot after
// kRowCap.  Returns the number that pass (it may exceed kRowCap).  Slots
// past n (when not FULL) never pass: callers use t > INT_MIN, or strict.
template <int V, bool STRICT>
__device__ __forceinline__ int compact(const int (&x)[V], int t, int* buf) {
  int m = 0;  // wave-uniform
  const int spare = kRowCap + lane();
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const bool q = STRICT ? x[j] > t : x[j] >= t;
    const uint64_t b = ballot(q);
    const int pos = m + lanes_below(b);
    buf[min(q ? pos : kI32Max, spare)] = x[j];
    m += popc(b);
  }
  __builtin_amdgcn_wave_barrier();
  return m;
}

// radix_select counter over a row held in registers: the number of
// elements >= the candidate, compared as signed values (no biased copy of
// the row is kept).  Slots past n do not count.
template <int V, bool FULL>
struct RowCount {
  const int (&x)[V];
  int n;
  __device__ __forceinline__ int operator()(unsigned c) const {
    const int t = unbias(c);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < V; ++j)
      cnt += popc(ballot((FULL || lane() + kWave * j < n) && x[j] >= t));
    return cnt;
  }
};

// The top-k of a row of n <= 64 elements, element `lane` in x (INT_MIN
// past n): sorting it across the wave costs less than bounding it first
// (1e6 rows of 30 elements: 328 -> 201 us).
__device__ __forceinline__ void tiny_row_topk(int x, int n, int k, int* out) {
  const int v = n <= 32 ? wave_sort_desc<32>(x) : wave_sort_desc<kWave>(x);
  if (lane() < k) out[lane()] = v;
}

// The top-k of one row held in registers, V slots per lane.  FULL: every
// slot holds an element (in any order).  Otherwise x[j] is element
// lane + 64 j of the row, and slots past n hold INT_MIN and do not count.
// Writes out[0..k), descending.
template <int V, bool FULL>
__device__ __forceinline__ void row_topk(const int (&x)[V], int n, int k,
                                         int* out, RowsWaveLds& L) {
  auto valid = [&](int j) __attribute__((always_inline)) {
    return FULL || lane() + kWave * j < n;
  };
  // 2. The bound.
  int mx = x[0];
#pragma unroll
  for (int j = 1; j < V; ++j) mx = max(mx, x[j]);
  const int hi = wave_max(mx);
  auto row_min = [&]() __attribute__((always_inline)) {
    int mn = kI32Max;
#pragma unroll
    for (int j = 0; j < V; ++j) mn = min(mn, valid(j) ? x[j] : kI32Max);
    return wave_min(mn);
  };
  int T;
  if (k <= 32) {
    // 6 steps: a looser bound admits a few more candidates, but the
    // search costs less (A/B on 97,656 x 1,024 rows, top-20: 6 steps
    // 74.9 us, 8 steps 75.6, 10 steps 76.5).  Beyond k = 32 the k-th
    // largest lane maximum falls fast (at k = 64 it is the smallest, and
    // every element above it is a candidate): the elements are counted
    // instead.
    const unsigned bm[1] = {bias(mx)};
    T = unbias(radix_lower_bound(bias(wave_min(mx)), bias(hi), k, 6,
                                 RegCount<1>{bm}));
  } else {
    T = unbias(radix_lower_bound(bias(row_min()), bias(hi), k, 8,
                                 RowCount<V, FULL>{x, n}));
  }

  // 3. Candidates: elements >= T (T > INT_MIN keeps the padding out); at
  // least k of them, since T is certified.
  const int m = T > kI32Min ? compact<V, false>(x, T, L.buf) : kRowCap + 1;

  if (m <= 32) {
    // 4. The usual case: at most 32 candidates, one per lane of the lower
    // half, sorted there; lanes 0..k-1 then hold the result in order.
    const int v = wave_sort_desc<32>(lane() < m ? L.buf[lane()] : kI32Min);
    if (lane() < k) out[lane()] = v;
  } else if (m <= kWave) {
    const int v = wave_sort_desc<kWave>(lane() < m ? L.buf[lane()] : kI32Min);
    if (lane() < k) out[lane()] = v;
  } else if (T == hi) {
    // The bound is the row maximum: at least k elements equal it, and they
    // are the result (a row of ties would otherwise rank all of them).
    for (int j = lane(); j < k; j += kWave) out[j] = hi;
  } else if (m <= 4 * kWave) {
    // 4'. Up to 256 candidates: two or four per lane, sorted across the
    // wave by a bitonic network (ranking them by counting took O(m^2):
    // 100,000 rows of 100, top-64, 89 us).
    // Rows of up to 512 elements, where k is often large for the row,
    // carry a network for up to 128 too; longer rows one network only (a
    // second made the common path of 97,656 rows of 1,024 about 1 %
    // slower: longer code).
    if (V <= 8 && m <= 2 * kWave)
      sort_out<2>(L.buf, m, k, out);
    else
      sort_out<4>(L.buf, m, k, out);
  } else {
    // Exact path: the k-th largest g by radix selection over the row, the
    // elements above g (fewer than k) ranked, then copies of g.
    const int g = unbias(radix_select(bias(row_min()), bias(hi), k,
                                      RowCount<V, FULL>{x, n}));
    const int ngt = compact<V, true>(x, g, L.buf);
    wave_rank_out(L.buf, ngt, k, out);
    for (int j = ngt + lane(); j < k; j += kWave) out[j] = g;
  }
  // The buffer is reused by the next row: finish reading it first.
  __builtin_amdgcn_wave_barrier();
}

// FULL: every row has exactly 64 * V elements and starts on a 16-byte
// boundary, so lane l loads 16-byte vectors l, l + 64, ... (each wave
// instruction reads 1 KiB of consecutive bytes) with no masks, and for
// rows of up to 1024 elements the next row's loads are issued before the
// current row is processed.
// Otherwise lane l loads single elements l, l + 64, ... clamped to the row
// (each wave instruction reads 256 consecutive bytes), for any row length,
// start and stride.
template <int V, bool FULL>
__global__ __launch_bounds__(kBlock) void topk_rows_kernel(RowsParams p) {
  __shared__ RowsWaveLds lds[kWaves];
  const int w = threadIdx.x / kWave;
  RowsWaveLds& L = lds[w];
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int n = p.n, k = p.k;
  int64_t r = (int64_t)blockIdx.x * kWaves + w;

  if constexpr (V == 1) {
    // Rows of at most 64 elements, one per lane.
    for (; r < p.rows; r += nwaves) {
      const int* __restrict__ src = p.in + r * p.ld;
      const int v =
          __builtin_nontemporal_load(src + (lane() < n ? lane() : n - 1));
      tiny_row_topk(lane() < n ? v : kI32Min, n, k, p.out + r * k);
    }
  } else if constexpr (FULL) {
    static_assert(V % 4 == 0, "whole 16-byte vectors per lane");
    constexpr int Q = V / 4;
    // Longer rows keep enough bytes in flight per wave without a second
    // buffer (and need the registers).
    constexpr bool kPrefetch = V <= 16;
    auto load = [&](int64_t row, v4i (&d)[Q]) __attribute__((always_inline)) {
      const v4i* src = reinterpret_cast<const v4i*>(p.in + row * p.ld);
#pragma unroll
      for (int q = 0; q < Q; ++q)
        d[q] = __builtin_nontemporal_load(src + lane() + kWave * q);
    };
    auto run = [&](const v4i (&d)[Q], int64_t row)
                   __attribute__((always_inline)) {
      int x[V];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        x[4 * q + 0] = d[q].x;
        x[4 * q + 1] = d[q].y;
        x[4 * q + 2] = d[q].z;
        x[4 * q + 3] = d[q].w;
      }
      row_topk<V, true>(x, n, k, p.out + row * k, L);
    };
    if constexpr (kPrefetch) {
      // Two buffers in turn (no register copies between rows): each row's
      // loads are issued before the row before it is processed.
      v4i a[Q], b[Q];
      if (r < p.rows) load(r, a);
      for (; r < p.rows; r += 2 * nwaves) {
        const int64_t r1 = r + nwaves;
        if (r1 < p.rows) load(r1, b);
        run(a, r);
        if (r1 >= p.rows) break;
        if (r1 + nwaves < p.rows) load(r1 + nwaves, a);
        run(b, r1);
      }
    } else {
      for (; r < p.rows; r += nwaves) {
        v4i a[Q];
        load(r, a);
        run(a, r);
      }
    }
  } else {
    for (; r < p.rows; r += nwaves) {
      const int* __restrict__ src = p.in + r * p.ld;
      // Opaque copy of n: keeps the compiler from hoisting the V clamped
      // addresses out of the loop, where they would hold 2 V registers.
      int nn = n;
      asm volatile("" : "+s"(nn));
      int x[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int idx = lane() + kWave * j;
        const int v =
            __builtin_nontemporal_load(src + (idx < nn ? idx : nn - 1));
        x[j] = idx < nn ? v : kI32Min;
      }
      row_topk<V, false>(x, n, k, p.out + r * k, L);
    }
  }
}

}  // namespace ltk
