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
//  2. A certified bound T: for k <= 64, a lower bound on the k-th largest
//     of the 64 lane maxima (k lanes then hold an element >= T); for
//     larger k, a lower bound on the k-th largest element itself.  Both
//     come from a short bitwise radix search over ballot counts.
//  3. The elements >= T (about k to 2k of them on random data) are
//     compacted into the wave's LDS buffer at offsets from a wave prefix
//     sum of the per-lane counts.
//  4. Each is ranked by counting (a 64-bit key: biased value, then the
//     complement of its buffer slot, so ranks are distinct and equal
//     values take consecutive ranks); ranks < k are the row's result, in
//     order.
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

// One wave's LDS: kRowCap candidate slots, 16 slots of padding for the
// 16-wide ranking reads, then one slot per lane that takes the writes of
// lanes with nothing to write (so the compaction has no branches).
constexpr int kRowDump = kRowCap + 16;
struct RowsWaveLds {
  alignas(16) int buf[kRowDump + kWave];
};

// Inclusive prefix sum over the wave (row shifts within 16-lane rows, then
// the two row broadcasts), and the wave total.
__device__ __forceinline__ int wave_scan_incl(int v, int& total) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  total = __builtin_amdgcn_readlane(v, 63);
  return v;
}

// Rank each of the m (<= kRowCap) values in buf by counting and write those
// of rank < k to out.  Slots m .. m rounded up to 16 are first set to
// INT_MIN, whose keys never exceed a real one (a real INT_MIN sits in a
// lower slot).  Every lane reads the same 16 bytes at a time (an LDS
// broadcast).
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
    for (int j0 = 0; j0 < m; j0 += 16) {
      v4i o4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) o4[t] = q[j0 / 4 + t];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int o[4] = {o4[t].x, o4[t].y, o4[t].z, o4[t].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 4 * t + e;
          r += (((uint64_t)bias(o[e]) << 32) | (uint32_t)~j) > ki;
        }
      }
    }
    if (i < m && r < k) out[r] = v;
  }
}

template <int V>
__global__ __launch_bounds__(kBlock) void topk_rows_kernel(RowsParams p) {
  __shared__ RowsWaveLds lds[kWaves];
  const int w = threadIdx.x / kWave;
  RowsWaveLds& L = lds[w];
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int n = p.n, k = p.k;

  for (int64_t r = (int64_t)blockIdx.x * kWaves + w; r < p.rows;
       r += nwaves) {
    const int* __restrict__ src = p.in + r * p.ld;
    int* dst = p.out + r * k;

    // 1. The row, lane-strided; slots past n hold INT_MIN (the loads are
    // clamped to the last element, so none is skipped or out of range).
    int x[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int idx = lane() + kWave * j;
      const int v = __builtin_nontemporal_load(src + (idx < n ? idx : n - 1));
      x[j] = idx < n ? v : kI32Min;
    }

    // 2. The bound.
    int mx = x[0], mn = kI32Max;
#pragma unroll
    for (int j = 1; j < V; ++j) mx = max(mx, x[j]);
#pragma unroll
    for (int j = 0; j < V; ++j)
      mn = min(mn, lane() + kWave * j < n ? x[j] : kI32Max);
    const int hi = wave_max(mx);
    const int lo = wave_min(mn);
    int T;
    if (k <= kWave) {
      const unsigned bm[1] = {bias(mx)};
      T = unbias(radix_lower_bound(bias(wave_min(mx)), bias(hi), k, 8,
                                   RegCount<1>{bm}));
    } else {
      unsigned u[V];
#pragma unroll
      for (int j = 0; j < V; ++j) u[j] = bias(x[j]);
      // Padding counts only at INT_MIN, where real elements already
      // number n >= k.
      T = unbias(radix_lower_bound(bias(lo), bias(hi), k, 8,
                                   RegCount<V>{u}));
    }

    // 3. Candidates: elements >= T.  T > INT_MIN keeps the padding out.
    int m = kRowCap + 1;
    if (T > kI32Min) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) c += x[j] >= T;
      const int incl = wave_scan_incl(c, m);
      if (m <= kRowCap) {
        int off = incl - c;
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const bool q = x[j] >= T;
          L.buf[q ? off : kRowDump + lane()] = x[j];
          off += q;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }

    if (m <= kRowCap) {
      // 4. Rank by counting.
      wave_rank_out(L.buf, m, k, dst);
    } else {
      // Exact path: the k-th largest g by radix selection over the row,
      // the elements above g (fewer than k) ranked, then copies of g.
      unsigned u[V];
#pragma unroll
      for (int j = 0; j < V; ++j)
        u[j] = lane() + kWave * j < n ? bias(x[j]) : 0u;
      // Padding is biased to 0 and only counts at 0 (INT_MIN), where the
      // n >= k real elements already reach it.
      const int g = unbias(radix_select(bias(lo), bias(hi), k,
                                        RegCount<V>{u}));
      int c = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) c += x[j] > g;
      int ngt;
      int off = wave_scan_incl(c, ngt) - c;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const bool q = x[j] > g;
        L.buf[q ? off : kRowDump + lane()] = x[j];
        off += q;
      }
      __builtin_amdgcn_wave_barrier();
      wave_rank_out(L.buf, ngt, k, dst);
      for (int j = ngt + lane(); j < k; j += kWave) dst[j] = g;
    }
    // The buffer is reused by the next row: finish reading it first.
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace ltk
