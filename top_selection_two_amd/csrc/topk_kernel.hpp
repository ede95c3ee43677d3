// Top-K over int32: both stages of the two-stage reduction in one launch.
//
// Sources:
//   [TopK] "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计"
//          §2.1 (stage 1: each thread keeps a descending top-k list over a
//          grid-stride share of the input, the block then merges the lists
//          into its k candidates), §2.2 (stage 2: one block merges the
//          per-block candidates), §4.2 (the insertion test against the
//          list's k-th entry, unrolled), §5.2 (duplicates must survive).
//   [Reduce] "CUDA归约优化完全指南：从入门到精通", Level 3-4 (many elements
//          per thread while loading; wave-level exchange instead of shared
//          memory for the final steps).
//
// What differs from the pages, and why (gfx950, wave64):
//  * Each lane streams 16-byte loads (global_load_dwordx4), U of them per
//    tile; a workgroup owns a contiguous run of tiles.
//  * The insertion test uses a shared, *certified* lower bound T besides the
//    lane's own k-th entry.  T is certified when the lists of this workgroup
//    jointly hold at least k entries >= T; then every element x <= T can be
//    skipped without changing the result (ties included: k copies >= T are
//    already held).  The bound is refreshed on a schedule as the k-th
//    largest of the workgroup's 256 lane heads, found by bitwise radix
//    selection over ballot counts, so that after a few tiles almost every
//    16-element group is rejected by one max-of-16 and one wave vote.
//  * Per-lane lists stay in VGPRs (static indexing, capacity KCAP >= k);
//    insertion is a branch-free max/min bubble that stops at k.
//  * Merges drop everything below T and select by counting rather than by
//    sorting: the wave finds the k-th largest live value g (radix select
//    over ballots), keeps the entries > g and pads with copies of g; wave 0
//    then does the same over the four wave results.  The result of a block
//    is its exact top-k as a multiset (unordered), plus its max and k-th.
//  * Stage 2 runs in the last workgroup to finish (ticket counter, release/
//    acquire fences), not in a second launch.  It first derives a certified
//    bound T2 from the block maxima (k-th largest of them) and the block
//    k-th values (their max), keeps only candidates >= T2, selects the k-th
//    largest g among them, and writes the < k values above g in descending
//    order followed by copies of g.
#pragma once

#include "wave.hpp"

namespace ltk {

struct TopkParams {
  const int* in;
  int64_t n;
  int64_t head;      // leading elements before the first 16-byte boundary
  int64_t ntiles;    // full tiles of the aligned body
  int64_t covered;   // elements in those tiles (they start at `head`)
  int k;
  int grid;          // stage-1 workgroups
  int refresh;       // certificate refresh period, in tiles (power of 2)
  int* cand;         // [grid * k]  per-block candidates (unordered)
  int* heads;        // [grid]      max of each block's candidates
  int* kths;         // [grid]      k-th largest of each block's candidates
  unsigned* ticket;  // completion counter; 0 between calls
  int* out;          // [k]         result, descending
};

constexpr int kSurvCap = 4096;  // stage-2 survivors staged in LDS

template <int KCAP>
struct TopkShared {
  unsigned heads[2][kBlock];
  int wave_out[kWaves][KCAP];
  int wave_cnt[kWaves];
  int red[2][kWaves];
  int bcast[8];
  int is_last;
  int surv[kSurvCap];
  int gt[kMaxK];
};

// Insert x into the descending list L[0..k); returns the new L[k-1].
// Lanes whose x does not exceed L[k-1] leave their list unchanged.
template <int KCAP>
__device__ __forceinline__ int list_insert(int (&L)[KCAP], int x, int k) {
  int hi = x;
  // Constant trip count so the loop unrolls fully and L stays in VGPRs;
  // the guard is a wave-uniform scalar branch.
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    if (i < k) {
      hi = max(L[i], x);
      x = min(L[i], x);
      L[i] = hi;
    }
  }
  return hi;
}

// Wave-uniform count of list entries >= s (lists are descending, so the
// entries >= s form a prefix of each list and the scan stops at the first
// level no lane reaches).
template <int KCAP>
__device__ __forceinline__ int list_count_ge(const int (&L)[KCAP], int k,
                                             int s) {
  int n = 0;
  bool more = true;  // wave-uniform: some lane still reaches this level
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    if (more) {
      const uint64_t b = ballot(i < k && L[i] >= s);
      more = b != 0;
      n += popc(b);
    }
  }
  return n;
}

// Write the wave's list entries >= s (strict: > s) to dst, level by level;
// returns how many there are (only the first `cap` are written).
template <int KCAP>
__device__ __forceinline__ int list_emit(const int (&L)[KCAP], int k, int s,
                                         bool strict, int* dst, int cap) {
  int base = 0;
  bool more = true;  // wave-uniform
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    if (more) {
      const bool p = i < k && (strict ? (L[i] > s) : (L[i] >= s));
      const uint64_t b = ballot(p);
      more = b != 0;
      const int pos = base + lanes_below(b);
      if (p && pos < cap) dst[pos] = L[i];
      base += popc(b);
    }
  }
  return base;
}

// radix_select counter over the wave's lane lists.
template <int KCAP>
struct ListCount {
  const int (&L)[KCAP];
  int k;
  __device__ __forceinline__ int operator()(unsigned c) const {
    return list_count_ge<KCAP>(L, k, unbias(c));
  }
};

template <int KCAP>
__device__ __forceinline__ void admit(int (&L)[KCAP], int x, int k, int tsh,
                                      int& thr) {
  if (ballot(x > thr)) {
    const int last = list_insert<KCAP>(L, x, k);
    thr = max(last, tsh);
  }
}

// One tile's worth of values (U x 4 per lane): a max-of-16 and one vote
// reject the whole group in the common case.
template <int KCAP, int U>
__device__ __forceinline__ void consume(int (&L)[KCAP], const v4i (&d)[U],
                                        int k, int tsh, int& thr) {
  int mu[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    mu[u] = max(max(d[u].x, d[u].y), max(d[u].z, d[u].w));
  int m = mu[0];
#pragma unroll
  for (int u = 1; u < U; ++u) m = max(m, mu[u]);
  if (!ballot(m > thr)) return;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ballot(mu[u] > thr)) continue;
    admit<KCAP>(L, d[u].x, k, tsh, thr);
    admit<KCAP>(L, d[u].y, k, tsh, thr);
    admit<KCAP>(L, d[u].z, k, tsh, thr);
    admit<KCAP>(L, d[u].w, k, tsh, thr);
  }
}

// Raise the workgroup's certified bound to the k-th largest of its 256 lane
// heads (k <= 128 < 256).  Every wave computes the same value from the same
// LDS snapshot.  Contains one barrier: call uniformly across the block.
template <int KCAP>
__device__ __forceinline__ void refresh_bound(const int (&L)[KCAP], int k,
                                              int& tsh, int& thr,
                                              TopkShared<KCAP>& sh, int& buf) {
  sh.heads[buf][threadIdx.x] = bias(L[0]);
  __syncthreads();
  unsigned u[kWaves];
  int mx = kI32Min;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    u[j] = sh.heads[buf][lane() + kWave * j];
    mx = max(mx, unbias(u[j]));
  }
  buf ^= 1;
  const RegCount<kWaves> cnt{u};
  const unsigned lo = bias(tsh);
  if (cnt(lo) >= k) {
    mx = wave_max(mx);
    tsh = unbias(radix_select(lo, bias(mx), k, cnt));
  }
  thr = max(thr, tsh);
}

template <int U>
__device__ __forceinline__ void load_tile(const v4i* __restrict__ body,
                                          int64_t t, v4i (&d)[U]) {
  const int64_t base = t * (int64_t)(kBlock * U) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < U; ++u) d[u] = body[base + u * kBlock];
}

// Block-wide sum of one int per thread (barrier inside; call uniformly).
template <int KCAP>
__device__ __forceinline__ int block_sum(int v, TopkShared<KCAP>& sh,
                                         int& parity) {
  const int64_t ws = wave_sum((int64_t)v);
  if (lane() == 0) sh.red[parity][threadIdx.x / kWave] = (int)ws;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += sh.red[parity][w];
  parity ^= 1;
  return s;
}

// Append the lanes where p holds to an LDS list (one LDS atomic per wave).
__device__ __forceinline__ void wave_append(bool p, int v, int* counter,
                                            int* dst, int cap) {
  const uint64_t b = ballot(p);
  if (b == 0) return;
  int base = 0;
  if (lane() == 0) base = atomicAdd(counter, popc(b));
  base = uni(base);
  const int pos = base + lanes_below(b);
  if (p && pos < cap) dst[pos] = v;
}

// Stage 2, run by the last workgroup: merge grid*k candidates into out[0..k).
template <int KCAP>
__device__ __forceinline__ void topk_stage2(const TopkParams& p,
                                            TopkShared<KCAP>& sh) {
  const int G = p.grid, k = p.k;
  const int w = threadIdx.x / kWave;
  const int tid = threadIdx.x;

  // (A) certified bound from the block summaries (wave 0).
  if (w == 0) {
    constexpr int VH = kMaxGrid / kWave;
    unsigned uh[VH];
    int mx = kI32Min, kt = kI32Min;
#pragma unroll
    for (int j = 0; j < VH; ++j) {
      const int b = lane() + kWave * j;
      int h = kI32Min;
      if (b < G) {
        h = p.heads[b];
        kt = max(kt, p.kths[b]);
      }
      uh[j] = bias(h);
      mx = max(mx, h);
    }
    mx = wave_max(mx);
    kt = wave_max(kt);
    int ta = kI32Min;
    if (G >= k) ta = unbias(radix_select(0u, bias(mx), k, RegCount<VH>{uh}));
    if (lane() == 0) {
      sh.bcast[0] = max(ta, kt);  // T2
      sh.bcast[1] = mx;           // largest candidate
      sh.bcast[2] = 0;            // survivor count
      sh.bcast[3] = 0;            // count of values above g
    }
  }
  __syncthreads();
  const int T2 = sh.bcast[0], mx = sh.bcast[1];

  // (B) survivors >= T2 into LDS.
  const int64_t nc = (int64_t)G * k;
  for (int64_t base = 0; base < nc; base += kBlock) {
    const int64_t i = base + tid;
    const int c = (i < nc) ? p.cand[i] : kI32Min;
    wave_append(i < nc && c >= T2, c, &sh.bcast[2], sh.surv, kSurvCap);
  }
  __syncthreads();
  const int m = sh.bcast[2];

  // (C) g = k-th largest survivor (there are >= k: T2 is certified).
  unsigned g;
  if (m <= 8 * kWave) {
    if (w == 0) {
      unsigned u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = lane() + kWave * j;
        u[j] = q < m ? bias(sh.surv[q]) : 0u;
      }
      g = radix_select(bias(T2), bias(mx), k, RegCount<8>{u});
      if (lane() == 0) sh.bcast[4] = (int)g;
    }
    __syncthreads();
    g = (unsigned)sh.bcast[4];
  } else {
    int parity = 0;
    const bool in_lds = m <= kSurvCap;
    auto count_ge = [&](unsigned c) __attribute__((always_inline)) -> int {
      const int s = unbias(c);
      int mine = 0;
      if (in_lds) {
        for (int i = tid; i < m; i += kBlock) mine += sh.surv[i] >= s;
      } else {
        for (int64_t i = tid; i < nc; i += kBlock) {
          const int v = p.cand[i];
          mine += (v >= s) & (v >= T2);
        }
      }
      return block_sum(mine, sh, parity);
    };
    g = radix_select(bias(T2), bias(mx), k, count_ge);
  }
  const int gs = unbias(g);

  // (D) values above g (fewer than k), ranked; then copies of g.
  if (m <= kSurvCap) {
    for (int base = 0; base < m; base += kBlock) {
      const int i = base + tid;
      const int c = i < m ? sh.surv[i] : kI32Min;
      wave_append(i < m && c > gs, c, &sh.bcast[3], sh.gt, kMaxK);
    }
  } else {
    for (int64_t base = 0; base < nc; base += kBlock) {
      const int64_t i = base + tid;
      const int c = (i < nc) ? p.cand[i] : kI32Min;
      wave_append(i < nc && c > gs, c, &sh.bcast[3], sh.gt, kMaxK);
    }
  }
  __syncthreads();
  const int ngt = sh.bcast[3];
  if (tid < ngt) {
    const int v = sh.gt[tid];
    int r = 0;
    for (int j = 0; j < ngt; ++j) {
      const int o = sh.gt[j];
      r += (o > v) | ((o == v) & (j < tid));
    }
    p.out[r] = v;
  } else if (tid < k) {
    p.out[tid] = gs;
  }
  if (tid == 0) *p.ticket = 0u;
}

template <int KCAP, int U>
__global__ __launch_bounds__(kBlock) void topk_kernel(TopkParams p) {
  __shared__ TopkShared<KCAP> sh;
  const int blk = blockIdx.x;
  const int k = p.k;
  const int w = threadIdx.x / kWave;

  int L[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; ++i) L[i] = kI32Min;
  int tsh = kI32Min;  // certified bound shared by the workgroup
  int thr = kI32Min;  // this lane's test: max(L[k-1], tsh)
  int buf = 0;

  // ---- stage 1: stream this workgroup's tiles ---------------------------
  const v4i* __restrict__ body = reinterpret_cast<const v4i*>(p.in + p.head);
  const int64_t t0 = p.ntiles * blk / p.grid;
  const int64_t t1 = p.ntiles * (blk + 1) / p.grid;
  const int R = p.refresh;
  v4i cur[U], nxt[U];
  if (t0 < t1) load_tile<U>(body, t0, cur);
  for (int64_t t = t0; t < t1; ++t) {
    if (t + 1 < t1) load_tile<U>(body, t + 1, nxt);
    consume<KCAP, U>(L, cur, k, tsh, thr);
    const int j = (int)(t - t0);
    if ((j < R && (j & (j + 1)) == 0) || (j & (R - 1)) == R - 1)
      refresh_bound<KCAP>(L, k, tsh, thr, sh, buf);
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
  // Elements outside the full tiles: the unaligned head and the tail.
  if (blk == p.grid - 1) {
    const int64_t left = p.n - p.covered;
    for (int64_t base = 0; base < left; base += kBlock) {
      const int64_t i = base + threadIdx.x;
      int x = kI32Min;
      if (i < left) x = p.in[i < p.head ? i : p.covered + i];
      admit<KCAP>(L, x, k, tsh, thr);
    }
  }
  refresh_bound<KCAP>(L, k, tsh, thr, sh, buf);
  const int T = tsh;

  // ---- wave merge: each wave's top-k of its entries >= T ----------------
  {
    const int live = list_count_ge<KCAP>(L, k, T);
    int cnt;
    if (live <= k) {
      list_emit<KCAP>(L, k, T, false, sh.wave_out[w], KCAP);
      cnt = live;
    } else {
      const int hi = wave_max(L[0]);
      const unsigned g =
          radix_select(bias(T), bias(hi), k, ListCount<KCAP>{L, k});
      const int gs = unbias(g);
      const int above = list_emit<KCAP>(L, k, gs, true, sh.wave_out[w], KCAP);
      for (int j = lane(); j < k - above; j += kWave)
        sh.wave_out[w][above + j] = gs;
      cnt = k;
    }
    if (lane() == 0) sh.wave_cnt[w] = cnt;
  }
  __syncthreads();

  // ---- block merge (wave 0): top-k of the four wave results -------------
  if (w == 0) {
    constexpr int V = kWaves * KCAP / kWave;
    unsigned u[V];
    int mx = kI32Min;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int q = lane() + kWave * j;
      const int ww = q / KCAP, o = q % KCAP;
      const int v = o < sh.wave_cnt[ww] ? sh.wave_out[ww][o] : kI32Min;
      u[j] = bias(v);
      mx = max(mx, v);
    }
    mx = wave_max(mx);
    const unsigned g = radix_select(bias(T), bias(mx), k, RegCount<V>{u});
    int* dst = p.cand + (int64_t)blk * k;
    int base = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const bool q = u[j] > g;
      const uint64_t b = ballot(q);
      if (q) dst[base + lanes_below(b)] = unbias(u[j]);
      base += popc(b);
    }
    for (int j = lane(); j < k - base; j += kWave) dst[base + j] = unbias(g);
    if (lane() == 0) {
      p.heads[blk] = mx;
      p.kths[blk] = unbias(g);
    }
  }

  // ---- hand-off: the last workgroup to finish runs stage 2 --------------
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    sh.is_last = atomicAdd(p.ticket, 1u) == (unsigned)(p.grid - 1);
  __syncthreads();
  if (!sh.is_last) return;
  __threadfence();
  topk_stage2<KCAP>(p, sh);
}

}  // namespace ltk
