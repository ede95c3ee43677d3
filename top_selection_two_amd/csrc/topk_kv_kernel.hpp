// Key-value Top-K: the k largest elements of an int32 or float32 array
// together with their positions, both stages in one launch.
//
// Sources:
//   [TopK]  "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计", §2
//           (the two-stage design), §6 (the reduction keeps a candidate
//           list of items ordered by their score).
//   [Radix] "GPU基数排序优化：10亿级数据处理与性能调优", §8 (key-value pairs
//           carried together; floating-point keys through a suitable bit
//           transform).
//
// With positions the answer is unique only under a tie rule; the one used
// here orders by value, descending, then by position, ascending.  Every
// element becomes a 64-bit key
//     key = (order(value) << 32) | ~position        (position < 2^32)
// where order() maps the value to an unsigned 32-bit integer with the same
// order (int32: flip the sign bit; float32: flip all bits of negatives,
// the sign bit of the rest, so -0 < +0 and NaNs sit at the two ends).  The
// keys are distinct, so "the k largest keys" is exactly the rule, and the
// key 0 (order 0, position 2^32 - 1) is free to mark an empty list slot.
//
// The structure is that of topk_kernel (see there for the streaming ring,
// the filter and the certified bound); what changes:
//  * Lists hold keys (two VGPRs per slot); insertion compares keys.
//  * The filter still looks at 32-bit values first.  A lane sees its
//    elements in increasing position, so a later element whose value equals
//    the lane's k-th entry is worse than it: the lane-local test stays
//    "skip values <= the k-th entry's value".  The shared bound T is
//    certified on values only, and an element whose value equals T may
//    still win on position, so that test becomes "skip values < T".
//  * The epilogue bound is the exact k-th largest lane-head KEY, found by
//    ranking the 256 head keys; entries with keys >= it (usually about k)
//    are ranked by key.  If too many reach it, the k-th largest key is
//    selected by counting (two 32-bit radix passes) and exactly k remain.
//  * Stage 2 works on keys throughout: block maxima and k-th keys certify
//    the bound T2, survivors are ranked by key (or selected by counting),
//    and the result is written as values (in the input's own bits) plus
//    int64 positions.
#pragma once

#include "topk_kernel.hpp"

namespace ltk {

struct TopkKvParams {
  const int* in;      // int32 values, or float32 bit patterns
  int64_t n;          // < 2^32
  int64_t head;       // leading elements before the first 16-byte boundary
  int64_t ntiles;     // full tiles of the aligned body
  int64_t covered;    // elements in those tiles (they start at `head`)
  int k;
  int grid;
  int refresh;        // certificate refresh period, in tiles (power of 2)
  uint64_t* cand;     // [grid * k]  per-block candidate keys, descending
  uint64_t* heads;    // [grid]      largest candidate key of each block
  uint64_t* kths;     // [grid]      k-th largest candidate key of each block
  uint64_t* ticket;   // completion counter (epoch-tagged, see Tagged)
  uint32_t epoch;     // this launch's
  int* out_v;         // [k]         values (input bits), descending
  int64_t* out_i;     // [k]         their positions
};

// The value as a signed int32 with the order the keys use: the identity for
// int32; for float32 bits b, b with the 31 low bits flipped when negative.
// The map is its own inverse.
template <bool F32>
__device__ __forceinline__ int kv_value(int b) {
  return F32 ? (b ^ ((b >> 31) & 0x7fffffff)) : b;
}

__device__ __forceinline__ uint64_t kv_key(int s, uint32_t pos) {
  return ((uint64_t)bias(s) << 32) | (uint32_t)~pos;
}
__device__ __forceinline__ int key_value(uint64_t key) {
  return unbias((unsigned)(key >> 32));
}
__device__ __forceinline__ uint32_t key_pos(uint64_t key) {
  return ~(uint32_t)key;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) {
  return a > b ? a : b;
}
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) {
  return a < b ? a : b;
}

// A lane's candidate list: slot i holds the key (bias(v[i]) << 32) | w[i],
// kept as its two 32-bit words (the value in its signed order, and the low
// word ~position) so that insertion works on 32-bit registers.  Descending
// by key; an empty slot is the key 0 (v = INT_MIN, w = 0).
template <int KCAP>
struct KvList {
  int v[KCAP];
  uint32_t w[KCAP];
  __device__ __forceinline__ uint64_t key(int i) const {
    return ((uint64_t)bias(v[i]) << 32) | w[i];
  }
};

// Insert the key (xv, xw) into the list (see list_insert); on return
// (xv, xw) is the evicted key.  One comparison per slot decides the slot's
// new key and the key carried on.
//
// LANE_ORDER: the key comes after every key already in this lane's list
// (larger position), which holds for the whole stream: a lane visits its
// elements in increasing position.  Then the key order is the value order
// with the new key placed after equal values, so the value words alone
// decide.  One corner differs from whole keys: a value of INT_MIN never
// displaces an empty slot.  Such an element is never needed: by then its
// block's first tile has supplied 4096 keys that beat it (smaller
// positions, values >= INT_MIN), and k <= 128.  Otherwise (the head and
// tail elements visited last) whole keys are compared.
//
// As in list_insert, the bubble stops after a chunk of 8 slots once no lane
// carries a value above `tsk` (T - 1 for the certified bound T, see
// kv_tsk): a key whose value is below T is never among the top-k, and the
// key carried down only decreases.
template <int KCAP, bool FIT, bool LANE_ORDER>
__device__ __forceinline__ void kv_list_insert(KvList<KCAP>& L, int& xv,
                                               uint32_t& xw, int k, int tsk) {
  static_assert(KCAP % 8 == 0, "list capacity must be a multiple of 8");
#pragma unroll
  for (int c = 0; c < KCAP; c += 8) {
    if ((FIT || c < k) && (c == 0 || ballot(xv > tsk))) {
#pragma unroll
      for (int i = c; i < c + 8; ++i) {
        const int lv = L.v[i];
        const uint32_t lw = L.w[i];
        const bool gt = LANE_ORDER ? xv > lv
                                   : (xv > lv) | ((xv == lv) & (xw > lw));
        L.v[i] = gt ? xv : lv;
        L.w[i] = gt ? xw : lw;
        xv = gt ? lv : xv;
        xw = gt ? lw : xw;
      }
    }
  }
}

// tsk: the shared bound's contribution to the lane threshold: T - 1, or
// INT_MIN while T is INT_MIN (values of INT_MIN are not needed after the
// first tile, see kv_list_insert).
__device__ __forceinline__ int kv_tsk(int tsh) {
  return tsh == kI32Min ? kI32Min : tsh - 1;
}

template <bool F32, int U>
__device__ __forceinline__ void kv_values(v4i (&d)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    d[u].x = kv_value<F32>(d[u].x);
    d[u].y = kv_value<F32>(d[u].y);
    d[u].z = kv_value<F32>(d[u].z);
    d[u].w = kv_value<F32>(d[u].w);
  }
}

// One tile (values already in key order).  A max-of-16 vote rejects the
// whole tile in the common case.  Otherwise each lane marks its elements
// above its threshold and the wave runs insertion rounds: in each round
// every lane inserts its earliest marked element (so a lane still inserts
// in position order), and the rounds end when no lane has one left.  A
// tile with a few admissions spread over many lanes and element slots
// costs one or two rounds instead of one per slot.
template <int KCAP, bool FIT, int U>
__device__ __forceinline__ void kv_consume(KvList<KCAP>& L, const v4i (&d)[U],
                                           uint32_t pos0, int k, int tsk,
                                           int& thr, uint64_t& lost) {
  constexpr int M = 4 * U;
  static_assert(M <= 16, "slot masks are 16 bits");
  int e[M];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    e[4 * u + 0] = d[u].x;
    e[4 * u + 1] = d[u].y;
    e[4 * u + 2] = d[u].z;
    e[4 * u + 3] = d[u].w;
  }
  int m = e[0];
#pragma unroll
  for (int j = 1; j < M; ++j) m = max(m, e[j]);
  if (!ballot(m > thr)) return;
  uint32_t pend = 0;
#pragma unroll
  for (int j = 0; j < M; ++j) pend |= e[j] > thr ? (1u << j) : 0u;
  do {
    // the earliest marked slot j (M when none), its value by a select tree
    const uint32_t j = (uint32_t)__builtin_ctz(pend | (1u << M));
    int a[M];
#pragma unroll
    for (int t = 0; t < M; ++t) a[t] = e[t];
#pragma unroll
    for (int w = M / 2; w >= 1; w >>= 1) {
      const uint32_t bit = (uint32_t)((M / 2) / w);
#pragma unroll
      for (int t = 0; t < w; ++t) a[t] = (j & bit) ? a[2 * t + 1] : a[2 * t];
    }
    // slot j = 4u + c lies at pos0 + 4 * kBlock * u + c
    const uint32_t pos = pos0 + (j >> 2) * (uint32_t)(4 * kBlock) + (j & 3u);
    // The threshold may have risen since the slot was marked; a lane with
    // nothing to insert inserts the empty key, which changes nothing.
    const bool act = pend != 0 && a[0] > thr;
    int xv = act ? a[0] : kI32Min;
    uint32_t xw = act ? ~pos : 0u;
    kv_list_insert<KCAP, FIT, true>(L, xv, xw, k, tsk);
    // An evicted key bounds every later element of this lane (they come at
    // larger positions).
    thr = max(thr, max(xv, tsk));
    // Short lists (FIT false: KCAP < k is allowed) may drop a key of the
    // block's top-k: remember the largest key dropped (see kv_lost).
    if (!FIT) lost = umax64(lost, kv_key(xv, ~xw));
    pend &= pend - 1;
  } while (ballot(pend != 0));
}

// First tile: a bitonic network over the 4U keys (see init_list), on whole
// keys.
template <int KCAP, int U>
__device__ __forceinline__ void kv_init_list(KvList<KCAP>& L,
                                             const v4i (&d)[U], uint32_t pos0,
                                             int& thr) {
  constexpr int M = 4 * U;
  static_assert((M & (M - 1)) == 0, "the network needs a power of two");
  uint64_t v[M];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t p = pos0 + (uint32_t)(4 * kBlock * u);
    v[4 * u + 0] = kv_key(d[u].x, p);
    v[4 * u + 1] = kv_key(d[u].y, p + 1);
    v[4 * u + 2] = kv_key(d[u].z, p + 2);
    v[4 * u + 3] = kv_key(d[u].w, p + 3);
  }
#pragma unroll
  for (int size = 2; size <= M; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          // one comparison: swap when the pair is out of this stage's order
          const bool desc = (i & size) == 0;
          const bool swap = desc ? v[j] > v[i] : v[i] > v[j];
          const uint64_t a = v[i];
          v[i] = swap ? v[j] : a;
          v[j] = swap ? a : v[j];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    L.v[i] = i < M ? key_value(v[i]) : kI32Min;
    L.w[i] = i < M ? (uint32_t)v[i] : 0u;
  }
  if (KCAP <= M) thr = max(thr, L.v[KCAP - 1]);
}

// Certified value bound from the lane-head snapshot (see refresh_bound).
template <int KCAP, class SH>
__device__ __forceinline__ void kv_refresh_bound(const KvList<KCAP>& L,
                                                 int k, int& tsh, int& thr,
                                                 SH& sh) {
  __hip_atomic_store(&sh.heads[threadIdx.x], bias(L.v[0]), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_WORKGROUP);
  unsigned u[kWaves];
  int mx = kI32Min;
#pragma unroll
  for (int j = 0; j < kWaves; ++j) {
    u[j] = __hip_atomic_load(&sh.heads[lane() + kWave * j], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    mx = max(mx, unbias(u[j]));
  }
  const RegCount<kWaves> cnt{u};
  const unsigned lo = bias(tsh);
  if (cnt(lo) >= k) {
    mx = wave_max(mx);
    tsh = unbias(radix_lower_bound(lo, bias(mx), k, 6, cnt));
  }
  thr = max(thr, kv_tsk(tsh));
  // Ties at the top: if this wave's own lists hold at least k entries of
  // the value of its largest head, hv, a later element of value hv loses
  // to all of them (this wave's later elements come at larger positions),
  // so values <= hv can be skipped, not only values < T.  The snapshot's
  // heads cannot certify that: another wave may already be a tile ahead.
  // Only the first four levels are counted (a lower count, so the test
  // stays sufficient): 256 slots cover k <= 128 when the ties spread over
  // half the lanes, and a full KCAP-level walk costs more on distinct
  // values than the rule saves (27 us of 136 on the top-100 of 1e8).
  constexpr int D = KCAP < 4 ? KCAP : 4;
  const int hv = wave_max(L.v[0]);
  int c = 0;
#pragma unroll
  for (int i = 0; i < D; ++i) c += popc(ballot(L.v[i] == hv));
  if (c >= k) thr = max(thr, hv);
}

// Ranks of distinct keys by counting (see block_rank64 and rank_all, which
// do the same for values): the rank of keys[i] is the number of larger
// keys.  kv_block_rank64: n <= 64 keys, whole workgroup, ranks[] zero on
// entry, barriers inside.  kv_rank_all: n <= kBlock, one key per thread,
// keys[] with room for n rounded up to 8; a barrier inside.  Slots past n
// are set to 0, which no real key is below.
__device__ __forceinline__ uint64_t kv_block_rank64(uint64_t* keys, int n,
                                                    int* ranks) {
  const int i = threadIdx.x & (kWave - 1);
  const int g = threadIdx.x / kWave;
  if ((int)threadIdx.x >= n && threadIdx.x < kWave) keys[threadIdx.x] = 0ull;
  __syncthreads();
  const uint64_t v = keys[i];
  const v4i* q = reinterpret_cast<const v4i*>(keys + 16 * g);
  int r = 0;
#pragma unroll
  for (int qq = 0; qq < 8; ++qq) {
    const v4i o4 = q[qq];
    const uint64_t a = ((uint64_t)(uint32_t)o4.y << 32) | (uint32_t)o4.x;
    const uint64_t b = ((uint64_t)(uint32_t)o4.w << 32) | (uint32_t)o4.z;
    r += (a > v) + (b > v);
  }
  if (i < n && r > 0) atomicAdd(&ranks[i], r);
  __syncthreads();
  return v;
}

__device__ __forceinline__ int kv_rank_all(uint64_t* keys, int n,
                                           uint64_t& v) {
  const int t = threadIdx.x;
  const int n8 = (n + 7) & ~7;
  for (int j = n + t; j < n8; j += kBlock) keys[j] = 0ull;
  __syncthreads();
  v = keys[t];
  const v4i* q = reinterpret_cast<const v4i*>(keys);
  int r = 0;
  for (int j0 = 0; j0 < n; j0 += 8) {
    v4i o4[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) o4[qq] = q[j0 / 2 + qq];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint64_t a = ((uint64_t)(uint32_t)o4[qq].y << 32) |
                         (uint32_t)o4[qq].x;
      const uint64_t b = ((uint64_t)(uint32_t)o4[qq].w << 32) |
                         (uint32_t)o4[qq].z;
      r += (a > v) + (b > v);
    }
  }
  return r;
}

// The same for n <= 2 * kBlock keys, two per thread: keys[t] and
// keys[t + kBlock] (0 past n, ranked meaninglessly); keys[] with room for
// 2 * kBlock + 8.  A barrier inside: call uniformly.  Under heavy ties this
// replaces selection by counting (64 block-wide counting steps, each a
// round of barriers: tens of microseconds) with one pass of comparisons.
__device__ __forceinline__ void kv_rank_all2(uint64_t* keys, int n,
                                             uint64_t& v0, int& r0,
                                             uint64_t& v1, int& r1) {
  const int t = threadIdx.x;
  const int n8 = (n + 7) & ~7;
  for (int j = n + t; j < n8; j += kBlock) keys[j] = 0ull;
  __syncthreads();
  v0 = t < n ? keys[t] : 0ull;
  v1 = t + kBlock < n ? keys[t + kBlock] : 0ull;
  const v4i* q = reinterpret_cast<const v4i*>(keys);
  r0 = 0;
  r1 = 0;
  for (int j0 = 0; j0 < n; j0 += 8) {
    v4i o4[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) o4[qq] = q[j0 / 2 + qq];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint64_t a = ((uint64_t)(uint32_t)o4[qq].y << 32) |
                         (uint32_t)o4[qq].x;
      const uint64_t b = ((uint64_t)(uint32_t)o4[qq].w << 32) |
                         (uint32_t)o4[qq].z;
      r0 += (a > v0) + (b > v0);
      r1 += (a > v1) + (b > v1);
    }
  }
}

// Append the lanes where p holds to an LDS key list (one LDS atomic per
// wave); returns the wave's base position (wave-uniform).
__device__ __forceinline__ int kv_wave_append(bool p, uint64_t v,
                                              int* counter, uint64_t* dst,
                                              int cap) {
  const uint64_t b = ballot(p);
  if (b == 0) return 0;
  int base = 0;
  if (lane() == 0) base = atomicAdd(counter, popc(b));
  base = uni(base);
  const int pos = base + lanes_below(b);
  if (p && pos < cap) dst[pos] = v;
  return base;
}

// The k-th largest of a set of distinct keys spread over the workgroup, by
// radix selection with 8-bit digits ([Radix] §3.2's digits, used to select
// instead of sort): eight passes, each counting into a 256-bin LDS
// histogram the digit of every key whose higher digits equal those chosen
// so far, then taking the bin that holds the k-th largest.  (Counting bit
// by bit took 65 passes: key-value top-128 of 1e6 values in [0, 1000),
// which then selected over 521 tied survivors in memory, took 488 us so,
// 107 us with digits.)
// visit(f) calls f(key) for each key this thread holds (a fixed, uniform
// loop structure); at least k keys must exist.  The histogram lives in
// sh.hkeys, free wherever this is called (after the epilogue's use of it).
// Barriers inside: call uniformly.
template <class SH, class Visit>
__device__ __forceinline__ uint64_t kv_select(int k, SH& sh, Visit&& visit) {
  constexpr int kBins = 256;  // one per thread
  static_assert(kBlock == kBins, "one bin per thread");
  unsigned* h = reinterpret_cast<unsigned*>(sh.hkeys);
  const int t = threadIdx.x, w = t / kWave;
  uint64_t prefix = 0ull;
  int kleft = k;
  for (int d = 7; d >= 0; --d) {
    const unsigned shift = 8u * (unsigned)d;
    // The bits above this digit (none for the first).
    const uint64_t high = d == 7 ? 0ull : ~0ull << (shift + 8u);
    h[t] = 0u;
    __syncthreads();
    visit([&](uint64_t key) __attribute__((always_inline)) {
      if ((key & high) == prefix)
        atomicAdd(&h[(unsigned)(key >> shift) & 0xffu], 1u);
    });
    __syncthreads();
    // Thread t looks at bin 255 - t: its inclusive scan is the count of
    // keys in the bucket at or above that bin.
    const int c = (int)h[kBins - 1 - t];
    const int incl_w = wave_scan_incl(c);
    if (lane() == kWave - 1) sh.red[0][w] = incl_w;
    __syncthreads();
    int incl = incl_w;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) incl += j < w ? sh.red[0][j] : 0;
    if (incl >= kleft && incl - c < kleft) {
      sh.bcast[0] = kBins - 1 - t;
      sh.bcast[1] = incl - c;
    }
    __syncthreads();
    prefix |= (uint64_t)(unsigned)sh.bcast[0] << shift;
    kleft -= sh.bcast[1];
    __syncthreads();  // h, red and bcast are written again next pass
  }
  return prefix;
}

// ---- LDS layouts ----------------------------------------------------------
template <int KCAP>
struct TopkKvShared {
  unsigned heads[kBlock];                 // lane-head snapshot (biased)
  alignas(16) uint64_t hkeys[kBlock + 8]; // lane-head keys, then ranks' use
  alignas(16) uint64_t blist[2 * kBlock + 8]; // keys >= the final bound
  int ranks[kWave];
  int bcnt;
  int red[2][kWaves];
  int bcast[8];
  uint64_t bkey[2];
  int is_last;
};

constexpr int kKvSurvCap = 512;  // stage-2 survivor keys staged in LDS
struct KvStage2Lds {
  alignas(16) uint64_t surv[kKvSurvCap + 8];
  alignas(16) uint64_t gmax[kBlock + 8];  // group maxima of the block maxima
  uint64_t heads[kMaxGrid];
  int blocks[kMaxGrid];                   // blocks whose maximum reaches T2
  int longb[kMaxGrid];                    // ... and read past their prefix
  int gmax_rank[kWave];
  int surv_rank[kWave];
};

// Visit entries e0 .. e0 + per - 1 of the candidate key lists of the
// flagged blocks (blocks[0..nb), total = nb * per), 8 agent-coherent 8-byte
// loads per thread in flight at a time; f(valid, key, block, entry) is
// called uniformly, `entry` counted from e0.
template <class F>
__device__ __forceinline__ void kv_scan_lists(const TopkKvParams& p,
                                              const int* blocks, int e0,
                                              int per, int total, F&& f) {
  const int k = p.k;
  constexpr int B = 8;
  for (int base = 0; base < total; base += kBlock * B) {
    uint64_t v[B];
    int lb[B], le[B];
    bool ok[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      int idx = base + j * kBlock + (int)threadIdx.x;
      ok[j] = idx < total;
      idx = ok[j] ? idx : total - 1;
      const int fb = idx / per;
      le[j] = idx - fb * per;
      lb[j] = blocks[fb];
      v[j] = ld_agent(p.cand + (int64_t)lb[j] * k + e0 + le[j]);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) f(ok[j], v[j], lb[j], le[j]);
  }
}

// Every key of the flagged blocks' lists (total = nb * k); f(valid, key).
template <class F>
__device__ __forceinline__ void kv_scan_flagged(const TopkKvParams& p,
                                                const int* blocks, int total,
                                                F&& f) {
  kv_scan_lists(p, blocks, 0, p.k, total,
                [&](bool ok, uint64_t c, int, int)
                    __attribute__((always_inline)) { f(ok, c); });
}

// Write the i-th result (rank r < k) from its key.
template <bool F32>
__device__ __forceinline__ void kv_write_out(const TopkKvParams& p, int r,
                                             uint64_t key) {
  p.out_v[r] = kv_value<F32>(key_value(key));
  p.out_i[r] = (int64_t)key_pos(key);
}

// ---- stage 2 --------------------------------------------------------------
// The grid's k largest keys from the per-block candidates:
//  1. block maxima into LDS (one round trip), the largest block k-th key
//     T2b on the way;
//  2. T2a = the k-th largest of group maxima over disjoint groups of blocks
//     (64 groups for k <= 32, else 256, ranked by key); T2 = max(T2a, T2b):
//     at least k candidate keys are >= T2;
//  3. survivors = candidate keys >= T2 of the blocks whose maximum reaches
//     it (read from memory: the first kPrefix keys of each such list, and
//     the rest only of a list whose kPrefix-th key still reaches T2, as
//     the lists are descending), into LDS;
//  4. up to 256 survivors are ranked; more are cut to exactly k by
//     selecting the k-th largest key by counting, then ranked.
template <bool F32, int KCAP>
__device__ __forceinline__ void topk_kv_stage2(const TopkKvParams& p,
                                               TopkKvShared<KCAP>& sh,
                                               KvStage2Lds& s2) {
  const int G = p.grid, k = p.k, tid = threadIdx.x;
  const int w = tid / kWave;
  if (tid < kWave) {
    s2.gmax_rank[tid] = 0;
    s2.surv_rank[tid] = 0;
  }
  if (tid == 0) {
    sh.bcast[2] = 0;  // survivors
    sh.bcast[5] = 0;  // flagged blocks
    sh.bcast[7] = 0;  // flagged blocks read past their prefix
    sh.bkey[0] = 0;   // T2b
    sh.bkey[1] = 0;   // T2a (stays 0 when equal empty-group keys tie)
  }
  // (1) block maxima into LDS, whole KiB chunks (the heads area holds
  // kMaxGrid keys, so the last chunk stays inside it).
  {
    const int ws = __builtin_amdgcn_readfirstlane(w);
    const char* hsrc = reinterpret_cast<const char*>(uni_ptr(p.heads));
    const uint32_t hlds = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)lds_offset(s2.heads));
    const uint32_t voff = (uint32_t)lane() * 16u;
    const int chunks = (G * 8 + 1023) / 1024;
    for (int c = ws; c < chunks; c += kWaves)
      copy_1k_to_lds(hsrc + c * 1024, hlds + c * 1024u, voff);
  }
  uint64_t kt = 0;
  for (int b = tid; b < G; b += kBlock) kt = umax64(kt, ld_agent(p.kths + b));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  {
    const uint32_t lo = (uint32_t)kt, hi = (uint32_t)(kt >> 32);
    // wave max of a 64-bit key: high words first, then low words of the
    // lanes holding the top high word
    const unsigned whi = (unsigned)unbias(wave_max(unbias(hi)));
    const unsigned wlo = (unsigned)unbias(
        wave_max(unbias(hi == whi ? lo : 0u)));
    if (lane() == 0)
      atomicMax(reinterpret_cast<unsigned long long*>(&sh.bkey[0]),
                (unsigned long long)(((uint64_t)whi << 32) | wlo));
  }
  // (2) group maxima
  // (64 groups only up to k = 32: at k = 64 the k-th largest of 64 group
  // maxima is their least and bounds nothing; key-value top-64 of 1e8
  // took 108.6 us with it against 78.1 us with 256 groups.)
  const bool narrow = k <= kWave / 2;
  if (narrow) {
    if (w == 0) {
      const int per = (G + kWave - 1) / kWave;
      uint64_t gm = 0;
      for (int j = 0; j < per; ++j) {
        const int b = lane() * per + j;
        if (b < G) gm = umax64(gm, s2.heads[b]);
      }
      s2.gmax[lane()] = gm;
    }
  } else {
    const int per = (G + kBlock - 1) / kBlock;
    uint64_t gm = 0;
    for (int j = 0; j < per; ++j) {
      const int b = tid * per + j;
      if (b < G) gm = umax64(gm, s2.heads[b]);
    }
    s2.gmax[tid] = gm;
  }
  __syncthreads();
  // The k-th largest group maximum.  Empty groups hold 0, which certifies
  // nothing (with fewer than k blocks the bound is 0).
  if (narrow) {
    const uint64_t gv = kv_block_rank64(s2.gmax, kWave, s2.gmax_rank);
    if (tid < kWave && s2.gmax_rank[tid] == k - 1) sh.bkey[1] = gv;
  } else {
    uint64_t gv;
    if (kv_rank_all(s2.gmax, kBlock, gv) == k - 1) sh.bkey[1] = gv;
  }
  __syncthreads();
  if (G < k) {
    // Fewer lists than k: their maxima certify nothing.  The first
    // j = ceil(k / G) keys of every list are G j >= k candidates, so the
    // k-th largest of them bounds the result's k-th key (key-value top-128
    // of 5e5 over 122 blocks took 508 us with no bound).  G j < G + k <
    // 2 kMaxK = kBlock keys, one per thread, ranked in s2.gmax (free by
    // now); the bound joins T2b's slot, which stage 2 reads only below.
    const int j = (k + G - 1) / G;
    const int cnt = G * j;
    if (tid < cnt) {
      const int b = tid / j, e = tid - b * j;
      s2.gmax[tid] = ld_agent(p.cand + (int64_t)b * k + e);
    }
    uint64_t v;
    const int rk = kv_rank_all(s2.gmax, cnt, v);
    if (tid < cnt && rk == k - 1) sh.bkey[0] = umax64(sh.bkey[0], v);
    __syncthreads();
  }
  uint64_t T2 = umax64(sh.bkey[0], sh.bkey[1]);

  // (3) flagged blocks, then their candidate keys >= T2.  Survivors are a
  // prefix of each (descending) list: about one per list is usual.
  // Reading whole lists took nflag * k / (8 * kBlock) dependent round
  // trips.
  int nflag = 0, total = 0, m = 0;
  auto gather = [&]() __attribute__((always_inline)) {
    if (tid == 0) {
      sh.bcast[2] = 0;
      sh.bcast[5] = 0;
      sh.bcast[7] = 0;
    }
    __syncthreads();
    for (int b0 = 0; b0 < G; b0 += kBlock) {
      const int b = b0 + tid;
      const bool f = b < G && s2.heads[b] >= T2;
      wave_append(f, b, &sh.bcast[5], s2.blocks, kMaxGrid);
    }
    __syncthreads();
    nflag = sh.bcast[5];
    total = nflag * k;
    const int pf = min(kPrefix, k);
    kv_scan_lists(p, s2.blocks, 0, pf, nflag * pf,
                  [&](bool ok, uint64_t c, int b, int e)
                      __attribute__((always_inline)) {
                        const bool s = ok && c >= T2;
                        kv_wave_append(s, c, &sh.bcast[2], s2.surv,
                                       kKvSurvCap);
                        wave_append(s && e == pf - 1 && k > pf, b,
                                    &sh.bcast[7], s2.longb, kMaxGrid);
                      });
    __syncthreads();
    const int nlong = sh.bcast[7];
    if (nlong > 0) {
      kv_scan_lists(p, s2.longb, pf, k - pf, nlong * (k - pf),
                    [&](bool ok, uint64_t c, int, int)
                        __attribute__((always_inline)) {
                          kv_wave_append(ok && c >= T2, c, &sh.bcast[2],
                                         s2.surv, kKvSurvCap);
                        });
    }
    __syncthreads();
    m = sh.bcast[2];
  };
  gather();
  if (m > 2 * kBlock) {
    // Ties at the top make group maxima a weak bound: they compare keys by
    // position, and the groups are runs of consecutive blocks, whose first
    // tiles are early in the row.  (Key-value top-32 of 1e7 values in
    // [0, 1000): the 32nd largest of 64 group maxima left 1,025 survivors
    // and the selection by counting over memory took 240 us.)  A tighter
    // certified bound from the lists' first keys (below), then gather again
    // with it.  Over 256 blocks, the k-th largest of all G block maxima,
    // each a candidate: wave 0 holds the G maxima, 16 per lane, and selects
    // the k-th largest key by ballots: its high word from that of T2a
    // upwards (the group maxima are block maxima, so at least k of those
    // reach T2a), then its low word among the maxima with that high word.
    const uint64_t t2a = sh.bkey[1];
    __syncthreads();  // every survivor count and bound has been read
    const int jl = min(k, 2 * kBlock / G);  // list entries that fit a ranking
    if (jl >= 2) {
      // Up to 256 blocks: the first jl keys of every list, ranked two per
      // thread (G jl <= 512 keys, at least k).  Under ties a list's first
      // keys are its earliest copies of the top value, so their k-th
      // largest reaches further into the ties than the k-th largest block
      // maximum.  (Key-value top-128 of 1e6 values in [0, 1000) over 192
      // blocks: the k-th block maximum left 521 survivors, more than the
      // ranking holds.)
      const int cnt = G * jl;
      for (int i = tid; i < cnt; i += kBlock) {
        const int b = i / jl, e = i - b * jl;
        s2.surv[i] = ld_agent(p.cand + (int64_t)b * k + e);
      }
      uint64_t v0, v1;
      int r0, r1;
      kv_rank_all2(s2.surv, cnt, v0, r0, v1, r1);
      if (tid < cnt && r0 == k - 1) sh.bkey[1] = v0;
      if (tid + kBlock < cnt && r1 == k - 1) sh.bkey[1] = v1;
    } else if (w == 0) {
      constexpr int V = kMaxGrid / kWave;
      unsigned hu[V], hl[V];
      unsigned mx = 0u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int b = lane() + kWave * j;
        const uint64_t key = b < G ? s2.heads[b] : 0ull;
        hu[j] = (unsigned)(key >> 32);
        hl[j] = (unsigned)key;
        mx = max(mx, hu[j]);
      }
      mx = (unsigned)unbias(wave_max(unbias(mx)));
      const RegCount<V> cnt{hu};
      const unsigned lo_hi = (unsigned)(t2a >> 32);
      const unsigned tv = radix_select(lo_hi, max(mx, lo_hi), k, cnt);
      const int need = k - (tv == 0xffffffffu ? 0 : cnt(tv + 1u));
      auto count_lo = [&](unsigned c) __attribute__((always_inline)) -> int {
        int n = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) n += popc(ballot(hu[j] == tv && hl[j] >= c));
        return n;
      };
      const unsigned tl = radix_select(tv == lo_hi ? (unsigned)t2a : 0u,
                                       0xffffffffu, need, count_lo);
      if (lane() == 0) sh.bkey[1] = ((uint64_t)tv << 32) | tl;
    }
    __syncthreads();
    T2 = umax64(T2, sh.bkey[1]);
    gather();
  }

  // (4) up to 2 * kBlock survivors are ranked two per thread; more (heavy
  // ties) are first cut to exactly k by selecting the k-th key by counting
  if (m > kBlock && m <= 2 * kBlock) {
    uint64_t v0, v1;
    int r0, r1;
    kv_rank_all2(s2.surv, m, v0, r0, v1, r1);
    if (tid < m && r0 < k) kv_write_out<F32>(p, r0, v0);
    if (tid + kBlock < m && r1 < k) kv_write_out<F32>(p, r1, v1);
    return;
  }
  if (m > kBlock) {
    uint64_t g;
    if (m <= kKvSurvCap) {
      g = kv_select(k, sh, [&](auto&& f) {
        for (int i = tid; i < m; i += kBlock) f(s2.surv[i]);
      });
    } else {
      g = kv_select(k, sh, [&](auto&& f) {
        kv_scan_flagged(p, s2.blocks, total, [&](bool ok, uint64_t c) {
          if (ok && c >= T2) f(c);
        });
      });
    }
    // Exactly k keys are >= g: gather them afresh.
    __syncthreads();
    if (tid == 0) sh.bcast[2] = 0;
    __syncthreads();
    if (m <= kKvSurvCap) {
      for (int i0 = 0; i0 < m; i0 += kBlock) {
        const int i = i0 + tid;
        const uint64_t c = i < m ? s2.surv[i] : 0ull;
        const bool q = i < m && c >= g;
        __syncthreads();  // every read of this round before any write
        kv_wave_append(q, c, &sh.bcast[2], s2.surv, kKvSurvCap);
      }
    } else {
      kv_scan_flagged(p, s2.blocks, total, [&](bool ok, uint64_t c) {
        kv_wave_append(ok && c >= g, c, &sh.bcast[2], s2.surv, kKvSurvCap);
      });
    }
    __syncthreads();
    m = sh.bcast[2];  // == k
  }
  if (m <= kWave) {
    const uint64_t v = kv_block_rank64(s2.surv, m, s2.surv_rank);
    if (tid < m) {
      const int r = s2.surv_rank[tid];
      if (r < k) kv_write_out<F32>(p, r, v);
    }
  } else {
    uint64_t v;
    const int r = kv_rank_all(s2.surv, m, v);
    if (tid < m && r < k) kv_write_out<F32>(p, r, v);
  }
}

// Short lists (FIT false: KCAP < k).  A lane keeps its KCAP largest keys,
// so a key of the block's top-k is dropped when one lane meets more than
// KCAP of them.  Every key a lane drops is at most the largest key it
// evicted, `lost` (a key skipped by the lane threshold is below the evicted
// key that raised it, or below the certified bound).  If no lane evicted a
// key above the block's k-th key g (sh.bkey[0], written by the result's
// k-th rank), the lists held every key >= g and the result stands: the
// common case, at the cost of one block maximum.  Otherwise the block's
// top-k is found again, exactly, by counting over its elements read back
// from memory (kv_select: eight passes, then one pass gathering the k
// keys >= the k-th): slower, and only for inputs where one lane of a block
// meets more than KCAP of the block's top-k.  Barriers inside: call
// uniformly, after the result has been written.
template <bool F32, int U, int KCAP>
__device__ __forceinline__ void kv_lost_check(const TopkKvParams& p, int blk,
                                           int k, uint64_t lost,
                                           TopkKvShared<KCAP>& sh,
                                           uint64_t* dst) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.bkey[1] = 0;
  __syncthreads();
  {
    // wave maximum of a 64-bit key: high words, then the low words of the
    // lanes holding the top high word
    const uint32_t lo = (uint32_t)lost, hi = (uint32_t)(lost >> 32);
    const unsigned whi = (unsigned)unbias(wave_max(unbias(hi)));
    const unsigned wlo = (unsigned)unbias(wave_max(unbias(hi == whi ? lo : 0u)));
    if (lane() == 0)
      atomicMax(reinterpret_cast<unsigned long long*>(&sh.bkey[1]),
                (unsigned long long)(((uint64_t)whi << 32) | wlo));
  }
  __syncthreads();
  const uint64_t g = sh.bkey[0], worst = sh.bkey[1];
  if (worst < g) return;

  // Every element of the block as a key, each thread visiting the same
  // number of times (lanes past the end visit the empty key 0).
  auto visit = [&](auto&& f) __attribute__((always_inline)) {
    const v4i* __restrict__ body = reinterpret_cast<const v4i*>(p.in + p.head);
    const int64_t count = tiles_of(p.ntiles, blk, p.grid);
    for (int64_t i = 0; i < count; ++i) {
      const int64_t t = blk + i * p.grid;
      const v4i* src = body + t * (int64_t)(kBlock * U);
      v4i d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = src[u * kBlock + tid];
      kv_values<F32, U>(d);
      const uint32_t pos0 =
          (uint32_t)(p.head + t * (int64_t)(4 * kBlock * U)) + 4u * tid;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t q = pos0 + (uint32_t)(4 * kBlock * u);
        f(kv_key(d[u].x, q));
        f(kv_key(d[u].y, q + 1));
        f(kv_key(d[u].z, q + 2));
        f(kv_key(d[u].w, q + 3));
      }
    }
    if (blk == p.grid - 1) {
      const int64_t left = p.n - p.covered;
      for (int64_t base = 0; base < left; base += kBlock) {
        const int64_t i = base + tid;
        const int64_t pos = i < p.head ? i : p.covered + i;
        f(i < left ? kv_key(kv_value<F32>(p.in[pos]), (uint32_t)pos) : 0ull);
      }
    }
  };
  const uint64_t gk = kv_select(k, sh, visit);
  __syncthreads();
  if (tid == 0) sh.bcnt = 0;
  if (tid < kWave) sh.ranks[tid] = 0;
  __syncthreads();
  visit([&](uint64_t key) {
    kv_wave_append(key >= gk && key != 0ull, key, &sh.bcnt, sh.blist, kBlock);
  });
  __syncthreads();
  const int lb = sh.bcnt;  // == k: keys are distinct
  uint64_t v;
  int rk = kBlock;
  if (lb <= kWave) {
    v = kv_block_rank64(sh.blist, lb, sh.ranks);
    if (tid < lb) rk = sh.ranks[tid];
  } else {
    rk = kv_rank_all(sh.blist, lb, v);
  }
  if (tid < lb && rk < k) {
    st_agent(dst + rk, v);
    if (rk == 0) st_agent(p.heads + blk, v);
    if (rk == k - 1) st_agent(p.kths + blk, v);
  }
}

template <int KCAP, bool FIT, int U, bool F32>
__global__ __launch_bounds__(kBlock) void topk_kv_kernel(TopkKvParams p) {
  __shared__ TopkKvShared<KCAP> sh;
  __shared__ v4i ring_lds[kWaves][kRing][U][kWave];
  static_assert(sizeof(ring_lds) >= sizeof(KvStage2Lds), "ring too small");
  const int blk = blockIdx.x;
  const int k = p.k;
  const int w = threadIdx.x / kWave;

  KvList<KCAP> L;
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    L.v[i] = kI32Min;
    L.w[i] = 0u;
  }
  int tsh = kI32Min;   // this wave's certified value bound
  int thr = kI32Min;   // skip values <= thr (the first tile skips nothing)
  uint64_t lost = 0;   // short lists: the largest key this lane dropped
  sh.heads[threadIdx.x] = 0u;
  if (threadIdx.x == 0) sh.bcnt = 0;
  if (threadIdx.x < kWave) sh.ranks[threadIdx.x] = 0;
  __syncthreads();

  // ---- stage 1: the streaming ring of topk_kernel ----------------------
  const v4i* __restrict__ body = reinterpret_cast<const v4i*>(p.in + p.head);
  const int64_t count = tiles_of(p.ntiles, blk, p.grid);
  const int R = p.refresh;
  if (count > 0) {
    v4i(*ring)[U][kWave] = ring_lds[w];
    uint32_t voff[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      voff[u] = (uint32_t)((u * kBlock + threadIdx.x) * sizeof(v4i));
    const char* first = reinterpret_cast<const char*>(body) +
                        (int64_t)blk * kTileBytes<U>;
    const int64_t stride = (int64_t)p.grid * kTileBytes<U>;
    // Peek at the block's last tile first.  At least k of its lanes hold a
    // value >= the k-th largest of the lane maxima found there, so every
    // value strictly below that is out of the block's top-k, whatever its
    // position; equal values still go through.  Tiles stay in position
    // order.  On ascending input the lanes would otherwise insert nearly
    // every element (key-value top-20 / top-100 of 1e8 sorted took 507 us
    // / 2.5 ms).  The bound is certified on the final lane heads too: a
    // lane whose maximum there reaches it either admits that maximum or
    // passes a higher certified bound.  Cost on uniform input: 0.2 / 0.4 /
    // 0.8 / 2.1 / 3.3 us at top-20 / 32 / 64 / 100 / 128 of 1e8.  (Issuing
    // the ring's first tiles before the peek measured 1 us slower still.)
    if (count >= 2) {
      const v4i* last = reinterpret_cast<const v4i*>(first + (count - 1) * stride);
      v4i e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) e[u] = last[u * kBlock + threadIdx.x];
      kv_values<F32, U>(e);
      int m = kI32Min;
#pragma unroll
      for (int u = 0; u < U; ++u)
        m = max(m, max(max(e[u].x, e[u].y), max(e[u].z, e[u].w)));
      sh.heads[threadIdx.x] = bias(m);
      __syncthreads();
      unsigned hu[kWaves];
      int mx = kI32Min, mn = kI32Max;
#pragma unroll
      for (int j = 0; j < kWaves; ++j) {
        hu[j] = sh.heads[lane() + kWave * j];
        mx = max(mx, unbias(hu[j]));
        mn = min(mn, unbias(hu[j]));
      }
      mx = wave_max(mx);
      mn = wave_min(mn);
      // Eight bits between the least and the largest lane maximum (every
      // lane maximum reaches the least, so the search may start there).
      // Searching from 0 over the whole range left the bound at 0 on small
      // values (all of [0, 1000) shares the top 22 bits): on sorted input
      // every lane then inserted every element through whole-list
      // bubbles.
      tsh = unbias(radix_lower_bound(bias(mn), bias(mx), k, 8,
                                     RegCount<kWaves>{hu}));
      thr = kv_tsk(tsh);
      __syncthreads();  // every wave has read the peeked maxima
      sh.heads[threadIdx.x] = 0u;
    }
    // First position of tile i of this block, advanced per tile.  Tiles
    // go in position order (unlike topk_kernel's tile_order): the
    // value-only admission test skips a value equal to the bound, which is
    // right only if every element behind the bound has an earlier
    // position, that is a larger key.
    uint32_t tpos = (uint32_t)(p.head + (int64_t)blk * (4 * kBlock * U));
    const uint32_t tstep = (uint32_t)p.grid * (uint32_t)(4 * kBlock * U);
#pragma unroll
    for (int j = 0; j < kRing; ++j)
      if (j < count) issue_tile_lds<U>(first + j * stride, voff, ring[j]);
    for (int64_t i = 0; i < count; ++i) {
      wait_tile_loads<U, kRing>(i + kRing - 1 < count);
      const int slot = (int)(i & (kRing - 1));
      v4i d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = ring[slot][u][lane()];
      wait_lds_reads();
      if (i + kRing < count)
        issue_tile_lds<U>(first + (i + kRing) * stride, voff, ring[slot]);
      kv_values<F32, U>(d);
      // Position of this lane's first element of the tile (n < 2^32).
      const uint32_t pos0 = tpos + 4u * threadIdx.x;
      tpos += tstep;
      if (i == 0)
        kv_init_list<KCAP, U>(L, d, pos0, thr);
      else
        kv_consume<KCAP, FIT, U>(L, d, pos0, k, kv_tsk(tsh), thr, lost);
      // After each of the first two tiles every lane publishes its head and
      // the workgroup waits, so that bound refresh sees all 256 fresh
      // heads: the early bounds are much tighter and far fewer elements are
      // admitted in the tiles that follow.
      if (i <= 1) {
        __hip_atomic_store(&sh.heads[threadIdx.x], bias(L.v[0]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
        lds_barrier();
      }
      if (refresh_due(i, R)) kv_refresh_bound(L, k, tsh, thr, sh);
    }
  }
  // The unaligned head and the tail: positions out of the lane's order, so
  // only the shared bound (index-free) filters them; insertion compares
  // whole keys.
  if (blk == p.grid - 1) {
    visit_rest<kBlock * U * 4>(
        p.in, p.n, p.head, p.covered,
        [&](int x, int64_t pos, bool ok) __attribute__((always_inline)) {
          const int s = ok ? kv_value<F32>(x) : kI32Min;
          const bool q = ok && s >= tsh;
          // Inserting the empty key 0 leaves a list unchanged.
          if (ballot(q)) {
            int xv = q ? s : kI32Min;
            uint32_t xw = q ? ~(uint32_t)pos : 0u;
            kv_list_insert<KCAP, FIT, false>(L, xv, xw, k, kv_tsk(tsh));
            if (!FIT) lost = umax64(lost, kv_key(xv, ~xw));
          }
        });
  }

  // ---- epilogue: the block's k largest keys ------------------------------
  // T = the exact k-th largest lane-head key (k distinct heads reach it, so
  // every one of the block's top-k keys does too), found by every wave from
  // the final snapshot: the k-th largest head value by radix select over
  // ballots, then, among the heads of that value, the right one by their
  // low words (a second search only when several heads share the value).
  sh.heads[threadIdx.x] = bias(L.v[0]);
  sh.hkeys[threadIdx.x] = L.key(0);
  __syncthreads();
  uint64_t T;
  {
    unsigned u[kWaves];
    uint32_t lw[kWaves];
    int mx = kI32Min;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) {
      u[j] = sh.heads[lane() + kWave * j];
      lw[j] = (uint32_t)sh.hkeys[lane() + kWave * j];
      mx = max(mx, unbias(u[j]));
    }
    mx = wave_max(mx);
    const RegCount<kWaves> cnt{u};
    // tsh is certified on these heads (they only grew since), so the
    // searches may start there.  First a short search (8 bits): a value
    // that at least k heads reach, hence every one of the block's top-k
    // keys too.  When few heads reach it, the smallest key of that value
    // is the bound; otherwise (many heads near the top, ties) the exact
    // k-th largest head key keeps the candidates few.  For k above 32 the
    // short search rarely leaves few heads, so it is not tried.
    const unsigned tq =
        k <= kWave / 2 ? radix_lower_bound(bias(tsh), bias(mx), k, 8, cnt)
                       : 0u;
    if (k <= kWave / 2 && cnt(tq) <= kWave) {
      T = (uint64_t)tq << 32;
    } else {
    const unsigned tv = radix_select(bias(tsh), bias(mx), k, cnt);
    const int above = tv == 0xffffffffu ? 0 : cnt(tv + 1u);
    const int need = k - above;  // >= 1 heads of value tv are needed
    int ties = 0;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) ties += popc(ballot(u[j] == tv));
    uint32_t tl;
    if (ties == need) {
      // all of them: the smallest low word among them
      uint32_t m = 0xffffffffu;
#pragma unroll
      for (int j = 0; j < kWaves; ++j) m = u[j] == tv ? min(m, lw[j]) : m;
      tl = (uint32_t)unbias((unsigned)wave_min(unbias(m)));
    } else {
      auto count_lo = [&](unsigned c) __attribute__((always_inline)) -> int {
        int n = 0;
#pragma unroll
        for (int j = 0; j < kWaves; ++j)
          n += popc(ballot(u[j] == tv && lw[j] >= c));
        return n;
      };
      tl = radix_select(0u, 0xffffffffu, need, count_lo);
    }
    T = ((uint64_t)tv << 32) | tl;
    }
  }
  uint64_t* dst = p.cand + (int64_t)blk * k;
  {
    bool more = true;  // wave-uniform
#pragma unroll
    for (int i = 0; i < KCAP; ++i) {
      if (more) {
        const bool q = i < k && L.key(i) >= T && L.key(i) != 0ull;
        const uint64_t b = ballot(q);
        more = b != 0;
        if (more) {
          int base = 0;
          if (lane() == 0) base = atomicAdd(&sh.bcnt, popc(b));
          base = uni(base);
          const int pos = base + lanes_below(b);
          if (q && pos < 2 * kBlock) sh.blist[pos] = L.key(i);
          // Stop once the list has overflowed (the count then exceeds
          // 2 * kBlock, which sends the workgroup to the fallback).  A list
          // filled exactly to capacity must go on: a deeper level may hold
          // more entries, and stopping would leave the count looking
          // complete.
          more = base + popc(b) <= 2 * kBlock;
        }
      }
    }
  }
  __syncthreads();
  int lb = sh.bcnt;
  if (lb > 2 * kBlock) {
    // Too many keys reach T: select the k-th largest g among the list
    // entries >= T by counting, then keep exactly the k keys >= g.
    // The entries >= T of a lane are a prefix of its list; each wave visits
    // only as deep as its longest such prefix (a few levels under ties),
    // not all KCAP slots, in each of the 64 counting steps.
    int depth = 0;
    {
      bool more = true;  // wave-uniform
#pragma unroll
      for (int i = 0; i < KCAP; ++i) {
        if (more) {
          more = ballot(i < k && L.key(i) >= T && L.key(i) != 0ull) != 0;
          depth += more;
        }
      }
    }
    const uint64_t g = kv_select(k, sh, [&](auto&& f) {
#pragma unroll
      for (int i = 0; i < KCAP; ++i)
        if (i < depth && L.key(i) >= T && L.key(i) != 0ull) f(L.key(i));
    });
    if (threadIdx.x == 0) sh.bcnt = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KCAP; ++i) {
      const bool q = i < k && L.key(i) >= g && L.key(i) != 0ull;
      kv_wave_append(q, L.key(i), &sh.bcnt, sh.blist, kBlock);
    }
    __syncthreads();
    lb = sh.bcnt;  // == k
  }
  if (lb <= kBlock) {
    uint64_t v;
    int rk = kBlock;
    if (lb <= kWave) {
      v = kv_block_rank64(sh.blist, lb, sh.ranks);
      if ((int)threadIdx.x < lb) rk = sh.ranks[threadIdx.x];
    } else {
      rk = kv_rank_all(sh.blist, lb, v);
    }
    if ((int)threadIdx.x < lb && rk < k) {
      st_agent(dst + rk, v);
      if (rk == 0) st_agent(p.heads + blk, v);
      if (rk == k - 1) {
        st_agent(p.kths + blk, v);
        sh.bkey[0] = v;
      }
    }
  } else {
    // Ties: up to 2 * kBlock keys reach T, ranked two per thread.
    uint64_t v0, v1;
    int r0, r1;
    kv_rank_all2(sh.blist, lb, v0, r0, v1, r1);
    const int t = threadIdx.x;
    if (t < lb && r0 < k) {
      st_agent(dst + r0, v0);
      if (r0 == 0) st_agent(p.heads + blk, v0);
      if (r0 == k - 1) {
        st_agent(p.kths + blk, v0);
        sh.bkey[0] = v0;
      }
    }
    if (t + kBlock < lb && r1 < k) {
      st_agent(dst + r1, v1);
      if (r1 == 0) st_agent(p.heads + blk, v1);
      if (r1 == k - 1) {
        st_agent(p.kths + blk, v1);
        sh.bkey[0] = v1;
      }
    }
  }
  if constexpr (!FIT) kv_lost_check<F32, U>(p, blk, k, lost, sh, dst);

  // ---- hand-off: the last workgroup to finish runs stage 2 --------------
  if (!last_to_finish(p.ticket, p.grid, p.epoch, &sh.is_last)) return;
  topk_kv_stage2<F32, KCAP>(
      p, sh, *reinterpret_cast<KvStage2Lds*>(&ring_lds[0][0][0][0]));
}

}  // namespace ltk
