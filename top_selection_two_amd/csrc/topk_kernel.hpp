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
//  * Tiles (256 lanes x U x 16 bytes) are dealt round-robin to the
//    workgroups; each wave streams its quarter of every tile straight into
//    its own LDS ring (global-to-LDS loads, non-temporal) kRing tiles ahead
//    of the one it examines, so inserting never leaves the memory pipe
//    empty.  A lane's first tile fills its list through a sorting network.
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
//  * The workgroup's candidates are its exact top-k: the list entries that
//    reach the final bound T (usually about k of them) are gathered in LDS
//    and each is ranked by counting, which also orders them; only under
//    heavy ties do the waves fall back to selection (radix select over
//    ballots).  Each workgroup also publishes its largest candidate and its
//    k-th.
//  * Stage 2 runs in the last workgroup to finish (ticket counter and
//    agent-coherent stores and loads, see last_to_finish), not in a second
//    launch.  It keeps only candidates >= a certified bound T2 (k
//    candidates are known to reach it) and ranks the survivors by counting;
//    see topk_stage2.
#pragma once

#include "wave.hpp"

namespace ltk {

// One launch covers `rows` rows of n elements each (row r starts at
// in + r * ld); a single array is one row.  Each row gets `grid`
// workgroups, blockIdx.x = row * grid + sub.  With grid > 1 the per-block
// candidates of row r sit at cand + r * grid * k (heads, kths at
// r * grid) and the last of the row's workgroups to finish merges them;
// with grid == 1 the workgroup's own top-k is the row's result.
struct TopkParams {
  const int* in;
  int64_t n;         // elements per row
  int64_t ld;        // elements between row starts
  int k;
  int grid;          // stage-1 workgroups per row
  int refresh;       // certificate refresh period, in tiles (power of 2)
  int* cand;         // [rows * grid * k]  per-block candidates
  int* heads;        // [rows * grid]      max of each block's candidates
  int* kths;         // [rows * grid]      k-th largest of each block's
  uint64_t* ticket;  // [rows]             completion counters (see Tagged)
  uint32_t epoch;    // this launch's
  int* out;          // [rows * k]         results, descending
};

// Where a row's elements lie: `head` leading elements before the first
// 16-byte boundary, then `ntiles` full tiles (`covered` elements), then the
// tail.
struct RowGeometry {
  int64_t head, ntiles, covered;
};

template <int U>
__device__ __forceinline__ RowGeometry row_geometry(const int* row,
                                                    int64_t n) {
  RowGeometry g;
  const uint32_t a = (uint32_t)(uintptr_t)row;
  g.head = (int64_t)(((16u - (a & 15u)) & 15u) >> 2);
  if (g.head > n) g.head = n;
  g.ntiles = ((n - g.head) >> 2) / (kBlock * U);
  g.covered = g.ntiles * (kBlock * U * 4);
  return g;
}

// A set of descending candidate lists: list b holds its entries at
// cand[b * stride + e], e < per.
struct CandView {
  const int* cand;
  int64_t stride;
  int per;
};

constexpr int kSurvCap = 1024;  // stage-2 survivors staged in LDS
constexpr int kRing = 4;        // tiles in flight per wave (power of 2)
template <int U>
constexpr int64_t kTileBytes = (int64_t)kBlock * U * 16;  // one tile

// The tile examined i-th of a workgroup's `count`: the last one first,
// then the rest in order.  Any order gives the same result (equal values
// are interchangeable here; the key-value kernel, where positions break
// ties, keeps position order); this one keeps monotone input cheap.  In ascending order each lane would otherwise meet
// ever larger values and insert nearly every element (top-64 of 1e8 sorted
// took 541 us); in descending order the first tile, examined second, fills
// the lists and the bound from the largest values.
__device__ __forceinline__ int64_t tile_order(int64_t i, int64_t count) {
  return i == 0 ? count - 1 : i - 1;
}

// Stage-2 scratch in LDS.  It lives in the memory of the last workgroup's
// streaming ring (declared separately, see topk_kernel), which is idle by
// then.  `cand` receives every candidate when grid*k <= kDirectCand.
constexpr int kDirectCand = 12288;
static_assert(2 * kMaxK <= kBlock, "stage 2 ranks up to 2k values, one per thread");

struct Stage2Lds {
  int surv[kSurvCap];
  int gt[kMaxK];
  int blocks[kMaxGrid];  // blocks whose maximum reaches T2
  int heads[kMaxGrid];   // block maxima
  int cand[kDirectCand];
  alignas(16) int gmax[kBlock + 16];  // group maxima of the block maxima
  int gmax_rank[kWave];
  int surv_rank[kWave];
};

template <int KCAP>
struct TopkShared {
  unsigned heads[kBlock];  // snapshot of the lane heads (biased)
  // List entries >= the final bound, gathered from all waves, and their
  // ranks (see block_rank64).
  alignas(16) int blist[kBlock + 16];
  int ranks[kWave];
  int bcnt;
  int wave_out[kWaves][kMaxK];  // each wave's top-k (k <= kMaxK)
  int wave_cnt[kWaves];
  int kth;                      // the result's k-th value
  int red[2][kWaves];
  int bcast[8];
  int is_last;
};

// Insert x into the descending list; returns the evicted value.  The
// bubble (min into a temporary, max in place: two instructions per slot)
// runs over the slots up to k8, the first multiple of 8 that is >= k, so
// the list holds the top-k8 >= k of the elements admitted to it.  Every
// entry left in the list is >= the evicted value, so that value is a valid
// lane threshold.  Lanes whose x does not exceed L[k8-1] leave their list
// unchanged (and return x).
//
// The bubble stops early, after any chunk of 8 slots, once no lane carries
// a value >= `floor`, a certified bound of the workgroup: a value below it
// is never among the top-k (see the filter in consume), and the value
// carried down only decreases, so dropping it there loses nothing.  The
// slots below keep their old, still valid, entries.
//
// FIT: the capacity is exactly k8, so every slot is used.  Otherwise (large
// k) the slots beyond k8 stay INT_MIN and whole chunks of 8 are skipped
// with one wave-uniform branch each.
template <int KCAP, bool FIT>
__device__ __forceinline__ int list_insert(int (&L)[KCAP], int x, int k,
                                           int floor) {
  static_assert(KCAP % 8 == 0, "list capacity must be a multiple of 8");
#pragma unroll
  for (int c = 0; c < KCAP; c += 8) {
    if ((FIT || c < k) && (c == 0 || ballot(x >= floor))) {
#pragma unroll
      for (int i = c; i < c + 8; ++i) {
        const int lo = min(L[i], x);
        L[i] = max(L[i], x);
        x = lo;
      }
    }
  }
  return x;
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

// `lost`: with short lists (FIT false: KCAP < k is allowed), the largest
// value this lane evicted (see short_list_check).
template <int KCAP, bool FIT>
__device__ __forceinline__ void admit(int (&L)[KCAP], int x, int k, int tsh,
                                      int& thr, int& lost) {
  if (ballot(x > thr)) {
    const int evicted = list_insert<KCAP, FIT>(L, x, k, tsh);
    thr = max(thr, max(evicted, tsh));
    if (!FIT) lost = max(lost, evicted);
  }
}

// One tile's worth of values (U x 4 per lane).  A max-of-16 and one vote
// reject the whole tile in the common case.  Otherwise each lane marks its
// elements above its threshold and the wave runs insertion rounds: in each
// round every lane inserts one marked element (its earliest, picked by a
// select tree), until no lane has one left.  Admissions spread over many
// lanes and element slots then cost one or two rounds instead of one per
// slot.
template <int KCAP, bool FIT, int U>
__device__ __forceinline__ void consume(int (&L)[KCAP], const v4i (&d)[U],
                                        int k, int tsh, int& thr, int& lost) {
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
    // The threshold may have risen since the element was marked; a lane
    // with nothing to insert inserts INT_MIN, which changes nothing.
    const int x = (pend != 0 && a[0] > thr) ? a[0] : kI32Min;
    const int evicted = list_insert<KCAP, FIT>(L, x, k, tsh);
    thr = max(thr, max(evicted, tsh));
    if (!FIT) lost = max(lost, evicted);
    pend &= pend - 1;
  } while (ballot(pend != 0));
}

// The first tile of a lane's stream goes straight into its (empty) list:
// a bitonic sorting network orders the 4U values (descending, no branches,
// 2 instructions per compare-exchange), and the list keeps the largest
// min(KCAP, 4U) of them -- the same list that inserting them one by one
// would build.
template <int KCAP, int U>
__device__ __forceinline__ void init_list(int (&L)[KCAP], const v4i (&d)[U],
                                          int& thr) {
  constexpr int M = 4 * U;
  static_assert((M & (M - 1)) == 0, "the network needs a power of two");
  int v[M];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    v[4 * u + 0] = d[u].x;
    v[4 * u + 1] = d[u].y;
    v[4 * u + 2] = d[u].z;
    v[4 * u + 3] = d[u].w;
  }
#pragma unroll
  for (int size = 2; size <= M; size <<= 1) {
#pragma unroll
    for (int stride = size / 2; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const int hi = max(v[i], v[j]);
          const int lo = min(v[i], v[j]);
          const bool desc = (i & size) == 0;
          v[i] = desc ? hi : lo;
          v[j] = desc ? lo : hi;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KCAP; ++i) L[i] = i < M ? v[i] : kI32Min;
  thr = KCAP <= M ? L[KCAP - 1] : kI32Min;
}

// Raise this wave's certified bound towards the k-th largest of the
// workgroup's 256 lane heads (k <= 128 < 256).
//
// Every lane keeps its current head (list maximum) in an LDS snapshot.  A
// list's head never decreases, so any value that was ever a lane's head is
// still <= that lane's current head: the k-th largest of ANY mix of current
// and older snapshot entries is <= the k-th largest current head, hence
// certified.  A wave therefore publishes its own heads and reads the
// snapshot without waiting for the other waves: no barrier, and each wave
// keeps its own bound.  The top 6 undecided bits of the search are enough:
// the bound lands within 1/64 of the gap between the old bound and the
// k-th head, for a fraction of the steps.
template <int KCAP, class SH>
__device__ __forceinline__ void refresh_bound(const int (&L)[KCAP], int k,
                                              int& tsh, int& thr, SH& sh) {
  __hip_atomic_store(&sh.heads[threadIdx.x], bias(L[0]), __ATOMIC_RELAXED,
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
  thr = max(thr, tsh);
}

// Refresh after local tiles 0, 1, 3 (while the bound improves fastest), then
// after every R-th tile.
__device__ __forceinline__ bool refresh_due(int64_t j, int R) {
  return (j < R && (j & (j + 1)) == 0) || (j & (R - 1)) == R - 1;
}

// Block-wide sum of one int per thread (barrier inside; call uniformly).
template <class SH>
__device__ __forceinline__ int block_sum(int v, SH& sh,
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

// Visit the candidates of the flagged blocks (blocks[0..nb), cv.per each;
// total = nb * cv.per): 16 independent agent-coherent loads per thread are
// in flight before any is used.  f(valid, value, list, entry) is called
// uniformly across the block; `list` is the entry's list in cv.
template <class F>
__device__ __forceinline__ void scan_flagged_at(const CandView& cv,
                                                const int* blocks, int total,
                                                F&& f) {
  const int per = cv.per;
  constexpr int B = 16;
  for (int base = 0; base < total; base += kBlock * B) {
    int v[B], lb[B], le[B];
    bool ok[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      int idx = base + j * kBlock + (int)threadIdx.x;
      ok[j] = idx < total;
      idx = ok[j] ? idx : total - 1;
      const int fb = idx / per;
      le[j] = idx - fb * per;
      lb[j] = blocks[fb];
      v[j] = ld_agent(cv.cand + (int64_t)lb[j] * cv.stride + le[j]);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) f(ok[j], v[j], lb[j], le[j]);
  }
}

// The same with f(valid, value).
template <class F>
__device__ __forceinline__ void scan_flagged(const CandView& cv,
                                             const int* blocks, int total,
                                             F&& f) {
  scan_flagged_at(cv, blocks, total,
                  [&](bool ok, int v, int, int) __attribute__((always_inline)) {
                    f(ok, v);
                  });
}

// Entries read first from each flagged list that is not in LDS.
constexpr int kPrefix = 8;

// ---- stage 2, run by the last workgroup ---------------------------------
// Merge grid*k candidates into out[0..k):
//  1. One round trip to memory copies every block maximum into LDS
//     (device-coherent global-to-LDS loads), and every candidate too when
//     grid*k <= kDirectCand; the largest block k-th value T2b is read on
//     the way.
//  2. T2a = the k-th largest of group maxima over disjoint groups of blocks
//     (64 groups for k <= 32, else 256): k distinct candidates reach it.
//     T2 = max(T2a, T2b) is certified: at least k candidates are >= T2.
//  3. Only blocks whose maximum reaches T2 can contribute; their candidates
//     >= T2 (the survivors) go to LDS, read from LDS or, when they were not
//     copied, from memory.
//  4. Few survivors (the usual case) are ranked by counting, which writes
//     the result in order.  Many (heavy ties near the top) go through
//     selection of the k-th largest by counting; if more than kSurvCap
//     survive, the counting rescans the flagged blocks in memory.
// Each step is spread over the whole workgroup with barriers between: a
// serial loop in one wave would cost a round trip between the vector and
// scalar units per element.

struct Stage2Bound {
  int t2;     // certified: at least k candidates are >= t2
  int mx;     // the largest candidate
  int m;      // survivors (>= t2); those beyond kSurvCap were not stored
  int total;  // candidates of the flagged blocks
};

// Copy 1 KiB of device memory that other workgroups published (with
// agent-scope stores, before their ticket) into LDS: 16 bytes per lane,
// lane-contiguous, a device-coherent load (sc1) like ld_agent.  `src` and
// `lds` (an LDS byte address) must be wave-uniform values in scalar
// registers; `voff` is lane() * 16.
__device__ __forceinline__ void copy_1k_to_lds(const char* src, uint32_t lds,
                                               uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "global_load_lds_dwordx4 %[vo], %[base] sc1\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [lds] "s"(lds), [vo] "v"(voff), [base] "s"(src)
      : "memory");
}

// Ranking by counting.  The rank of vals[i] among vals[0..n) is how many
// of them are larger, or equal at a lower index, so the ranks of
// vals[0..n) are 0..n-1 in descending order of value.  Each comparison is
// one unsigned 64-bit compare of keys (biased value, then the complement
// of the index), so it stays in the vector unit; slots past n are first
// set to INT_MIN, whose keys never exceed a real one (a real INT_MIN has a
// lower index).
__device__ __forceinline__ uint64_t rank_key(int v, int i) {
  return ((uint64_t)bias(v) << 32) | (uint32_t)~i;
}

// n <= 64, with the whole workgroup: thread t compares value t % 64 with
// the 16 values 16 * (t / 64) .. + 15; the four partial counts meet in
// ranks[] by LDS atomics.  vals: 16-byte aligned, 64 slots; ranks: 64
// slots, zero on entry (set before an earlier barrier).  Barriers inside:
// call uniformly.  Returns this thread's value (meaningful for threads
// < n); its rank is then ranks[threadIdx.x].
__device__ __forceinline__ int block_rank64(int* vals, int n, int* ranks) {
  const int i = threadIdx.x & (kWave - 1);
  const int g = threadIdx.x / kWave;
  if ((int)threadIdx.x >= n && threadIdx.x < kWave) vals[threadIdx.x] = kI32Min;
  __syncthreads();
  const int v = vals[i];
  const uint64_t ki = rank_key(v, i);
  const v4i* q = reinterpret_cast<const v4i*>(vals + 16 * g);
  int r = 0;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const v4i o4 = q[qq];
    const int o[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r += rank_key(o[e], 16 * g + 4 * qq + e) > ki;
  }
  if (i < n && r > 0) atomicAdd(&ranks[i], r);
  __syncthreads();
  return v;
}

// n <= kBlock, one value per thread: thread t ranks vals[t] against all n,
// 16 values per step, all read before any is used.  vals: 16-byte
// aligned, kBlock + 16 slots.  A barrier inside: call uniformly.  Threads
// t >= n get a meaningless result.
__device__ __forceinline__ int rank_all(int* vals, int n, int& v) {
  const int t = threadIdx.x;
  const int n16 = (n + 15) & ~15;
  for (int j = n + t; j < n16; j += kBlock) vals[j] = kI32Min;
  __syncthreads();
  v = vals[t];
  const uint64_t kt = rank_key(v, t);
  const v4i* q = reinterpret_cast<const v4i*>(vals);
  int r = 0;
  for (int j0 = 0; j0 < n; j0 += 16) {
    v4i o4[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) o4[qq] = q[j0 / 4 + qq];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int o[4] = {o4[qq].x, o4[qq].y, o4[qq].z, o4[qq].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) r += rank_key(o[e], j0 + 4 * qq + e) > kt;
    }
  }
  return r;
}

// (1) Fill for the top-k kernel's own candidates: whole KiB chunks of the
// block maxima (and of every candidate when all_in_lds) go to LDS in one
// round trip; the largest block k-th value is T2b.  The last chunk may read
// up to 1 KiB past a row's maxima or candidates: the maxima are followed by
// the k-th values and the candidates by the maxima in the scratch area, so
// it stays inside it, and the LDS areas hold kMaxGrid and kDirectCand
// (multiples of 256) ints.  Ints past G or `total` are ignored.
template <class SH>
__device__ __forceinline__ void stage2_fill_blocks(const int* heads,
                                                   const int* kths,
                                                   const int* cand, int G,
                                                   int total, bool all_in_lds,
                                                   SH& sh, Stage2Lds& s2) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  constexpr int kChunkInts = 1024 / 4;
  const int hchunks = (G + kChunkInts - 1) / kChunkInts;
  const int chunks =
      hchunks + (all_in_lds ? (total + kChunkInts - 1) / kChunkInts : 0);
  {
    // Scalar bookkeeping: the wave index as a scalar, so that every
    // address below is computed once per wave, not per lane.
    const int ws = __builtin_amdgcn_readfirstlane(w);
    const char* hsrc = reinterpret_cast<const char*>(uni_ptr(heads));
    const char* csrc = reinterpret_cast<const char*>(uni_ptr(cand));
    const uint32_t hlds = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)lds_offset(s2.heads));
    const uint32_t clds = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)lds_offset(s2.cand));
    const uint32_t voff = (uint32_t)lane() * 16u;
    for (int c = ws; c < chunks; c += kWaves) {
      if (c < hchunks)
        copy_1k_to_lds(hsrc + c * 1024, hlds + c * 1024u, voff);
      else
        copy_1k_to_lds(csrc + (c - hchunks) * 1024,
                       clds + (c - hchunks) * 1024u, voff);
    }
  }
  int kt = kI32Min;
  for (int b = tid; b < G; b += kBlock) kt = max(kt, ld_agent(kths + b));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  kt = wave_max(kt);
  if (lane() == 0) atomicMax(&sh.bcast[6], kt);
}

// (1) Fill for G descending lists seen through a view (merging): each
// list's first entry is its maximum; a list of at least k entries
// certifies its k-th (T2b).
template <class SH>
__device__ __forceinline__ void stage2_fill_lists(const CandView& cv, int G,
                                                  int k, SH& sh,
                                                  Stage2Lds& s2) {
  int kt = kI32Min;
  for (int b = threadIdx.x; b < G; b += kBlock) {
    const int* l = cv.cand + (int64_t)b * cv.stride;
    s2.heads[b] = ld_agent(l);
    if (cv.per >= k) kt = max(kt, ld_agent(l + (k - 1)));
  }
  __syncthreads();
  kt = wave_max(kt);
  if (lane() == 0) atomicMax(&sh.bcast[6], kt);
}

// Zero the stage-2 counters.  Barriers follow inside every fill before any
// of them is updated.
template <class SH>
__device__ __forceinline__ void stage2_init(SH& sh, Stage2Lds& s2) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    s2.gmax_rank[tid] = 0;
    s2.surv_rank[tid] = 0;
  }
  if (tid == 0) {
    sh.bcast[1] = kI32Min;  // largest block maximum
    sh.bcast[2] = 0;        // survivors
    sh.bcast[5] = 0;        // flagged blocks
    sh.bcast[6] = kI32Min;  // T2b
    sh.bcast[7] = 0;        // flagged lists read past their prefix
  }
}

// (2) and (3), after a fill: the certified bound T2 and the survivors.
// `all_in_lds`: the candidates were copied to s2.cand (contiguous lists,
// stride == per).
template <class SH>
__device__ __forceinline__ Stage2Bound stage2_bound(const CandView& cv, int G,
                                                    int k, bool all_in_lds,
                                                    SH& sh, Stage2Lds& s2) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int per = cv.per;

  // (2) Group maxima into s2.gmax.  k <= 32: wave 0 forms 64 groups, lane
  // l taking blocks l*per .. l*per + per - 1 (per = G/64 rounded up to a
  // multiple of 4, read as 16-byte LDS loads).  Otherwise every thread
  // forms one group of G/256 (rounded up) blocks.  Empty groups hold
  // INT_MIN, which certifies nothing beyond the trivial bound.  (The k-th
  // largest of only 64 group maxima is a weak bound once k nears 64: at
  // k = 64 it is the smallest of them, and top-64 of 1e8 took 82.3 us
  // with it against 74.5 us with 256 groups.)
  const bool narrow = k <= kWave / 2;
  int gm = kI32Min;
  if (narrow) {
    if (w == 0) {
      constexpr int VH = kMaxGrid / kWave;
      const int gper = (((G + kWave - 1) / kWave) + 3) & ~3;
      const v4i* h4 = reinterpret_cast<const v4i*>(s2.heads + lane() * gper);
#pragma unroll
      for (int q = 0; q < VH / 4; ++q) {
        if (4 * q < gper) {
          const v4i t = h4[q];
          const int b = lane() * gper + 4 * q;
          gm = max(gm, b < G ? t.x : kI32Min);
          gm = max(gm, b + 1 < G ? t.y : kI32Min);
          gm = max(gm, b + 2 < G ? t.z : kI32Min);
          gm = max(gm, b + 3 < G ? t.w : kI32Min);
        }
      }
      s2.gmax[lane()] = gm;
    }
  } else {
    const int gper = (G + kBlock - 1) / kBlock;
    for (int j = 0; j < gper; ++j) {
      const int b = tid * gper + j;
      if (b < G) gm = max(gm, s2.heads[b]);
    }
    s2.gmax[tid] = gm;
  }
  gm = wave_max(gm);
  if (lane() == 0 && gm > kI32Min) atomicMax(&sh.bcast[1], gm);
  __syncthreads();
  if (narrow) {
    const int gv = block_rank64(s2.gmax, kWave, s2.gmax_rank);
    if (tid < kWave && s2.gmax_rank[tid] == k - 1) sh.bcast[0] = gv;
  } else if (w == 0) {
    // 256 group maxima, 4 per lane: a lower bound on the k-th largest,
    // within 1/256 of its range (certified all the same; see
    // radix_lower_bound).  The range starts at the smallest maximum of a
    // group that has blocks, which at least ng >= k group maxima reach (the
    // search's precondition): the INT_MIN of an empty group (fewer than
    // 256 blocks) would stretch it over all 2^32 values, and the bound
    // would then admit a large share of all candidates (top-100 of 1e6
    // took 204 us with 244 blocks so, 11 us without).  With fewer than k
    // groups nothing but INT_MIN is certified.
    const int gper = (G + kBlock - 1) / kBlock;
    const int ng = (G + gper - 1) / gper;  // groups that have blocks
    unsigned u[kWaves];
    int lo = kI32Max;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) {
      const int x = s2.gmax[lane() + kWave * j];
      u[j] = bias(x);
      if (lane() + kWave * j < ng) lo = min(lo, x);
    }
    if (ng < k) lo = kI32Min;
    const unsigned t = radix_lower_bound(bias(wave_min(lo)),
                                         bias(sh.bcast[1]), k, 8,
                                         RegCount<kWaves>{u});
    if (lane() == 0) sh.bcast[0] = unbias(t);
  }
  __syncthreads();
  if (G < k && (k + G - 1) / G <= per) {
    // Fewer lists than k: their maxima certify nothing.  The first
    // j = ceil(k / G) entries of every list are G j >= k candidates, so
    // the k-th largest of them is a lower bound on the result's k-th (top-
    // 128 of 5e5 over 122 blocks took 183 us with no bound, top-100 of 2e5
    // over 48 blocks 100 us).  G j < G + k < 2 kMaxK = kBlock values, one
    // per thread, ranked in s2.gmax (free by now).
    const int j = (k + G - 1) / G;
    const int cnt = G * j;
    if (tid < cnt) {
      const int b = tid / j, e = tid - b * j;
      s2.gmax[tid] = all_in_lds
                         ? s2.cand[b * per + e]
                         : ld_agent(cv.cand + (int64_t)b * cv.stride + e);
    }
    int v;
    const int rk = rank_all(s2.gmax, cnt, v);
    if (tid < cnt && rk == k - 1) sh.bcast[0] = max(sh.bcast[0], v);
    __syncthreads();
  }
  Stage2Bound r;
  r.t2 = max(sh.bcast[0], sh.bcast[6]);
  r.mx = sh.bcast[1];
  r.m = 0;
  r.total = 0;

  // (3) The blocks whose maximum reaches T2.
  for (int b0 = 0; b0 < G; b0 += kBlock) {
    const int b = b0 + tid;
    const bool f = b < G && s2.heads[b] >= r.t2;
    wave_append(f, b, &sh.bcast[5], s2.blocks, kMaxGrid);
  }
  __syncthreads();
  r.total = sh.bcast[5] * per;
  if (r.t2 == r.mx) return r;  // the caller writes k copies of mx

  // Survivors.  Candidates equal to INT_MIN are left out: if T2 is INT_MIN
  // and fewer than k candidates exceed it, the result is padded with
  // INT_MIN, which is the same.
  const int tf = r.t2 == kI32Min ? kI32Min + 1 : r.t2;
  if (all_in_lds) {
    // Every list is descending, so its survivors are a prefix of it: thread
    // i walks flagged list i while its entries reach T2 (a wave as long as
    // its longest prefix, about two entries).  Scanning whole lists took
    // ceil(flagged * k / 256) rounds (top-64 of 1e7: 18 rounds, 3.6 us).
    const int nflag = sh.bcast[5];
    for (int l0 = 0; l0 < nflag; l0 += kBlock) {
      const int l = l0 + tid;
      const int* lst = s2.cand + (l < nflag ? s2.blocks[l] : 0) * per;
      bool more = l < nflag;
      for (int e = 0; ballot(more); ++e) {
        const int v = more ? lst[e] : kI32Min;
        const bool s = more && v >= tf;
        wave_append(s, v, &sh.bcast[2], s2.surv, kSurvCap);
        more = s && e + 1 < per;
      }
    }
  } else {
    // Every list is descending, so its survivors are a prefix of it.  The
    // first kPrefix entries of all flagged lists take one pass (one round
    // trip to memory for up to kMaxGrid lists); the rest of a list is read
    // only when its last entry read still reaches T2, which is rare (about
    // one survivor per flagged list is usual).  Reading whole lists took
    // (G' * k) / (16 * kBlock) dependent round trips for G' flagged lists.
    // Those lists go to s2.cand, unused on this path.
    const int pf = min(kPrefix, per);
    const int nflag = sh.bcast[5];
    scan_flagged_at(CandView{cv.cand, cv.stride, pf}, s2.blocks, nflag * pf,
                    [&](bool ok, int c, int b, int e)
                        __attribute__((always_inline)) {
                          const bool s = ok && c >= tf;
                          wave_append(s, c, &sh.bcast[2], s2.surv, kSurvCap);
                          wave_append(s && e == pf - 1 && per > pf, b,
                                      &sh.bcast[7], s2.cand, kDirectCand);
                        });
    __syncthreads();
    const int nlong = sh.bcast[7];
    if (nlong > 0) {
      scan_flagged(CandView{cv.cand + pf, cv.stride, per - pf}, s2.cand,
                   nlong * (per - pf), [&](bool ok, int c) {
                     wave_append(ok && c >= tf, c, &sh.bcast[2], s2.surv,
                                 kSurvCap);
                   });
    }
  }
  __syncthreads();
  r.m = sh.bcast[2];
  return r;
}

// Stage 2 proper, after stage2_init, a fill and stage2_bound: rank or
// select, and write the k results to out (agent-coherent stores, so that
// another workgroup of the same launch may read them).
template <class SH>
__device__ __forceinline__ void stage2_finish(const CandView& cv, int k,
                                              const Stage2Bound& r, int* out,
                                              SH& sh, Stage2Lds& s2) {
  const int w = threadIdx.x / kWave;
  const int tid = threadIdx.x;
  const int T2 = r.t2, mx = r.mx, m = r.m, total = r.total;

  if (T2 == mx) {
    // At least k candidates are >= T2 and none exceeds mx: k copies of mx.
    for (int j = tid; j < k; j += kBlock) st_agent(out + j, mx);
    return;
  }

  // Few survivors (the usual case): each is ranked by counting, so the
  // result comes out in order with no selection step.  Equal values get
  // consecutive ranks.  If T2 was INT_MIN, fewer than k may have survived:
  // the rest of the result is INT_MIN.
  if (m <= kBlock) {
    int v, rk = kBlock;
    if (m <= kWave) {
      v = block_rank64(s2.surv, m, s2.surv_rank);
      if (tid < m) rk = s2.surv_rank[tid];
    } else {
      rk = rank_all(s2.surv, m, v);
    }
    if (tid < m && rk < k) st_agent(out + rk, v);
    for (int j = m + tid; j < k; j += kBlock) st_agent(out + j, kI32Min);
    return;
  }

  // Many survivors (heavy ties near the top): select g, the k-th largest
  // survivor (there are >= k: T2 is certified), by counting.
  const bool in_lds = m <= kSurvCap;
  if (tid == 0) sh.bcast[3] = 0;  // count of values above g
  unsigned g;
  if (m <= 8 * kWave) {
    if (w == 0) {
      unsigned u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = lane() + kWave * j;
        u[j] = q < m ? bias(s2.surv[q]) : 0u;
      }
      g = radix_select(bias(T2), bias(mx), k, RegCount<8>{u});
      if (lane() == 0) sh.bcast[4] = (int)g;
    }
    __syncthreads();
    g = (unsigned)sh.bcast[4];
  } else {
    int parity = 0;
    auto count_ge = [&](unsigned c) __attribute__((always_inline)) -> int {
      const int s = unbias(c);
      int mine = 0;
      if (in_lds) {
        for (int i = tid; i < m; i += kBlock) mine += s2.surv[i] >= s;
      } else {
        scan_flagged(cv, s2.blocks, total, [&](bool ok, int v) {
          mine += ok & (v >= s) & (v >= T2);
        });
      }
      return block_sum(mine, sh, parity);
    };
    g = radix_select(bias(T2), bias(mx), k, count_ge);
  }
  const int gs = unbias(g);

  // Values above g (fewer than k), ranked; then copies of g.
  if (in_lds) {
    for (int base = 0; base < m; base += kBlock) {
      const int i = base + tid;
      const int c = i < m ? s2.surv[i] : kI32Min;
      wave_append(i < m && c > gs, c, &sh.bcast[3], s2.gt, kMaxK);
    }
  } else {
    scan_flagged(cv, s2.blocks, total, [&](bool ok, int c) {
      wave_append(ok && c > gs, c, &sh.bcast[3], s2.gt, kMaxK);
    });
  }
  __syncthreads();
  const int ngt = sh.bcast[3];
  if (tid < ngt) {
    const int v = s2.gt[tid];
    int rk = 0;
    for (int j = 0; j < ngt; ++j) {
      const int o = s2.gt[j];
      rk += (o > v) | ((o == v) & (j < tid));
    }
    st_agent(out + rk, v);
  } else if (tid < k) {
    st_agent(out + tid, gs);
  }
}

// Stage 2 of the top-k kernel for one row: merge the row's grid * k block
// candidates into out[0..k).
template <class SH>
__device__ __forceinline__ void topk_stage2(const TopkParams& p, SH& sh,
                                            Stage2Lds& s2) {
  const int G = p.grid, k = p.k;
  const bool all_in_lds = (int64_t)G * k <= kDirectCand;
  const CandView cv{p.cand, k, k};
  stage2_init(sh, s2);
  stage2_fill_blocks(p.heads, p.kths, p.cand, G, G * k, all_in_lds, sh, s2);
  const Stage2Bound r = stage2_bound(cv, G, k, all_in_lds, sh, s2);
  stage2_finish(cv, k, r, p.out, sh, s2);
}

// Short lists (FIT false: KCAP < k).  A lane keeps its KCAP largest values,
// so a value of the workgroup's top-k is dropped when one lane meets more
// than KCAP values above the workgroup's k-th largest.  Every value a lane
// drops is at most the largest value it evicted, `lost` (a value skipped by
// the lane threshold is below the evicted value that raised it, or below
// the certified bound).  Equal values are interchangeable here, so if no
// lane evicted a value above the result's k-th value (sh.kth), the lists
// held every value above it and the result stands: the common case, at the
// cost of one block maximum.  Otherwise the workgroup's top-k is found
// again, exactly, by counting over its elements read back from memory
// (radix selection of the k-th largest g from the lists' k-th value up,
// then the values above g ranked and copies of g): slow, and only for
// inputs where one lane meets more than KCAP of its workgroup's top-k.
// Barriers inside: call uniformly, after the result has been written.
template <int KCAP, int U, class SH>
__device__ __forceinline__ void short_list_check(
    const int* __restrict__ rin, int64_t n, int blk, int grid, int k,
    int lost, int head, int* dst, int* head_out, int* kth_out, SH& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh.bcast[2] = kI32Min;
    sh.bcast[3] = kI32Min;
  }
  __syncthreads();  // also publishes sh.kth
  const int wl = wave_max(lost);
  const int wh = wave_max(head);
  if (lane() == 0) {
    atomicMax(&sh.bcast[2], wl);
    atomicMax(&sh.bcast[3], wh);
  }
  __syncthreads();
  const int gl = sh.kth, worst = sh.bcast[2], mx = sh.bcast[3];
  if (worst <= gl) return;

  // Every element of the workgroup, each thread visiting the same number
  // of times (lanes past the end visit INT_MIN, which counts for nothing
  // above the lists' k-th value).
  const RowGeometry geo = row_geometry<U>(rin, n);
  auto visit = [&](auto&& f) __attribute__((always_inline)) {
    const v4i* __restrict__ body = reinterpret_cast<const v4i*>(rin + geo.head);
    const int64_t count = tiles_of(geo.ntiles, blk, grid);
    for (int64_t i = 0; i < count; ++i) {
      const v4i* src = body + (blk + i * grid) * (int64_t)(kBlock * U);
      v4i d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = src[u * kBlock + tid];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f(d[u].x);
        f(d[u].y);
        f(d[u].z);
        f(d[u].w);
      }
    }
    if (blk == grid - 1) {
      const int64_t left = n - geo.covered;
      for (int64_t base = 0; base < left; base += kBlock) {
        const int64_t i = base + tid;
        f(i < left ? rin[i < geo.head ? i : geo.covered + i] : kI32Min);
      }
    }
  };
  int parity = 0;
  auto count_ge = [&](unsigned c) __attribute__((always_inline)) -> int {
    const int t = unbias(c);
    int m = 0;
    visit([&](int x) { m += x >= t; });
    return block_sum(m, sh, parity);
  };
  // The true k-th largest is >= the lists' (they hold a subset of the
  // elements), and no element exceeds the largest head (a lane's maximum
  // is never evicted).
  const int g = unbias(radix_select(bias(gl), bias(mx), k, count_ge));
  __syncthreads();
  if (tid == 0) sh.bcast[0] = 0;
  __syncthreads();
  visit([&](int x) { wave_append(x > g, x, &sh.bcast[0], sh.blist, kBlock); });
  __syncthreads();
  const int ngt = sh.bcast[0];  // < k
  int v;
  const int rk = rank_all(sh.blist, ngt, v);
  if (tid < ngt) st_agent(dst + rk, v);
  for (int j = ngt + tid; j < k; j += kBlock) st_agent(dst + j, g);
  if (head_out && tid == 0) {
    st_agent(head_out, mx);
    st_agent(kth_out, g);
  }
}

// The k largest of the elements that workgroup `blk` of `grid` owns in one
// row (rin[0..n): its round-robin tiles, and the head and the tail when it
// is the row's last workgroup), written in descending order to dst[0..k)
// with agent-coherent stores; with head_out, also its largest and k-th
// value (for a stage 2 to come).  Stage 1 and the block step of the
// two-stage design ([TopK] §2.1).  Barriers inside: call uniformly.  The
// caller's LDS (sh, ring_lds) must be free: on entry no thread may still
// read what an earlier call left there.
template <int KCAP, bool FIT, int U>
__device__ __forceinline__ void workgroup_topk(
    const int* __restrict__ rin, int64_t n, int blk, int grid, int k, int R,
    int* dst, int* head_out, int* kth_out, TopkShared<KCAP>& sh,
    v4i (&ring_lds)[kWaves][kRing][U][kWave]) {
  const RowGeometry geo = row_geometry<U>(rin, n);
  const int w = threadIdx.x / kWave;

  int L[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; ++i) L[i] = kI32Min;
  int tsh = kI32Min;  // this wave's certified bound
  int thr = kI32Min;  // this lane's test: max(its list's last entry, tsh)
  int lost = kI32Min;  // short lists: the largest value this lane evicted
  static_assert(FIT || KCAP >= 4 * U, "the first tile fits a short list");
  sh.heads[threadIdx.x] = 0u;  // biased INT_MIN: the weakest valid head
  if (threadIdx.x == 0) sh.bcnt = 0;
  if (threadIdx.x < kWave) sh.ranks[threadIdx.x] = 0;
  __syncthreads();

  // ---- stage 1: stream this workgroup's tiles ---------------------------
  // Tiles are dealt round-robin (tile blk, blk+grid, ...), so at any moment
  // the grid reads one compact window of HBM.  Each wave streams its
  // quarter of every tile straight into its own LDS ring (global_load_lds,
  // 16 B per lane, no VGPRs), kRing tiles ahead of the one it examines, so
  // the time spent inserting never leaves the memory pipe empty.
  const v4i* __restrict__ body = reinterpret_cast<const v4i*>(rin + geo.head);
  const int64_t count = tiles_of(geo.ntiles, blk, grid);
  if (count > 0) {
    v4i(*ring)[U][kWave] = ring_lds[w];
    // Byte offsets of this lane's loads within a tile, and the byte
    // distance between consecutive tiles of this workgroup.
    uint32_t voff[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      voff[u] = (uint32_t)((u * kBlock + threadIdx.x) * sizeof(v4i));
    const char* first = reinterpret_cast<const char*>(body) +
                        (int64_t)blk * kTileBytes<U>;
    const int64_t stride = (int64_t)grid * kTileBytes<U>;
    // The workgroup's last tile is examined first, then the others in
    // order (see tile_order): on ascending input the lists then start from
    // the largest values and the bound rejects nearly everything after.
    auto tile = [&](int64_t i) __attribute__((always_inline)) {
      return first + tile_order(i, count) * stride;
    };
#pragma unroll
    for (int j = 0; j < kRing; ++j)
      if (j < count) issue_tile_lds<U>(tile(j), voff, ring[j]);
    for (int64_t i = 0; i < count; ++i) {
      // Steady state: the kRing - 1 tiles after this one stay in flight.
      wait_tile_loads<U, kRing>(i + kRing - 1 < count);
      const int slot = (int)(i & (kRing - 1));
      v4i d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = ring[slot][u][lane()];
      wait_lds_reads();  // the slot is free once its data is in registers
      if (i + kRing < count)
        issue_tile_lds<U>(tile(i + kRing), voff, ring[slot]);
      if (i == 0)
        init_list<KCAP, U>(L, d, thr);
      else
        consume<KCAP, FIT, U>(L, d, k, tsh, thr, lost);
      // After each of the first two tiles every lane publishes its head and
      // the workgroup waits, so that bound refresh sees all 256 fresh
      // heads: the early bounds are much tighter and far fewer elements are
      // admitted in the tiles that follow.
      if (i <= 1) {
        __hip_atomic_store(&sh.heads[threadIdx.x], bias(L[0]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
        lds_barrier();
      }
      if (refresh_due(i, R)) refresh_bound(L, k, tsh, thr, sh);
      // Workgroups blk and blk + grid/2 usually share a CU (the grid fills
      // every CU once before the second round), and the hardware favours
      // the older one: on top-20 of 1e8 the first half finished streaming
      // 10 us before the second (46 against 56 us, median).  Raising each
      // half's priority in turn, in slots of 5.12 us, evened them (53 and
      // 56 us) and took 0.5-1 us off the call.
      if ((((unsigned)(__builtin_amdgcn_s_memrealtime() >> 9)) +
           (blk >= (grid >> 1) ? 1u : 0u)) & 1u)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
  }
  // Elements outside the full tiles: the unaligned head and the tail.
  if (blk == grid - 1) {
    visit_rest<kBlock * U * 4>(rin, n, geo.head, geo.covered,
                               [&](int x, int64_t, bool)
                                   __attribute__((always_inline)) {
                                     admit<KCAP, FIT>(L, x, k, tsh, thr, lost);
                                   });
  }
  // One more refresh of this wave's bound from the lane-head snapshot (no
  // barrier: the bound is certified whatever the other waves are doing).
  refresh_bound(L, k, tsh, thr, sh);
  const int T = tsh;  // certified for the workgroup; may differ per wave

  // ---- block candidates: the workgroup's exact top-k ---------------------
  // The entries >= T among the first k of every list include the
  // workgroup's top-k (T is at most its k-th largest value, and no list
  // entry past position k can be among them), and there are at least k of
  // them.  Usually they are few (about k): they are gathered in LDS and
  // each thread ranks one by counting, which writes the top-k in
  // descending order.  With heavy ties there can be more than fit; then
  // the waves select instead.
  {
    // Level by level while some lane reaches T, and only until the LDS
    // list has overflowed (the count keeps growing past kBlock then, which
    // is all the fallback needs to know).
    bool more = true;  // wave-uniform
#pragma unroll
    for (int i = 0; i < KCAP; ++i) {
      if (more) {
        const bool q = i < k && L[i] >= T;
        const uint64_t b = ballot(q);
        more = b != 0;
        if (more) {
          int base = 0;
          if (lane() == 0) base = atomicAdd(&sh.bcnt, popc(b));
          base = uni(base);
          const int pos = base + lanes_below(b);
          if (q && pos < kBlock) sh.blist[pos] = L[i];
          // Stop once the list has overflowed (the count then exceeds
          // kBlock, which sends the workgroup to the fallback).  A list
          // filled exactly to kBlock must go on: a deeper level may hold
          // more entries, and stopping would leave the count looking
          // complete.
          more = base + popc(b) <= kBlock;
        }
      }
    }
  }
  __syncthreads();
  const int lb = sh.bcnt;
  if (lb <= kWave) {
    // The usual case: at most 64 entries, sorted across wave 0's lanes (a
    // register bitonic network), lanes 0..k-1 write them in order.
    if (w == 0) {
      const int v = wave_sort_desc<kWave>(lane() < lb ? sh.blist[lane()]
                                                      : kI32Min);
      if (lane() < k) st_agent(dst + lane(), v);
      if (head_out && lane() == 0) st_agent(head_out, v);
      if (head_out && lane() == k - 1) st_agent(kth_out, v);
      if (lane() == k - 1) sh.kth = v;
    }
  } else if (lb <= kBlock) {
    int v;
    const int rk = rank_all(sh.blist, lb, v);
    if ((int)threadIdx.x < lb && rk < k) {
      st_agent(dst + rk, v);
      if (head_out && rk == 0) st_agent(head_out, v);
      if (head_out && rk == k - 1) st_agent(kth_out, v);
      if (rk == k - 1) sh.kth = v;
    }
  } else {
    // Wave merge: each wave's top-k of its entries >= T.
    {
      const int live = list_count_ge<KCAP>(L, k, T);
      int cnt;
      if (live <= k) {
        list_emit<KCAP>(L, k, T, false, sh.wave_out[w], kMaxK);
        cnt = live;
      } else {
        const int hi = wave_max(L[0]);
        const unsigned g =
            radix_select(bias(T), bias(hi), k, ListCount<KCAP>{L, k});
        const int gs = unbias(g);
        const int above =
            list_emit<KCAP>(L, k, gs, true, sh.wave_out[w], kMaxK);
        for (int j = lane(); j < k - above; j += kWave)
          sh.wave_out[w][above + j] = gs;
        cnt = k;
      }
      if (lane() == 0) sh.wave_cnt[w] = cnt;
    }
    __syncthreads();

    // Block merge (wave 0): top-k of the four wave results.  T of wave 0 is
    // a valid lower end for the search: the workgroup's k-th largest value
    // is >= it, and each wave result holds that wave's share of the top-k.
    // The values above the k-th (fewer than k) go to LDS, where the whole
    // workgroup ranks them, so the candidates come out in order here too.
    if (w == 0) {
      constexpr int WO = kMaxK;  // wave_out's row
      constexpr int V = (kWaves * WO + kWave - 1) / kWave;
      unsigned u[V];
      int mx = kI32Min;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int q = lane() + kWave * j;
        const int ww = q / WO, o = q % WO;
        const int v = (ww < kWaves && o < sh.wave_cnt[ww < kWaves ? ww : 0])
                          ? sh.wave_out[ww][o]
                          : kI32Min;
        u[j] = bias(v);
        mx = max(mx, v);
      }
      mx = wave_max(mx);
      const unsigned g = radix_select(bias(T), bias(mx), k, RegCount<V>{u});
      int base = 0;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const bool q = u[j] > g;
        const uint64_t b = ballot(q);
        if (q) sh.blist[base + lanes_below(b)] = unbias(u[j]);
        base += popc(b);
      }
      if (lane() == 0) {
        sh.bcast[0] = base;
        sh.bcast[1] = unbias(g);
        sh.kth = unbias(g);
        if (head_out) {
          st_agent(head_out, mx);
          st_agent(kth_out, unbias(g));
        }
      }
    }
    __syncthreads();
    const int ngt = sh.bcast[0], gv = sh.bcast[1];
    int v;
    const int rk = rank_all(sh.blist, ngt, v);  // ngt < k <= kBlock
    if ((int)threadIdx.x < ngt) st_agent(dst + rk, v);
    for (int j = ngt + (int)threadIdx.x; j < k; j += kBlock)
      st_agent(dst + j, gv);
  }
  if constexpr (!FIT)
    short_list_check<KCAP, U>(rin, n, blk, grid, k, lost, L[0], dst,
                              head_out, kth_out, sh);
}

template <int KCAP, bool FIT, int U>
__global__ __launch_bounds__(kBlock) void topk_kernel(TopkParams p) {
  __shared__ TopkShared<KCAP> sh;
  // Each wave's ring of kRing tiles (its quarter of each tile).  A separate
  // LDS object from `sh`, so that the compiler can tell LDS accesses to
  // `sh` apart from the in-flight ring loads and does not wait for those.
  __shared__ v4i ring_lds[kWaves][kRing][U][kWave];
  static_assert(sizeof(ring_lds) >= sizeof(Stage2Lds), "ring too small");
  // This workgroup's row, and its place among the row's workgroups.
  const int row = (int)(blockIdx.x / (unsigned)p.grid);
  const int blk = (int)blockIdx.x - row * p.grid;
  const int* __restrict__ rin = p.in + (int64_t)row * p.ld;
  const int64_t slot0 = (int64_t)row * p.grid;  // the row's first block slot
  const int k = p.k;
  // A row with one workgroup: its top-k is the row's result.
  const bool direct = p.grid == 1;
  int* dst = direct ? p.out + (int64_t)row * k : p.cand + (slot0 + blk) * k;
  workgroup_topk<KCAP, FIT, U>(rin, p.n, blk, p.grid, k, p.refresh, dst,
                               direct ? nullptr : p.heads + slot0 + blk,
                               direct ? nullptr : p.kths + slot0 + blk, sh,
                               ring_lds);

  // ---- hand-off: the last workgroup to finish runs stage 2 --------------
  if (direct) return;
  if (!last_to_finish(p.ticket + row, p.grid, p.epoch, &sh.is_last)) return;
  TopkParams q = p;  // the row's slice of the scratch and of the output
  q.cand = p.cand + slot0 * k;
  q.heads = p.heads + slot0;
  q.kths = p.kths + slot0;
  q.ticket = p.ticket + row;
  q.out = p.out + (int64_t)row * k;
  topk_stage2(q, sh, *reinterpret_cast<Stage2Lds*>(&ring_lds[0][0][0][0]));
}

// ---- merging descending lists ---------------------------------------------
// The k largest values of the union of m descending lists of `len` values
// each ([TopK] §6: several top-k results merged again; it is exactly the
// page's stage 2, §2.2, applied to lists the caller provides).  Only the
// first min(len, k) entries of a list can be among the k largest, each
// list's first entry is its maximum and a list of at least k entries
// certifies its k-th, so the stage-2 machinery above applies as is.  One
// workgroup merges up to kMaxGrid lists; more lists are cut into groups of
// kMaxGrid, each group's top-k goes to scratch, and the last group to
// finish merges those (the same hand-off as the top-k kernel).
struct MergeParams {
  const int* lists;  // list b at lists + b * len, descending
  int64_t m;         // lists
  int len;           // entries per list
  int k;
  int groups;        // workgroups, each merging up to kMaxGrid lists
  int* cand;         // [groups * k] group results (groups > 1)
  uint64_t* ticket;  // completion counter (groups > 1; see Tagged)
  uint32_t epoch;    // this launch's
  int* out;          // [k]
};

struct MergeShared {
  int red[2][kWaves];
  int bcast[8];
  int is_last;
};

__global__ __launch_bounds__(kBlock) void topk_merge_kernel(MergeParams p) {
  __shared__ MergeShared sh;
  __shared__ Stage2Lds s2;
  const int g = blockIdx.x;
  const int64_t first = (int64_t)g * kMaxGrid;
  const int nl = (int)min((int64_t)kMaxGrid, p.m - first);
  const int k = p.k;
  const CandView cv{p.lists + first * p.len, p.len, min(p.len, k)};
  int* dst = p.groups == 1 ? p.out : p.cand + (int64_t)g * k;
  stage2_init(sh, s2);
  stage2_fill_lists(cv, nl, k, sh, s2);
  const Stage2Bound r = stage2_bound(cv, nl, k, false, sh, s2);
  stage2_finish(cv, k, r, dst, sh, s2);
  if (p.groups == 1) return;

  if (!last_to_finish(p.ticket, p.groups, p.epoch, &sh.is_last)) return;
  const CandView cg{p.cand, k, k};
  stage2_init(sh, s2);
  stage2_fill_lists(cg, p.groups, k, sh, s2);
  const Stage2Bound r2 = stage2_bound(cg, p.groups, k, false, sh, s2);
  stage2_finish(cg, k, r2, p.out, sh, s2);
}

}  // namespace ltk
