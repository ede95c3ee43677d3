// Top-k for large k (up to 16384) by radix selection, built on the
// histogram machinery of hist_kernel.hpp.
//
// Sources:
//   [Radix] "GPU基数排序优化：10亿级数据处理与性能调优" §3.2 (8-bit digits,
//           four passes for 32-bit keys) and §3.3 (one shared-memory
//           histogram per warp, merged at the end).
//   [TopK]  "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计" §2 (the
//           output: the k largest, descending, duplicates kept).
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
// orders the k values in LDS (placed by a digit, or sorted).
//
// Large inputs first try a shortcut: a sample fixes a threshold t (the
// value of a small rank in an evenly spaced sample), one filter pass
// copies the values above t aside and counts those equal to t, and when
// that copy is small one workgroup selects the top-k from it in LDS
// (select_finish_kernel); the digit passes then return at once.  When the
// copy is too large, or cannot hold the top-k, the digit passes run as
// above, so the sample affects the time only.
#pragma once

#include "hist_kernel.hpp"

namespace ltk {

constexpr int kMaxKSelect = 16384; // largest k of the radix-select path

constexpr int kCandCap = 1 << 22;  // candidate buffer, elements
// Candidates one workgroup selects from after the filter pass; larger
// copies go through the multi-workgroup selection passes.
constexpr int kFinishMax = 1 << 20;

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
  int thresh;       // sampled threshold of the filter pass
  int fast;         // the filter's copy is small: one workgroup finishes
  unsigned eqcount; // values equal to the threshold (filter pass)
};

// One digit pass of radix selection, or the gather.
struct SelectParams {
  const int* in;
  int64_t n, head, ntiles, covered;
  int grid;
  int dshift;   // the digit's lowest bit
  int first;    // the first pass: start from an empty prefix, kleft = k
  int k;
  RadixState* st;
  int* cand;    // [kCandCap] candidate buffer
  int* out;     // [k]
  uint64_t* acc;            // [256] epoch-tagged device counters
  uint64_t* ticket;
  uint32_t epoch;           // this launch's (see Tagged)
};

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
    // Selection already finished, or left to the finish kernel.
    if (s.done || s.fast) return;
  }
  const bool split = s.split && s.src == 0;
  const int grid = pass_grid<U>(p, s);
  if ((int)blockIdx.x >= grid) return;
  for (int i = threadIdx.x; i < kWaves * kDigitBins; i += kBlock) h[i] = 0u;
  __syncthreads();
  unsigned* hw = h + w * kDigitBins;
  const unsigned prefix = s.prefix, mask = s.mask;
  const unsigned dshift = (unsigned)p.dshift;

  Stager stg{stage[w], 0, &p.st->ccount, p.cand, (unsigned)kCandCap};
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
  if (split) stg.flush();
  __syncthreads();
  for (int b = threadIdx.x; b < kDigitBins; b += kBlock) {
    unsigned c = h[b];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) c += h[j * kDigitBins + b];
    acc_add(p.acc, kDigitBins, b, c, p.epoch);
  }

  if (!last_to_finish(p.ticket, grid, p.epoch, &is_last)) return;

  // Pick the digit holding the k-th largest: thread t looks at bin 255 - t,
  // so an inclusive prefix sum over threads is the count of the bucket's
  // elements at or above that bin.  Counts are capped at kCandCap, which
  // keeps the sums in 32 bits and leaves every comparison with kleft
  // (<= 16384) unchanged: the first bin whose capped sum reaches kleft is
  // reached by exact counts.
  const int t = threadIdx.x;
  const int b = kDigitBins - 1 - t;
  const uint64_t raw = acc_take(p.acc, kDigitBins, b, p.epoch);
  const int c = raw > (uint64_t)kCandCap ? kCandCap : (int)raw;
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
      p.st->fast = 0;
    }
  }
}

// The filter threshold for top-k with large n.  `grid` workgroups read
// grid * 1024 16-byte vectors spread evenly over the input (one per
// thread); t is to be the value of rank `need` among the S = grid * 4096
// sampled values (`need` is k scaled to the sample, with a wide margin).
// Each workgroup publishes a list that holds its `need` largest samples
// (usually every sample in the top-digit bins from its rank-`need` one up);
// the last workgroup finds the value of rank `need` in the union of those
// lists, which is that of the whole sample, exactly, with block_rank: four
// 8-bit digit levels of LDS histograms ([Radix] §3.2's digits).  The filter pass then copies every value above t
// aside and counts those equal to it: when at least k values are >= t,
// the top-k lies among them, whatever t is, so a poor sample costs time,
// never correctness.
constexpr int kSampleThreads = 1024;
constexpr int kSampleGridMax = 64;  // workgroups (S = 4096 values each)
constexpr int kNeedMax = 256;       // largest `need`
constexpr int kUnionSlots = 4 * kSampleThreads;  // grid * need <= this
struct SampleParams {
  const v4i* body;   // the 16-byte-aligned body of the input
  int64_t nvec;      // vectors in it
  uint64_t step;     // vectors between consecutive samples, 32.32 fixed
                     // point: sample i reads vector (i * step) >> 32
  int grid;          // workgroups, <= kSampleGridMax
  int need;          // 1 <= need <= kNeedMax, grid * need <= kUnionSlots
  RadixState* st;
  int* samp;         // [kSampleGridMax * kNeedMax] the published lists
  int* samp_cnt;     // [kSampleGridMax] their lengths
  uint64_t* ticket;
  uint32_t epoch;    // this launch's (see Tagged)
};

struct RankShared {
  unsigned h[kDigitBins];
  int scan[kSampleThreads / kWave];
  int pick[3];  // bin, count above it, count in it
  int cnt;
  int is_last;
};

// The highest of 256 bins (one LDS copy, h[0..256)) whose suffix count
// reaches `need` (bin 0 if none does), the count above it and the count in
// it, into sh.pick; threads t < 256 look at bin 255 - t.  Clears h.
__device__ __forceinline__ void pick256(RankShared& sh, int need) {
  const int t = threadIdx.x, w = t / kWave;
  const int b = kDigitBins - 1 - t;
  int c = 0, incl_w = 0;
  if (t < kDigitBins) {
    c = (int)sh.h[b];
    incl_w = wave_scan_incl(c);
    if (lane() == kWave - 1) sh.scan[w] = incl_w;
  }
  __syncthreads();
  if (t < kDigitBins) {
    int incl = incl_w;
#pragma unroll
    for (int j = 0; j < kDigitBins / kWave; ++j) incl += j < w ? sh.scan[j] : 0;
    const int above = incl - c;
    if ((incl >= need && above < need) || (b == 0 && incl < need)) {
      sh.pick[0] = b;
      sh.pick[1] = above;
      sh.pick[2] = c;
    }
    sh.h[b] = 0u;
  }
  __syncthreads();
}

// The biased value v of rank `need` (1 = the largest) among the PER values
// each thread of the workgroup holds (slot j only where bit j of `valid`
// is set), and in *above the number of values greater than v: four 8-bit
// digit levels, each an LDS histogram of the values whose higher digits
// equal those chosen so far.  There are at least `need` valid values.
// sh.h[0..256) is zero on entry and on return.
template <int PER>
__device__ __forceinline__ unsigned block_rank(const unsigned (&u)[PER],
                                               unsigned valid, int need,
                                               RankShared& sh, int* above) {
  unsigned prefix = 0u;
  int a = 0;
#pragma unroll
  for (int level = 0; level < 4; ++level) {
    const unsigned shift = 24u - 8u * level;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool in = (valid & (1u << j)) &&
                      (level == 0 || (u[j] >> (shift + 8u)) == (prefix >> (shift + 8u)));
      if (in) atomicAdd(&sh.h[(u[j] >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    pick256(sh, need - a);
    prefix |= (unsigned)sh.pick[0] << shift;
    a += sh.pick[1];
  }
  *above = a;
  return prefix;
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleParams p) {
  __shared__ RankShared sh;
  const int t = threadIdx.x;
  for (int i = t; i < kDigitBins; i += kSampleThreads) sh.h[i] = 0u;
  if (t == 0) sh.cnt = 0;
  unsigned u[4];
  {
    // Spread over the whole body: a whole-vector stride (nvec / S rounded
    // down) left up to S vectors at the end unread, the top of a sorted
    // input (top-1000 of 3e6 sorted values then copied 117,063 candidates
    // aside instead of about 1,700).
    const int64_t v = (int64_t)(
        ((uint64_t)blockIdx.x * kSampleThreads + (uint64_t)t) * p.step >> 32);
    // Vectors past the end (none: i < S gives v < nvec) count as
    // INT_MIN, never above a real threshold's rank.
    const v4i d = v < p.nvec ? __builtin_nontemporal_load(p.body + v)
                             : v4i{kI32Min, kI32Min, kI32Min, kI32Min};
    u[0] = bias(d.x);
    u[1] = bias(d.y);
    u[2] = bias(d.z);
    u[3] = bias(d.w);
  }
  __syncthreads();
  // This workgroup's list, at most cap = min(kUnionSlots / grid, kNeedMax)
  // (>= need) values that include its `need` largest: every sample in the
  // 8-bit bins (top digit) from the one holding its rank-`need` value up
  // (one histogram level), or, when more than cap share those bins,
  // exactly the `need` largest (all four levels).
  const int cap = min(kUnionSlots / p.grid, kNeedMax);
  int* mine = p.samp + blockIdx.x * kNeedMax;
#pragma unroll
  for (int j = 0; j < 4; ++j) atomicAdd(&sh.h[u[j] >> 24], 1u);
  __syncthreads();
  pick256(sh, p.need);
  const unsigned b1 = (unsigned)sh.pick[0];
  const int inb = sh.pick[1] + sh.pick[2];
  int len;
  // One LDS atomic per wave and slot places the appended values.
  auto publish = [&](bool q, unsigned x) __attribute__((always_inline)) {
    const uint64_t b = ballot(q);
    if (b == 0) return;
    int base = 0;
    if (lane() == 0) base = atomicAdd(&sh.cnt, popc(b));
    base = uni(base);
    const int pos = base + lanes_below(b);
    if (q && pos < cap) st_agent(mine + pos, (int)x);
  };
  if (inb <= cap) {
#pragma unroll
    for (int j = 0; j < 4; ++j) publish((u[j] >> 24) >= b1, u[j]);
    len = inb;
  } else {
    int a;
    const unsigned v = block_rank<4>(u, 0xfu, p.need, sh, &a);
#pragma unroll
    for (int j = 0; j < 4; ++j) publish(u[j] > v, u[j]);
    for (int i = a + t; i < p.need; i += kSampleThreads)
      st_agent(mine + i, (int)v);
    len = p.need;
  }
  if (t == 0) st_agent(p.samp_cnt + blockIdx.x, len);
  if (!last_to_finish(p.ticket, p.grid, p.epoch, &sh.is_last)) return;

  // The union of the lists: slot i is entry i % cap of list i / cap.
  // Every slot's value and its list's length are loaded together (slots
  // past a list's length hold stale values and are masked out).
  unsigned w[4], valid = 0;
  int len_of[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = j * kSampleThreads + t;
    const int g = min(i / cap, p.grid - 1), r = i - (i / cap) * cap;
    w[j] = (unsigned)ld_agent(p.samp + g * kNeedMax + r);
    len_of[j] = ld_agent(p.samp_cnt + g);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = j * kSampleThreads + t;
    if (i / cap < p.grid && i - (i / cap) * cap < len_of[j]) valid |= 1u << j;
  }
  int a2;
  const unsigned tv = block_rank<4>(w, valid, p.need, sh, &a2);
  if (t == 0) {
    p.st->thresh = unbias(tv);
    p.st->ccount = 0u;
    p.st->eqcount = 0u;
  }
}

// Copy every value above the sampled threshold t to the candidate buffer
// (one vote per 16-byte vector, staged appends) and count the values
// equal to t, then let the last workgroup decide, with gt values copied
// and eq equal to t:
//  * gt + eq >= k and gt <= kFinishMax: the top-k is the top-k of the
//    copy, completed with copies of t when gt < k; the finish kernel
//    selects it alone (fast);
//  * otherwise gt >= k and the copy holds all of them: the selection
//    passes read the copy;
//  * otherwise they read the input.
// Either way it writes the state the selection starts from.
// What the waves still hold at the end goes out with one device atomic per
// workgroup, not per wave: a stream's end puts every wave's last flush on
// the one counter at about the same time.
__device__ __forceinline__ void flush_block(Stager& stg, int (*stage)[kStage],
                                            int* wcnt) {
  const int w = threadIdx.x / kWave;
  if (lane() == 0) wcnt[w] = stg.cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int total = 0;
    for (int j = 0; j < kWaves; ++j) total += wcnt[j];
    wcnt[kWaves] = total ? (int)atomicAdd(stg.counter, (unsigned)total) : 0;
  }
  __syncthreads();
  unsigned base = (unsigned)wcnt[kWaves];
  for (int j = 0; j < w; ++j) base += (unsigned)wcnt[j];
  for (int i = lane(); i < stg.cnt; i += kWave) {
    const unsigned pos = base + (unsigned)i;
    if (pos < stg.cap) stg.dst[pos] = stage[w][i];
  }
  stg.cnt = 0;
}

template <int U>
__global__ __launch_bounds__(kBlock) void filter_kernel(SelectParams p) {
  __shared__ int stage[kWaves][kStage];
  __shared__ int wcnt[kWaves + 1];
  __shared__ unsigned weq[kWaves];
  __shared__ int is_last;
  const int w = threadIdx.x / kWave;
  const int t = p.st->thresh;
  Stager stg{stage[w], 0, &p.st->ccount, p.cand, (unsigned)kCandCap};
  unsigned eq = 0;  // wave-uniform count of values equal to t
  auto one = [&](int x, bool ok) __attribute__((always_inline)) {
    stg.put(ok && x > t, x);
    eq += (unsigned)popc(ballot(ok && x == t));
  };
  for_each_vector<U>(
      p.in, p.n, p.head, p.ntiles, p.covered, p.grid, (int)blockIdx.x,
      [&](const v4i& d) __attribute__((always_inline)) {
        if (ballot(max(max(d.x, d.y), max(d.z, d.w)) >= t) == 0) return;
        one(d.x, true);
        one(d.y, true);
        one(d.z, true);
        one(d.w, true);
      },
      one);
  flush_block(stg, stage, wcnt);
  if (lane() == 0) weq[w] = eq;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned e = 0;
    for (int j = 0; j < kWaves; ++j) e += weq[j];
    if (e) atomicAdd(&p.st->eqcount, e);
  }
  if (!last_to_finish(p.ticket, p.grid, p.epoch, &is_last)) return;
  if (threadIdx.x == 0) {
    const unsigned gt = ld_agent(&p.st->ccount);
    const unsigned eqs = ld_agent(&p.st->eqcount);
    const unsigned k = (unsigned)p.k;
    const bool fast = gt <= (unsigned)kFinishMax && (gt >= k || eqs >= k - gt);
    const bool copy = !fast && gt >= k && gt <= (unsigned)kCandCap;
    RadixState& s = *p.st;
    s.prefix = 0u;
    s.mask = 0u;
    s.kleft = p.k;
    s.done = 0;
    s.bucket = fast || copy ? (int)gt : 0;
    s.src = copy ? 1 : 0;
    s.split = 0;
    s.gcount = 0u;
    s.ccount = 0u;
    s.eqcount = 0u;
    s.fast = fast;
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
  if (s.fast) return;  // the finish kernel gathers from its own copy
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
  if (!last_to_finish(p.ticket, grid, p.epoch, &is_last)) return;
  if (!s.done) {
    const int g = unbias(s.prefix);
    for (int j = p.k - s.kleft + (int)threadIdx.x; j < p.k; j += kBlock)
      p.out[j] = g;
  }
}

// Sort src[0..k) (k <= kMaxKSelect) descending into dst[0..k) in one
// workgroup of 1024 threads (src may be lds, and dst src): a bitonic
// network over m = k rounded up to a power of two (at least 1024; padding
// INT_MIN).  Thread t holds elements t + 1024 j, j < V = m / 1024, in
// registers, so a compare-exchange step of distance d costs: d < 64, a
// lane exchange inside the wave (DPP and row swaps, in registers); d >=
// 1024, a swap between two of the thread's registers; 64 <= d < 1024, a
// round trip through LDS with two barriers, which takes two such steps
// at once when it can (only these need the workgroup).
constexpr int kSortThreads = 1024;

template <int V>
__device__ __forceinline__ void sort_desc_block(const int* src, int* dst,
                                                int k, int* lds) {
  constexpr int m = V * kSortThreads;
  const int t = threadIdx.x;
  int v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j * kSortThreads + t;
    v[j] = i < k ? src[i] : kI32Min;
  }
  __syncthreads();  // every read of src is done before lds is written
  // Keep the max at position i of a pair when i is the lower index of a
  // pair in a run sorted descending, or the upper in an ascending one.
  auto keep_max = [](int i, int d, int size) __attribute__((always_inline)) {
    return ((i & d) == 0) == ((i & size) == 0);
  };
  // Runs of up to 32: directions follow the lane bits.
#pragma unroll
  for (int j = 0; j < V; ++j) v[j] = bitonic_sort<2, 32>(v[j]);
  for (int size = 64; size <= m; size <<= 1) {
    for (int d = size >> 1; d >= kWave; d >>= 1) {
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
      } else {
        // Through LDS, two distances (d and d / 2) per round trip when
        // both need it: element i reads the other three of its group of
        // four and does both steps itself.
        const int h = d >> 1;
        const bool two = h >= kWave;
#pragma unroll
        for (int j = 0; j < V; ++j) lds[j * kSortThreads + t] = v[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int i = j * kSortThreads + t;
          const int o = lds[i ^ d];
          const int a = keep_max(i, d, size) ? max(v[j], o) : min(v[j], o);
          if (two) {
            const int c = lds[i ^ h], e = lds[i ^ h ^ d];
            const int c1 = keep_max(i ^ h, d, size) ? max(c, e) : min(c, e);
            v[j] = keep_max(i, h, size) ? max(a, c1) : min(a, c1);
          } else {
            v[j] = a;
          }
        }
        __syncthreads();
        if (two) d = h;  // both distances done
      }
    }
    // Distances 32 .. 1: the run's direction is the same for the wave.
#pragma unroll
    for (int j = 0; j < V; ++j)
      v[j] = merge_dir<32>(v[j], ((j * kSortThreads + t) & size) == 0);
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j * kSortThreads + t;
    if (i < k) dst[i] = v[j];
  }
}

__device__ __forceinline__ void sort_desc(const int* src, int* dst, int k,
                                          int* lds) {
  if (k <= kSortThreads) sort_desc_block<1>(src, dst, k, lds);
  else if (k <= 2 * kSortThreads) sort_desc_block<2>(src, dst, k, lds);
  else if (k <= 4 * kSortThreads) sort_desc_block<4>(src, dst, k, lds);
  else if (k <= 8 * kSortThreads) sort_desc_block<8>(src, dst, k, lds);
  else sort_desc_block<16>(src, dst, k, lds);
}

// The last step of radix selection, one workgroup of 1024 threads.
//
// After the selection passes and the gather (state.fast == 0), out holds
// the top-k unordered: place it by a digit (fin_place_all) or sort it.
//
// After a small filter copy (state.fast == 1) of m values above the
// threshold t: when m < k, they and k - m copies of t are the top-k.
// Otherwise select from the m candidates (m <= kFinishMax) here, with
// barriers instead of device counters between digits.  Every candidate is
// above t, so all of them share the leading one bits of bias(t): those
// bits start the prefix, and the digits below them follow ([Radix]
// §3.2's digits): up to 12 bits in one shared 4096-bin histogram while
// more than 8 bits remain, then 8-bit digits with one LDS histogram per
// wave.  When the copy fits in LDS (kFinBucketCap) the first digit pass
// copies it there and later passes read LDS; otherwise passes read the
// copy until a chosen bucket fits, and that pass keeps the bucket in LDS
// and the values above it as known members of the top-k.  The result is
// then placed by the first digit's counts (fin_place) when k and the bins
// are small enough, or else gathered (the values above the final bucket,
// or the whole bucket when it is needed entire, and copies of g) and
// sorted by a bitonic network in LDS.
constexpr int kFinThreads = kSortThreads;
constexpr int kFinWaves = kFinThreads / kWave;
// LDS: top (64 KiB) + bucket (76 KiB) + histograms (16 KiB) fill the
// 160 KiB a gfx950 workgroup may hold.
constexpr int kFinBucketCap = 19456;

struct FinishShared {
  int top[kMaxKSelect];  // known top-k members; then the sort's exchange
  alignas(16) int bucket[kFinBucketCap];
  unsigned h[kFinWaves * kDigitBins];
  int scan[kFinWaves];
  int ntop, nbucket;
  int pick[3];  // digit, count above it, count in it
  int maxc;     // the largest count of the first digit's bins
};

// Visit cand[0..m) as f(x, ok, i), kFinRound 16-byte vectors per thread
// and round; every thread takes part in every round (ok false where
// nothing is left), so f may use wave votes.  The loads of a round are
// unconditional, so they issue back to back: the last round reads up to
// kFinRound * kFinThreads vectors past m, which stay inside the candidate
// buffer (kCandCap elements, and m <= kFinishMax).
constexpr int kFinRound = 8;
static_assert(kFinishMax + 4 * kFinRound * kFinThreads <= kCandCap,
              "finish rounds must stay inside the candidate buffer");

template <class F>
__device__ __forceinline__ void fin_visit_copy(const int* cand, int m, F&& f) {
  const v4i* cv = reinterpret_cast<const v4i*>(cand);
  const int nv = m >> 2, t = threadIdx.x;
  for (int base = 0; base < nv; base += kFinRound * kFinThreads) {
    v4i d[kFinRound];
    bool ok[kFinRound];
#pragma unroll
    for (int u = 0; u < kFinRound; ++u) d[u] = cv[base + u * kFinThreads + t];
#pragma unroll
    for (int u = 0; u < kFinRound; ++u) ok[u] = base + u * kFinThreads + t < nv;
#pragma unroll
    for (int u = 0; u < kFinRound; ++u) {
      const int i = 4 * (base + u * kFinThreads + t);
      f(d[u].x, ok[u], i);
      f(d[u].y, ok[u], i + 1);
      f(d[u].z, ok[u], i + 2);
      f(d[u].w, ok[u], i + 3);
    }
  }
  const int rest = m & 3;
  if (rest) {
    const bool ok = t < rest;
    const int i = (nv << 2) + t;
    f(ok ? cand[i] : kI32Min, ok, i);
  }
}

// Two compactions from one pass over the copy (qa into a, qb into b), in
// rounds: each thread counts what passes among its slots of the round,
// one exclusive scan over the workgroup (both counts packed in one word)
// places the slots after what earlier rounds appended, and the thread
// writes them.  hist(x) sees every element on the way.  Positions at or
// past a cap are dropped (a guard); the counts come back in *na, *nb.
template <int N, class H, class QA, class QB>
__device__ __forceinline__ void fin_round(const int (&x)[N], const bool (&ok)[N],
                                          H&& hist, QA&& qa, QB&& qb, int* a,
                                          int cap_a, int* b, int cap_b,
                                          int& na, int& nb, int* scan) {
  const int t = threadIdx.x, w = t / kWave;
  int ca = 0, cb = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (ok[j]) {
      hist(x[j]);
      ca += qa(x[j]) ? 1 : 0;
      cb += qb(x[j]) ? 1 : 0;
    }
  }
  // Per round at most N * kFinThreads <= 2^15 of each: no carry.
  const int packed = ca | (cb << 16);
  const int incl_w = wave_scan_incl(packed);
  if (lane() == kWave - 1) scan[w] = incl_w;
  __syncthreads();
  int before = incl_w - packed, total = 0;
#pragma unroll
  for (int j = 0; j < kFinWaves; ++j) {
    const int v = scan[j];
    before += j < w ? v : 0;
    total += v;
  }
  int pa = na + (before & 0xffff), pb = nb + (before >> 16);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (ok[j] && qa(x[j])) {
      if (pa < cap_a) a[pa] = x[j];
      ++pa;
    }
    if (ok[j] && qb(x[j])) {
      if (pb < cap_b) b[pb] = x[j];
      ++pb;
    }
  }
  na += total & 0xffff;
  nb += total >> 16;
  __syncthreads();  // scan is reused by the next round
}

template <class H, class QA, class QB>
__device__ __forceinline__ void fin_copy_compact(const int* cand, int m,
                                                 H&& hist, QA&& qa, QB&& qb,
                                                 int* a, int cap_a, int* b,
                                                 int cap_b, int* na_out,
                                                 int* nb_out, int* scan) {
  const v4i* cv = reinterpret_cast<const v4i*>(cand);
  const int nv = m >> 2, t = threadIdx.x;
  int na = 0, nb = 0;
  for (int base = 0; base < nv; base += kFinRound * kFinThreads) {
    // Unconditional loads, as in fin_visit_copy.
    v4i d[kFinRound];
#pragma unroll
    for (int u = 0; u < kFinRound; ++u) d[u] = cv[base + u * kFinThreads + t];
    int x[4 * kFinRound];
    bool ok[4 * kFinRound];
#pragma unroll
    for (int u = 0; u < kFinRound; ++u) {
      const bool in = base + u * kFinThreads + t < nv;
      x[4 * u] = d[u].x;
      x[4 * u + 1] = d[u].y;
      x[4 * u + 2] = d[u].z;
      x[4 * u + 3] = d[u].w;
      ok[4 * u] = ok[4 * u + 1] = ok[4 * u + 2] = ok[4 * u + 3] = in;
    }
    fin_round(x, ok, hist, qa, qb, a, cap_a, b, cap_b, na, nb, scan);
  }
  const int rest = m & 3;
  if (rest) {
    const bool in = t < rest;
    const int x[1] = {in ? cand[(nv << 2) + t] : kI32Min};
    const bool ok[1] = {in};
    fin_round(x, ok, hist, qa, qb, a, cap_a, b, cap_b, na, nb, scan);
  }
  *na_out = na;
  *nb_out = nb;
}

// Visit b[0..nb) in LDS as f(x, ok, i), kFinRound elements per thread and
// round; the reads of a round (indices clamped into the array) issue
// together.
template <class F>
__device__ __forceinline__ void fin_visit_lds(const int* b, int nb, F&& f) {
  const int t = threadIdx.x;
  for (int base = 0; base < nb; base += kFinRound * kFinThreads) {
    int x[kFinRound];
#pragma unroll
    for (int j = 0; j < kFinRound; ++j)
      x[j] = b[min(base + j * kFinThreads + t, nb - 1)];
#pragma unroll
    for (int j = 0; j < kFinRound; ++j) {
      const int i = base + j * kFinThreads + t;
      f(x[j], i < nb, i);
    }
  }
}

// The digit holding the kleft-th largest of a wide histogram (one copy of
// kFinWideBins bins; thread t owns bins kFinWideBins - 1 - 4t - i, i < 4);
// clears it.
constexpr int kFinWideBits = 12;
constexpr int kFinWideBins = 1 << kFinWideBits;
// Placement by the first digit: staged in LDS up to this k (the last
// quarter of `top`), and taken while no bin holds more than kPlaceBinMax.
constexpr int kPlaceMaxK = kMaxKSelect - 3 * kFinWideBins;  // LDS staging
constexpr int kPlaceBinMax = 32;
static_assert(kFinWideBins == kFinWaves * kDigitBins, "shares the waves' copies");
static_assert(kFinWideBins == 4 * kFinThreads, "four bins per thread");

// With `rec`, it also records each bin's count (rec[kFinWideBins + b]) and
// the count of the bins above it (rec[b]), and the largest count in
// sh.maxc.
__device__ __forceinline__ void fin_pick_wide(FinishShared& sh, int kleft,
                                              int* rec) {
  const int t = threadIdx.x, w = t / kWave;
  int c[4], local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = (int)sh.h[kFinWideBins - 1 - 4 * t - i];
    local += c[i];
  }
  if (rec) {
    const int mc = wave_max(max(max(c[0], c[1]), max(c[2], c[3])));
    if (lane() == 0) atomicMax(&sh.maxc, mc);
  }
  const int incl_w = wave_scan_incl(local);
  if (lane() == kWave - 1) sh.scan[w] = incl_w;
  __syncthreads();
  int run = incl_w - local;
#pragma unroll
  for (int j = 0; j < kFinWaves; ++j) run += j < w ? sh.scan[j] : 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = kFinWideBins - 1 - 4 * t - i;
    if (run + c[i] >= kleft && run < kleft) {
      sh.pick[0] = b;
      sh.pick[1] = run;
      sh.pick[2] = c[i];
    }
    if (rec) {
      rec[b] = run;
      rec[kFinWideBins + b] = c[i];
    }
    run += c[i];
    sh.h[b] = 0u;
  }
  __syncthreads();
}

// The digit holding the kleft-th largest of the histogram (waves' copies
// summed; thread t < 256 looks at bin 255 - t); clears the histogram.
__device__ __forceinline__ void fin_pick(FinishShared& sh, int kleft) {
  const int t = threadIdx.x, w = t / kWave;
  const int b = kDigitBins - 1 - t;
  int c = 0, incl_w = 0;
  if (t < kDigitBins) {
#pragma unroll
    for (int j = 0; j < kFinWaves; ++j) c += (int)sh.h[j * kDigitBins + b];
    incl_w = wave_scan_incl(c);
    if (lane() == kWave - 1) sh.scan[w] = incl_w;
  }
  __syncthreads();
  if (t < kDigitBins) {
    int incl = incl_w;
    for (int j = 0; j < w; ++j) incl += sh.scan[j];
    const int above = incl - c;
    if (incl >= kleft && above < kleft) {
      sh.pick[0] = b;
      sh.pick[1] = above;
      sh.pick[2] = c;
    }
  }
  for (int i = t; i < kFinWaves * kDigitBins; i += kFinThreads) sh.h[i] = 0u;
  __syncthreads();
}

// Append the elements of the LDS bucket b[0..nb) for which q holds to
// dst[base..), in one round (reads clamped into the array, issued
// together), placed by fin_round's scan.
template <class Q>
__device__ __forceinline__ void fin_compact(const int* b, int nb, int* dst,
                                            int base, int cap, int* scan,
                                            Q&& q) {
  // The whole bucket in one round: nb <= kFinBucketCap, N slots per
  // thread.
  constexpr int N = kFinBucketCap / kFinThreads;
  static_assert(N * kFinThreads == kFinBucketCap, "one round covers the bucket");
  if (nb <= 0) return;
  const int t = threadIdx.x;
  int na = base, nn = 0;
  int x[N];
  bool ok[N];
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = b[min(j * kFinThreads + t, nb - 1)];
#pragma unroll
  for (int j = 0; j < N; ++j) ok[j] = j * kFinThreads + t < nb;
  fin_round(
      x, ok, [](int) {}, q, [](int) { return false; }, dst, cap,
      static_cast<int*>(nullptr), 0, na, nn, scan);
}

// Placement by the first digit, instead of gathering and sorting.  The
// first (wide) digit pass counted every bin of the copy, and a bin above
// b0 (the one holding the k-th largest) holds only top-k members, so the
// output position of a member of bin b > b0 is the count of the bins
// above b plus its rank inside b; b0's members (those `wanted`) start at
// above0.  Members are grouped by bin in a staging area (a cursor per bin
// in LDS), then each finds its rank among its bin's members by counting
// (larger values, or equal ones at a lower slot), and after a barrier all
// are written to their places.  The staging area is LDS for k <=
// kPlaceMaxK; for larger k it is `out` itself (__syncthreads orders global
// memory within the workgroup too), copied to the free bucket area in LDS
// for the ranking, and the places are written after a barrier.  The members are read from the LDS
// copy (SRC_LDS) or from the copy in memory.  `fill` copies of g end the
// result.  Taken when no first-digit bin holds more than kPlaceBinMax
// values.
constexpr int kPlaceSlots = kMaxKSelect / kFinThreads;  // per thread

template <bool GSTAGE, bool SRC_LDS, class W>
__device__ __forceinline__ void fin_place(FinishShared& sh, const int* cand,
                                          int m, int nb, int* out, int k,
                                          unsigned shift0, unsigned mask0,
                                          int b0, int above0, W&& wanted,
                                          int fill, int g) {
  const int t = threadIdx.x;
  const int* off = sh.top;                        // bins above, per bin
  const int* cnt = sh.top + kFinWideBins;         // count, per bin
  int* cur = sh.top + 2 * kFinWideBins;           // cursor, per bin
  int* stage = GSTAGE ? out : sh.top + 3 * kFinWideBins;
  const int cap = GSTAGE ? k : kPlaceMaxK;
  for (int i = t; i < kFinWideBins; i += kFinThreads) cur[i] = 0;
  __syncthreads();
  auto bin = [&](int x) __attribute__((always_inline)) {
    return (int)((bias(x) >> shift0) & mask0);
  };
  auto group = [&](int x, bool ok, int) __attribute__((always_inline)) {
    const int b = bin(x);
    if (ok && (b > b0 || (b == b0 && wanted(x)))) {
      const int pos = (b > b0 ? off[b] : above0) + atomicAdd(&cur[b], 1);
      if (pos < cap) stage[pos] = x;
    }
  };
  if (SRC_LDS)
    fin_visit_lds(sh.bucket, nb, group);
  else
    fin_visit_copy(cand, m, group);
  __syncthreads();
  const int n0 = cur[b0];
  const int members = min(above0 + n0, k);
  if (GSTAGE) {
    // The ranking reads each bin's members many times over: from LDS, not
    // memory.  The bucket area is free by now (members <= k <=
    // kFinBucketCap).
    static_assert(kMaxKSelect <= kFinBucketCap, "bucket area holds k values");
    for (int i = t; i < members; i += kFinThreads) sh.bucket[i] = stage[i];
    __syncthreads();
    stage = sh.bucket;
  }
  int fx[kPlaceSlots], fp[kPlaceSlots];
#pragma unroll
  for (int j = 0; j < kPlaceSlots; ++j) {
    const int q = j * kFinThreads + t;
    fp[j] = -1;
    fx[j] = 0;
    if (q < members) {
      const int x = stage[q];
      const int b = bin(x);
      const int lo = b > b0 ? off[b] : above0;
      const int n = b > b0 ? cnt[b] : n0;
      int r = 0;
      for (int i = lo; i < lo + n; ++i) {
        const int y = stage[i];
        r += (y > x || (y == x && i < q)) ? 1 : 0;
      }
      fx[j] = x;
      fp[j] = lo + r;
    }
  }
  __syncthreads();  // every read of the staging area comes first
#pragma unroll
  for (int j = 0; j < kPlaceSlots; ++j)
    if (fp[j] >= 0) out[fp[j]] = fx[j];
  for (int j = k - fill + t; j < k; j += kFinThreads) out[j] = g;
}

// Sort the k values of out[0..k) descending by placement instead of a
// sorting network: their leading bits in common fix a window of up to 12
// bits below them, a histogram of that digit and its suffix counts give
// each bin's first place, the values are grouped by bin in LDS (in place
// in the bucket area, after all of them are read), and each is ranked
// among its bin's values by counting.  Returns false, having changed
// nothing, when a bin holds more than kPlaceBinMax values (the caller then
// sorts).  Barriers inside: call uniformly.
__device__ __forceinline__ bool fin_place_all(FinishShared& sh, int* out,
                                              int k) {
  const int t = threadIdx.x;
  int x[kPlaceSlots];
  int lo = kI32Max, hi = kI32Min;
#pragma unroll
  for (int j = 0; j < kPlaceSlots; ++j) {
    const int q = j * kFinThreads + t;
    x[j] = q < k ? out[q] : 0;
    if (q < k) {
      lo = min(lo, x[j]);
      hi = max(hi, x[j]);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (t == 0) {
    sh.pick[0] = kI32Max;
    sh.pick[1] = kI32Min;
  }
  for (int i = t; i < kFinWideBins; i += kFinThreads) sh.h[i] = 0u;
  __syncthreads();
  if (lane() == 0) {
    atomicMin(&sh.pick[0], lo);
    atomicMax(&sh.pick[1], hi);
  }
  __syncthreads();
  const unsigned blo = bias(sh.pick[0]), bhi = bias(sh.pick[1]);
  if (blo == bhi) return true;  // all equal: any order is sorted
  const int top = 31 - __builtin_clz(blo ^ bhi);  // highest differing bit
  const unsigned shift = top >= kFinWideBits - 1 ? (unsigned)(top - kFinWideBits + 1) : 0u;
  const unsigned dmask = (2u << (top - (int)shift)) - 1u;
  auto bin = [&](int v) __attribute__((always_inline)) {
    return (int)((bias(v) >> shift) & dmask);
  };
#pragma unroll
  for (int j = 0; j < kPlaceSlots; ++j)
    if (j * kFinThreads + t < k) atomicAdd(&sh.h[bin(x[j])], 1u);
  if (t == 0) sh.maxc = 0;
  __syncthreads();
  fin_pick_wide(sh, k, sh.top);  // suffix counts and counts into top
  if (sh.maxc > kPlaceBinMax) return false;
  const int* off = sh.top;
  const int* cnt = sh.top + kFinWideBins;
  int* cur = sh.top + 2 * kFinWideBins;
  int* stage = sh.bucket;
  for (int i = t; i < kFinWideBins; i += kFinThreads) cur[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPlaceSlots; ++j) {
    if (j * kFinThreads + t < k) {
      const int b = bin(x[j]);
      stage[off[b] + atomicAdd(&cur[b], 1)] = x[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPlaceSlots; ++j) {
    const int q = j * kFinThreads + t;
    if (q < k) {
      const int v = stage[q];
      const int b = bin(v);
      const int l0 = off[b], n = cnt[b];
      int r = 0;
      for (int i = l0; i < l0 + n; ++i) {
        const int y = stage[i];
        r += (y > v || (y == v && i < q)) ? 1 : 0;
      }
      out[l0 + r] = v;  // stage and out are distinct
    }
  }
  return true;
}

__global__ __launch_bounds__(kFinThreads) void select_finish_kernel(
    SelectParams p) {
  __shared__ FinishShared sh;
  const int t = threadIdx.x, w = t / kWave, k = p.k;
  const RadixState s = *p.st;
  if (!s.fast) {
    // One value per thread sorts faster than it is placed.
    if (k <= kFinThreads || !fin_place_all(sh, p.out, k))
      sort_desc(p.out, p.out, k, sh.top);
    return;
  }
  const int m = s.bucket;
  if (m < k) {
    // Fewer than k values above t: all of them, sorted, then copies of t
    // (only the m values are sorted: under heavy ties m is small, often 0).
    const int* cand = p.cand;
    for (int i = t; i < m; i += kFinThreads) sh.top[i] = cand[i];
    for (int i = m + t; i < k; i += kFinThreads) p.out[i] = s.thresh;
    __syncthreads();
    if (m > 0) sort_desc(sh.top, p.out, m, sh.top);
    if (t == 0) p.st->fast = 0;
    return;
  }
  for (int i = t; i < kFinWaves * kDigitBins; i += kFinThreads) sh.h[i] = 0u;
  if (t == 0) {
    sh.ntop = 0;
    sh.nbucket = 0;
    sh.maxc = 0;
  }
  __syncthreads();
  const unsigned ut = bias(s.thresh);
  // The leading one bits of bias(t) are shared by every candidate.
  const int lead = ~ut == 0u ? 32 : __builtin_clz(~ut);
  unsigned mask = lead == 0 ? 0u : ~0u << (32 - lead);
  unsigned prefix = mask;
  int rem = 32 - lead;  // bits below the prefix
  int kleft = k, count = m, nb = 0;
  bool done = false, in_lds = false;
  // Placement by the first digit (see below): that digit's window, the
  // bin holding the k-th largest and the count above it.
  bool place = false, place_lds = false;  // place_lds: the copy is in LDS
  unsigned shift0 = 0u, mask0 = 0u;
  int b0 = 0, above0 = 0;
  bool first = true;
  while (rem > 0 && !done) {
    // Digits of up to 12 bits (one shared histogram of 4096 bins) while
    // more than 8 bits remain, then the rest (per-wave copies).
    const bool wide = rem > 8;
    const int nbits = wide ? min(rem, kFinWideBits) : rem;
    const unsigned dshift = (unsigned)(rem - nbits);
    const unsigned dmask = (1u << nbits) - 1u;
    unsigned* hw = wide ? sh.h : sh.h + w * kDigitBins;
    if (in_lds) {
      fin_visit_lds(sh.bucket, nb, [&](int x, bool ok, int)
                                       __attribute__((always_inline)) {
        const unsigned u = bias(x);
        if (ok && (u & mask) == prefix)
          atomicAdd(&hw[(u >> dshift) & dmask], 1u);
      });
    } else if (count == m && m <= kFinBucketCap) {
      // The whole copy is the bucket and fits: copy it to LDS as it is,
      // 16 bytes at a time (the bucket array is 16-byte aligned).
      const v4i* cv = reinterpret_cast<const v4i*>(p.cand);
      v4i* bv = reinterpret_cast<v4i*>(sh.bucket);
      const int nv = m >> 2;
      auto count_digit = [&](int x) __attribute__((always_inline)) {
        atomicAdd(&hw[(bias(x) >> dshift) & dmask], 1u);
      };
      for (int base = 0; base < nv; base += kFinRound * kFinThreads) {
        v4i d[kFinRound];
#pragma unroll
        for (int u = 0; u < kFinRound; ++u)
          d[u] = cv[base + u * kFinThreads + t];
#pragma unroll
        for (int u = 0; u < kFinRound; ++u) {
          const int i = base + u * kFinThreads + t;
          if (i < nv) {
            bv[i] = d[u];
            count_digit(d[u].x);
            count_digit(d[u].y);
            count_digit(d[u].z);
            count_digit(d[u].w);
          }
        }
      }
      if (t < (m & 3)) {
        const int x = p.cand[(nv << 2) + t];
        sh.bucket[(nv << 2) + t] = x;
        count_digit(x);
      }
      in_lds = true;
      nb = m;
      place = first && wide;
      place_lds = place;
    } else if (count <= kFinBucketCap) {
      // The bucket fits now: keep it in LDS, and the values above it (all
      // in the top-k) in top.
      int na, nt;
      fin_copy_compact(
          p.cand, m,
          [&](int x) __attribute__((always_inline)) {
            const unsigned u = bias(x);
            if ((u & mask) == prefix) atomicAdd(&hw[(u >> dshift) & dmask], 1u);
          },
          [&](int x) __attribute__((always_inline)) {
            return (bias(x) & mask) == prefix;
          },
          [&](int x) __attribute__((always_inline)) {
            return (bias(x) & mask) > prefix;
          },
          // (top holds the placement's bin counts when placing: the
          // values above are then left for the placement to find)
          sh.bucket, kFinBucketCap, sh.top, place ? 0 : k, &na, &nt, sh.scan);
      in_lds = true;
      nb = min(na, kFinBucketCap);
      if (t == 0) sh.ntop = nt;
    } else {
      fin_visit_copy(p.cand, m, [&](int x, bool ok, int)
                                    __attribute__((always_inline)) {
        const unsigned u = bias(x);
        if (ok && (u & mask) == prefix)
          atomicAdd(&hw[(u >> dshift) & dmask], 1u);
      });
      if (first) place = wide;
    }
    __syncthreads();
    if (wide)
      fin_pick_wide(sh, kleft, place && first ? sh.top : nullptr);
    else
      fin_pick(sh, kleft);
    const unsigned d = (unsigned)sh.pick[0];
    const int above = sh.pick[1];
    count = sh.pick[2];
    if (place && first) {
      place = sh.maxc <= kPlaceBinMax;
      shift0 = dshift;
      mask0 = dmask;
      b0 = (int)d;
      above0 = above;
    }
    first = false;
    prefix |= d << dshift;
    mask |= dmask << dshift;
    kleft -= above;
    done = count == kleft;  // the whole bucket is needed
    rem -= nbits;
  }
  // The rest of the top-k: values above the final bucket (or in it, when
  // it is needed whole) from wherever the bucket is held; k - kleft
  // values in all.
  auto wanted = [&](int x) __attribute__((always_inline)) {
    const unsigned key = bias(x) & mask;
    return key > prefix || (done && key == prefix);
  };
  if (place) {
    const int fill = done ? 0 : kleft, g = unbias(prefix);
    if (k <= kPlaceMaxK) {
      if (place_lds)
        fin_place<false, true>(sh, p.cand, m, nb, p.out, k, shift0, mask0, b0,
                               above0, wanted, fill, g);
      else
        fin_place<false, false>(sh, p.cand, m, nb, p.out, k, shift0, mask0,
                                b0, above0, wanted, fill, g);
    } else {
      if (place_lds)
        fin_place<true, true>(sh, p.cand, m, nb, p.out, k, shift0, mask0, b0,
                              above0, wanted, fill, g);
      else
        fin_place<true, false>(sh, p.cand, m, nb, p.out, k, shift0, mask0,
                               b0, above0, wanted, fill, g);
    }
    if (t == 0) p.st->fast = 0;
    return;
  }
  if (in_lds) {
    fin_compact(sh.bucket, nb, sh.top, sh.ntop, k, sh.scan, wanted);
  } else {
    int na, nn;
    fin_copy_compact(
        p.cand, m, [](int) {}, wanted, [](int) { return false; }, sh.top, k,
        sh.bucket, 0, &na, &nn, sh.scan);
  }
  if (!done) {
    // All 32 bits are resolved: the prefix is g, and kleft copies of it
    // complete the top-k.
    const int g = unbias(prefix);
    for (int j = k - kleft + t; j < k; j += kFinThreads) sh.top[j] = g;
  }
  __syncthreads();
  sort_desc(sh.top, p.out, k, sh.top);
  if (t == 0) p.st->fast = 0;
}

}  // namespace ltk
