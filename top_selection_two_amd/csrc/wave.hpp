// Wave64 device primitives for gfx950 (CDNA4).
//
// Everything here works on one 64-lane wavefront: compare results become a
// 64-bit lane mask in scalar registers (ballot), counts are scalar popcounts
// of those masks, and loop decisions taken on them are wave-uniform scalar
// branches.  No shared memory, no barriers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ltk {

constexpr int kWave = 64;
constexpr int kBlock = 256;             // threads per workgroup (4 waves)
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxK = 128;
constexpr int kMaxGrid = 1024;          // stage-1 workgroups, upper bound
constexpr int kI32Min = (int)0x80000000;
constexpr int kI32Max = 0x7fffffff;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi(
      (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
}

__device__ __forceinline__ int lane() { return (int)__lane_id(); }

__device__ __forceinline__ int uni(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ unsigned uni(unsigned v) {
  return (unsigned)__builtin_amdgcn_readfirstlane((int)v);
}

// Order-preserving map int32 -> uint32 (and back): signed order becomes
// unsigned order, so bitwise radix selection works on plain unsigned values.
// A pointer known to be the same in every lane, moved to scalar registers.
template <class T>
__device__ __forceinline__ T* uni_ptr(T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ unsigned bias(int x) {
  return (unsigned)x ^ 0x80000000u;
}
__device__ __forceinline__ int unbias(unsigned u) {
  return (int)(u ^ 0x80000000u);
}

// Wave-wide max / min with DPP row shifts and row broadcasts: after the
// four row_shr steps lane 15 of every 16-lane row holds that row's
// reduction, the two broadcasts carry it across rows, and lane 63 ends with
// the result of the whole wave.  Lanes without a source (or in a row the
// row mask leaves out) read the operator's identity, so the compiler can
// fold each move into the max or min as a DPP operand.
#define LTK_DPP(id, v, ctrl, rows) \
  __builtin_amdgcn_update_dpp((id), (v), (ctrl), (rows), 0xf, false)

__device__ __forceinline__ int wave_max(int v) {
  v = max(v, LTK_DPP(kI32Min, v, 0x111, 0xf));  // row_shr:1
  v = max(v, LTK_DPP(kI32Min, v, 0x112, 0xf));  // row_shr:2
  v = max(v, LTK_DPP(kI32Min, v, 0x114, 0xf));  // row_shr:4
  v = max(v, LTK_DPP(kI32Min, v, 0x118, 0xf));  // row_shr:8
  v = max(v, LTK_DPP(kI32Min, v, 0x142, 0xa));  // row_bcast:15 into rows 1, 3
  v = max(v, LTK_DPP(kI32Min, v, 0x143, 0xc));  // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_min(int v) {
  v = min(v, LTK_DPP(kI32Max, v, 0x111, 0xf));
  v = min(v, LTK_DPP(kI32Max, v, 0x112, 0xf));
  v = min(v, LTK_DPP(kI32Max, v, 0x114, 0xf));
  v = min(v, LTK_DPP(kI32Max, v, 0x118, 0xf));
  v = min(v, LTK_DPP(kI32Max, v, 0x142, 0xa));
  v = min(v, LTK_DPP(kI32Max, v, 0x143, 0xc));
  return __builtin_amdgcn_readlane(v, 63);
}

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

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    int lo = __shfl_xor((int)(uint32_t)v, o, kWave);
    int hi = __shfl_xor((int)(v >> 32), o, kWave);
    v += (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  }
  return v;
}

// Keep the compiler (IR passes and the machine scheduler) from moving
// memory operations or any instruction across this point.
// The streaming loops use it so that the loads of the next tile are not
// hoisted above the use of the current one: hoisting would leave both
// buffers live at once, force register copies at the loop latch, and the
// copies would wait for the loads that were meant to stay in flight.
__device__ __forceinline__ void sched_fence() {
  asm volatile("" ::: "memory");  // loads stay on their side at IR level
  __builtin_amdgcn_sched_barrier(0);
}

// Optimisation barriers on values.  ready(d) marks the point where the
// loaded tile d is first needed: every use of d comes after it, so the
// wait for d's loads is placed there and not earlier.  pin(x) keeps the
// compiler from reassociating work on x across this point (for example
// folding two tiles into one expression tree, which would make the first
// tile wait for the second tile's loads).
template <int U>
__device__ __forceinline__ void ready(v4i (&d)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) asm volatile("" : "+v"(d[u]));
}
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// The tiles of one workgroup: tile i of workgroup blk is global tile
// blk + i * grid of the 16-byte-aligned body; a tile is kBlock lanes x U
// 16-byte vectors, lane-contiguous per vector (each wave instruction reads
// 1 KiB of consecutive bytes).  Plain scalars rather than a struct, so that
// nothing about the stream ever lives in private memory.
__device__ __forceinline__ int64_t tiles_of(int64_t ntiles, int blk,
                                            int grid) {
  return blk < ntiles ? (ntiles - blk + grid - 1) / grid : 0;
}

// Load local tile i with buffer loads (non-temporal: every byte is read
// exactly once).  A prefetch past the end (i >= count) goes through a
// buffer of no bytes: its loads return zeros and read no memory, with the
// same instructions, so the wait before each tile stays the same on every
// path.  (Clamping to the last tile re-read it from HBM: 1.2-1.5 % extra
// traffic for the statistics and the histogram.)  The buffer's fourth
// word is the gfx9 default (32-bit data, no swizzle, no stride).
template <int U>
__device__ __forceinline__ void load_tile(const v4i* __restrict__ body,
                                          int blk, int grid, int64_t count,
                                          int64_t i, v4i (&d)[U]) {
  const bool in = i < count;
  const v4i* tile = body + (blk + (in ? i : 0) * grid) * (int64_t)(kBlock * U);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<v4i*>(tile), (short)0, in ? kBlock * U * 16 : 0,
      0x00020000);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const auto q = __builtin_amdgcn_raw_buffer_load_b128(
        r, (int)((threadIdx.x + u * kBlock) * 16), 0, 2 /* nt */);
    d[u] = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
  }
}

// Cross-workgroup hand-off without an agent-scope fence.
//
// The last workgroup to finish reads what every other workgroup published.
// An agent-scope release fence would make that legal for plain stores, but
// on this chip it writes back the whole L2 of the XCD, and a fence per
// workgroup costs about 0.2 us each, serialised (it more than doubles the
// time of a 400 MB streaming pass at 1024 workgroups).  Instead, published
// values are written with agent-scope atomic stores, which are coherent at
// device level (write-through, sc1), every wave waits for its own memory
// operations to complete before the workgroup takes its ticket, and the
// reader uses agent-scope atomic loads (sc1), which do not hit stale lines.
template <class T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
// The elements outside a stream's full tiles -- the unaligned head (fewer
// than 4) and the tail (less than one tile of TILE elements) -- one per
// thread and round, as f(x, pos, ok): x the element at position pos of
// `in`, ok false (x INT_MIN) past the end.  Every thread takes part in
// every round that has an element, so f may use wave votes.  The loads of
// all rounds are issued before the first call: one memory round trip, not
// one per round (a tail of 3,392 elements took 14 dependent round trips,
// about 4 us, on the last workgroup's path).
template <int TILE, class F>
__device__ __forceinline__ void visit_rest(const int* in, int64_t n,
                                           int64_t head, int64_t covered,
                                           F&& f) {
  constexpr int R = (3 + TILE + kBlock - 1) / kBlock;
  const int64_t left = n - covered;
  int x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = (int64_t)r * kBlock + threadIdx.x;
    x[r] = i < left ? in[i < head ? i : covered + i] : kI32Min;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = (int64_t)r * kBlock + threadIdx.x;
    if ((int64_t)r * kBlock < left) f(x[r], i < head ? i : covered + i, i < left);
  }
  // The stream geometry leaves fewer; any more go round by round.
  for (int64_t base = (int64_t)R * kBlock; base < left; base += kBlock) {
    const int64_t i = base + threadIdx.x;
    const int64_t pos = i < head ? i : covered + i;
    f(i < left ? in[pos] : kI32Min, pos, i < left);
  }
}

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void drain_memory_ops() {
  __builtin_amdgcn_s_waitcnt(0);
}

// ---- counters tagged with the launch's epoch ------------------------------
// Every launch gets an epoch from the host (a per-scratch counter, new for
// each launch).  A device counter shared by the workgroups of a launch
// (completion ticket, histogram bin) is one 64-bit word: the epoch's tag in
// the high bits, the launch's count in the low CB bits.  Whoever reads or
// takes the last count of a word leaves it "armed" for the next epoch (tag
// epoch + 1, count 0), so in the ordinary sequence of launches every add
// meets its own tag and costs one atomic.  A word with any other tag (left
// by a launch that never finished, or overwritten) is foreign: an add that
// returns a foreign word installs the launch's tag with its own amount by
// compare-and-swap, and if another workgroup installed it first, adds again
// (its first add went to the foreign value, which the installation
// replaced).  So a word's count never depends on what it held before the
// launch, unless its stale tag happens to equal the launch's own (one
// chance in 2^31 or more for an arbitrary value).
template <int CB>
struct Tagged {
  static constexpr uint64_t kCountMask = (1ull << CB) - 1ull;
  static constexpr uint32_t kTagMask = (uint32_t)((1ull << (64 - CB)) - 1ull);
  __device__ static uint64_t armed(uint32_t epoch) {
    return (uint64_t)(epoch & kTagMask) << CB;
  }
  __device__ static bool mine(uint64_t w, uint32_t epoch) {
    return (uint32_t)(w >> CB) == (epoch & kTagMask);
  }
  // Add c (> 0) to the launch's count in *w; returns the count before the
  // add.  The loop ends: each pass either succeeds or sees the word changed
  // by another of the launch's at most `grid` adds.
  __device__ static uint64_t add(uint64_t* w, uint64_t c, uint32_t epoch) {
    unsigned long long* a = reinterpret_cast<unsigned long long*>(w);
    const uint64_t o = atomicAdd(a, (unsigned long long)c);
    if (mine(o, epoch)) return o & kCountMask;
    uint64_t cur = o + c;
    for (;;) {
      const uint64_t prev = atomicCAS(a, (unsigned long long)cur,
                                      (unsigned long long)(armed(epoch) | c));
      if (prev == cur) return 0;
      if (mine(prev, epoch))
        return atomicAdd(a, (unsigned long long)c) & kCountMask;
      cur = prev;
    }
  }
  // The launch's count held in a word read after every add has completed
  // (0 if no add of this launch reached it).
  __device__ static uint64_t count(uint64_t w, uint32_t epoch) {
    return mine(w, epoch) ? (w & kCountMask) : 0ull;
  }
};
typedef Tagged<32> Ticket;    // completion tickets: 32-bit epoch, 32-bit count

// Take the workgroup's completion ticket after its published stores have
// completed; true in exactly one workgroup, the last one of the `grid` that
// take this ticket in this launch, which also arms the ticket for the next
// epoch.  Barriers inside: call uniformly.  `flag` is an LDS word.
__device__ __forceinline__ bool last_to_finish(uint64_t* ticket, int grid,
                                               uint32_t epoch, int* flag) {
  drain_memory_ops();
  __syncthreads();
  if (threadIdx.x == 0) {
    const bool last = Ticket::add(ticket, 1, epoch) == (uint64_t)(grid - 1);
    if (last) st_agent(ticket, Ticket::armed(epoch + 1u));
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// Direct global -> LDS streaming (gfx950 global_load_lds_dwordx4).  Each
// lane's 16 bytes land at M0 + 16 * lane, so one instruction moves 1 KiB
// of consecutive HBM bytes into 1 KiB of consecutive LDS without passing
// through VGPRs.  Issued non-temporal: every byte is read exactly once.
//
// The loads are written as inline assembly on purpose.  The compiler's own
// tracking of LDS-targeting loads makes it wait for ALL of them (vmcnt(0))
// before any LDS access that might alias, which would drain the ring at
// every tile.  Hidden in asm, they are ordered by hand instead:
// wait_tile_loads() (an explicit vmcnt wait) before a tile's slot is read,
// and wait_lds_reads() before a slot that was just read is refilled.  All
// of these carry a memory clobber, so the compiler moves no memory access
// across them and keeps the reads of the ring (whose address escapes into
// the asm).  M0 is saved and restored around each load, so the compiler's
// view of M0 is unchanged.  The streaming loop issues no other vector-memory
// instruction, so vmcnt counts exactly the outstanding tile loads.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(
      (const __attribute__((address_space(3))) void*)p);
}

// Issue the U loads of one tile: `tile` is the tile's first byte (a
// wave-uniform address, kept in SGPRs), `voff[u]` this lane's byte offset
// within it for load u, and `lds` the wave's slot in LDS.  No per-tile
// vector address arithmetic.
template <int U>
__device__ __forceinline__ void issue_tile_lds(const char* tile,
                                               const uint32_t (&voff)[U],
                                               v4i (*slot)[kWave]) {
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)lds_offset(&slot[0][0]));
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[lds]\n\t"
        "global_load_lds_dwordx4 %[vo], %[base] nt\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(saved)
        : [lds] "s"(lds + u * kWave * 16u), [vo] "v"(voff[u]),
          [base] "s"(tile)
        : "memory");
  }
}

// Before a tile's slot is read: wait until at most the loads of the tiles
// issued after it are pending.  In the steady state that is kRing - 1
// tiles of U loads; near the end of the stream everything is drained.
template <int U, int RING>
__device__ __forceinline__ void wait_tile_loads(bool steady) {
  static_assert(U * (RING - 1) <= 63, "vmcnt is a 6-bit counter");
  if (steady)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(U * (RING - 1)) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void wait_lds_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Workgroup barrier that waits for this wave's LDS traffic only: the tile
// loads in flight stay in flight (a __syncthreads() would drain them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Bitwise radix selection.  Given a wave-uniform range [lo, hi] (biased
// values) that is known to contain the answer, return the largest t in it
// with count_ge(t) >= k, where count_ge is a wave-uniform count of the
// values >= t.  Precondition: count_ge(lo) >= k.  Bits above the highest
// bit in which lo and hi differ are shared by every value of the range, so
// only the bits below it are decided, one per step.
template <class CountGe>
__device__ __forceinline__ unsigned radix_select(unsigned lo, unsigned hi,
                                                 int k, CountGe count_ge) {
  lo = uni(lo);
  hi = uni(hi);
  const unsigned diff = lo ^ hi;
  if (diff == 0u) return lo;
  const int top = 31 - __clz((int)diff);
  unsigned prefix = lo & ~((2u << top) - 1u);
  for (int b = top; b >= 0; --b) {
    const unsigned c = prefix | (1u << b);
    if (count_ge(c) >= k) prefix = c;
  }
  return prefix;
}

// The same search cut short after `steps` bits: the result is a value v
// with count_ge(v) >= k that is <= the exact answer, and close to it (the
// undecided low bits are zero).  Every prefix kept along the way satisfies
// the count, and lo itself does (precondition), so max(prefix, lo) does.
template <class CountGe>
__device__ __forceinline__ unsigned radix_lower_bound(unsigned lo, unsigned hi,
                                                      int k, int steps,
                                                      CountGe count_ge) {
  lo = uni(lo);
  hi = uni(hi);
  const unsigned diff = lo ^ hi;
  if (diff == 0u) return lo;
  const int top = 31 - __clz((int)diff);
  unsigned prefix = lo & ~((2u << top) - 1u);
  // Ties at the top (for example an input of equal values): if the largest
  // value already has k values at or above it, it is the exact answer.
  if (count_ge(hi) >= k) return hi;
  const int last = top - steps + 1 > 0 ? top - steps + 1 : 0;
  for (int b = top; b >= last; --b) {
    const unsigned c = prefix | (1u << b);
    if (count_ge(c) >= k) prefix = c;
  }
  return prefix > lo ? prefix : lo;
}

// Count over V biased values per lane held in registers.
template <int V>
struct RegCount {
  const unsigned (&u)[V];
  __device__ __forceinline__ int operator()(unsigned c) const {
    int n = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) n += popc(ballot(u[j] >= c));
    return n;
  }
};

// ---------------------------------------------------------------------------
// Bitonic compare-exchange across a wave, in registers.

// Lanes whose bit is set in `mask` take a, the others b: one v_cndmask
// whose condition is a constant lane mask held in a scalar register pair.
__device__ __forceinline__ int pick_lanes(uint64_t mask, int a, int b) {
  int r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(b), "v"(a), "s"(mask));
  return r;
}

// Lanes l with (l & bit) != 0.
constexpr uint64_t lanes_with(int bit) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if (l & bit) m |= 1ull << l;
  return m;
}

// Lanes that keep the larger value of their pair in the bitonic step with
// partner distance s inside runs of `size`: the lower lane of a pair in a
// run sorted descending, the upper lane in an ascending one.
constexpr uint64_t keep_max_lanes(int size, int s) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if (((l & s) == 0) == ((l & size) == 0)) m |= 1ull << l;
  return m;
}

// DPP controls: quad permutes [1,0,3,2] and [2,3,0,1], row rotations by 4,
// 8 and 12 (dst lane i of a 16-lane row reads lane (i - r) mod 16).
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e;
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128, kRowRor12 = 0x12c;

// One compare-exchange step of a bitonic network across the wave: every
// lane meets the lane at distance s (l ^ s) and keeps the max (lanes in
// KEEP) or the min.
// For s = 1, 2, 8 the partner arrives as a DPP operand of the max and of the
// min themselves (the identity as `old` lets the compiler fold the moves);
// for s = 4 two bank-masked row rotations build it (banks 1 and 3 of a row
// read 4 lanes down, banks 0 and 2 read 4 lanes up); for 16 and 32 the
// gfx950 row swaps return both halves of the exchange.
template <int S, uint64_t KEEP>
__device__ __forceinline__ int cx_keep(int v) {
  int hi, lo;
  if constexpr (S == 1 || S == 2 || S == 8) {
    constexpr int c = S == 1 ? kQuadXor1 : S == 2 ? kQuadXor2 : kRowRor8;
    hi = max(v, __builtin_amdgcn_update_dpp(kI32Min, v, c, 0xf, 0xf, false));
    lo = min(v, __builtin_amdgcn_update_dpp(kI32Max, v, c, 0xf, 0xf, false));
  } else {
    int o;
    if constexpr (S == 4) {
      const int t =
          __builtin_amdgcn_update_dpp(0, v, kRowRor4, 0xf, 0xa, false);
      o = __builtin_amdgcn_update_dpp(t, v, kRowRor12, 0xf, 0x5, false);
    } else {
      const auto r =
          S == 16 ? __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v,
                                                     false, false)
                  : __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v,
                                                     false, false);
      o = pick_lanes(lanes_with(S), (int)r[0], (int)r[1]);
    }
    hi = max(v, o);
    lo = min(v, o);
  }
  return pick_lanes(KEEP, hi, lo);
}

template <int SIZE, int S>
__device__ __forceinline__ int bitonic_step(int v) {
  return cx_keep<S, keep_max_lanes(SIZE, S)>(v);
}

// The last steps of a bitonic merge, partner distances S, S / 2, .., 1, in
// runs whose direction is the same for the whole wave (runs longer than
// the wave): descending, or ascending.
template <int S>
__device__ __forceinline__ int merge_dir(int v, bool desc) {
  v = desc ? cx_keep<S, ~lanes_with(S)>(v) : cx_keep<S, lanes_with(S)>(v);
  if constexpr (S > 1) v = merge_dir<S / 2>(v, desc);
  return v;
}

template <int SIZE, int S>
__device__ __forceinline__ int bitonic_merge(int v) {
  v = bitonic_step<SIZE, S>(v);
  if constexpr (S > 1) v = bitonic_merge<SIZE, S / 2>(v);
  return v;
}

template <int SIZE, int W>
__device__ __forceinline__ int bitonic_sort(int v) {
  v = bitonic_merge<SIZE, SIZE / 2>(v);
  if constexpr (SIZE < W) v = bitonic_sort<SIZE * 2, W>(v);
  return v;
}

// Bitonic sort of one value per lane, descending, within aligned groups of
// W lanes (W = 32 or 64): lane 0 of a group ends with its largest value.
// log2(W) (log2(W) + 1) / 2 compare-exchange steps, all in registers.
template <int W>
__device__ __forceinline__ int wave_sort_desc(int v) {
  return bitonic_sort<2, W>(v);
}

// Bitonic sort of 64 R values held R per lane (value j * 64 + lane in
// v[j]), descending: runs of one register sorted across the lanes in
// alternating directions (ascending as the complement of a descending
// sort: ~x reverses the order of int32 with no overflow), then each
// longer run merged by compare-exchanges between registers (partners 64
// and more apart) and lane exchanges (32 .. 1).  Afterwards v[0] holds the
// 64 largest, lane 0 the largest of all.
template <int R>
__device__ __forceinline__ void wave_sort_desc_regs(int (&v)[R]) {
  static_assert(R >= 1 && (R & (R - 1)) == 0, "R a power of two");
#pragma unroll
  for (int j = 0; j < R; ++j)
    v[j] = (j & 1) ? ~wave_sort_desc<kWave>(~v[j]) : wave_sort_desc<kWave>(v[j]);
#pragma unroll
  for (int size = 2; size <= R; size <<= 1) {  // runs of `size` registers
#pragma unroll
    for (int js = size / 2; js >= 1; js >>= 1) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if ((j & js) == 0) {
          const bool desc = (j & size) == 0;
          const int a = v[j], b = v[j | js];
          v[j] = desc ? max(a, b) : min(a, b);
          v[j | js] = desc ? min(a, b) : max(a, b);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = merge_dir<32>(v[j], (j & size) == 0);
  }
}

}  // namespace ltk
