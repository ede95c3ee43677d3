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
__device__ __forceinline__ unsigned bias(int x) {
  return (unsigned)x ^ 0x80000000u;
}
__device__ __forceinline__ int unbias(unsigned u) {
  return (int)(u ^ 0x80000000u);
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return uni(v);
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return uni(v);
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

}  // namespace ltk
