// libtopk host side: argument checks, launch geometry, per-(device, stream)
// scratch, and the C entry points declared in include/libtopk.h.
//
// The launch plan follows the two-stage design of
//   [TopK]   "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计", §2.2
//            (a first launch over the data leaves k candidates per block, a
//            single block merges them) and §4.2 (size the grid to the
//            machine rather than fixing it),
//   [Reduce] "CUDA归约优化完全指南：从入门到精通", "complete multi-level
//            reduction" (one partial per block, then a pass over partials;
//            check launch errors after each launch),
// with both stages fused into a single launch (see the kernel headers).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <memory>
#include <mutex>
#include <utility>

#include "libtopk.h"
#include "hist_kernel.hpp"
#include "select_kernel.hpp"
#include "reduce_kernel.hpp"
#include "stats_kernel.hpp"
#include "topk_kernel.hpp"
#include "topk_kv_kernel.hpp"
#include "topk_rows_kernel.hpp"
#include "seg_kernel.hpp"

namespace {

using namespace ltk;

constexpr int kTileVec = 4;         // 16-byte loads per lane per tile (U)
// Tiles between bound refreshes: every 16th for short lists (k <= 32),
// every 8th for longer ones, whose insertions cost more and profit more
// from a tighter bound (measured on 1e8 elements: k = 20, 32 faster at 16;
// k = 64, 100 faster at 8).
int refresh_period(int k) { return k <= 32 ? 16 : 8; }
constexpr int64_t kMaxN = (int64_t)1 << 32;

struct Scratch {
  void* base = nullptr;
  int* cand = nullptr;         // kMaxGrid * kMaxK
  int* heads = nullptr;        // kMaxGrid
  int* kths = nullptr;         // kMaxGrid
  int64_t* partials = nullptr; // kMaxGrid
  uint64_t* spart = nullptr;   // kMaxGrid * 4 (statistics partials)
  uint64_t* kvcand = nullptr;  // kMaxGrid * kMaxK (key-value candidates)
  uint64_t* kvheads = nullptr; // kMaxGrid
  uint64_t* kvkths = nullptr;  // kMaxGrid
  uint64_t* acc = nullptr;     // kMaxBins histogram counters (epoch-tagged)
  RadixState* rstate = nullptr;       // radix-selection state
  int* rcand = nullptr;               // kCandCap candidates + sample
                                      // lists, allocated by the first
                                      // top-k call with k > 128
  uint64_t* ticket = nullptr;  // kMaxGrid epoch-tagged tickets (one per row)
  // Segmented top-k: work lists, per-unit candidates and tickets, sized by
  // the largest n seen on the pair (grown on demand).
  void* seg_base = nullptr;
  int64_t seg_n = 0;
  // Launches on this scratch so far: each launch takes the next value as
  // its epoch, which tags the tickets and counters it uses (see Tagged in
  // wave.hpp).
  std::shared_ptr<std::atomic<uint32_t>> epochs;
  // Segmented top-k calls so far: each call's tag for the counters its two
  // launches share (the next call arms them).
  std::shared_ptr<std::atomic<uint32_t>> seg_calls;
};

// The epoch of a new launch on a scratch (never 0, which freshly cleared
// words carry).
uint32_t next_epoch(std::atomic<uint32_t>& c) {
  uint32_t e = c.fetch_add(1u) + 1u;
  while (e == 0u) e = c.fetch_add(1u) + 1u;
  return e;
}

constexpr size_t kCandBytes = (size_t)kMaxGrid * kMaxK * sizeof(int);
constexpr size_t kHeadBytes = (size_t)kMaxGrid * sizeof(int);
constexpr size_t kPartBytes = (size_t)kMaxGrid * sizeof(int64_t);
constexpr size_t kStatBytes = (size_t)kMaxGrid * 4 * sizeof(uint64_t);
constexpr size_t kKvCandBytes = (size_t)kMaxGrid * kMaxK * sizeof(uint64_t);
constexpr size_t kKvHeadBytes = (size_t)kMaxGrid * sizeof(uint64_t);
constexpr size_t kAccBytes = (size_t)kMaxBins * sizeof(uint64_t);
constexpr size_t kStateBytes = 256;
constexpr size_t kTicketBytes = (size_t)kMaxGrid * sizeof(uint64_t);
constexpr size_t kScratchBytes = kCandBytes + 2 * kHeadBytes + kPartBytes +
                                 kStatBytes + kKvCandBytes +
                                 2 * kKvHeadBytes + kAccBytes + kStateBytes +
                                 kTicketBytes;

std::mutex g_mu;
std::map<std::pair<int, void*>, Scratch> g_cache;
std::map<int, int> g_cus;          // device -> compute units
std::atomic<int> g_grid_override{0};

// With LIBTOPK_DEBUG set in the environment, HIP failures are described on
// stderr; otherwise the library prints nothing.
void debug_hip(const char* what, hipError_t e) {
  static const bool on = getenv("LIBTOPK_DEBUG") != nullptr;
  if (on) fprintf(stderr, "libtopk: %s: %s\n", what, hipGetErrorString(e));
}

__global__ void zero_words(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Test hook: overwrite n 64-bit words with pseudo-random nonzero values
// (a SplitMix64-style mix of seed and index).
__global__ void scramble_words(uint64_t* p, int n, uint64_t seed) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t z = seed + 0x9e3779b97f4a7c15ull * (uint64_t)(i + 1);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  p[i] = (z ^ (z >> 31)) | 1ull;
}

int current_device(int* dev) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1)
    return LIBTOPK_ERR_HIP;
  if (hipGetDevice(dev) != hipSuccess) return LIBTOPK_ERR_HIP;
  return LIBTOPK_OK;
}

// Caller holds g_mu.
int compute_units(int dev) {
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess || cus < 1)
    cus = 256;
  g_cus[dev] = cus;
  return cus;
}

// Workgroups of kernel `fn` (kBlock threads) that fit on one CU at once,
// as the runtime computes it from the kernel's registers and LDS; 1 if the
// query fails.  Caller holds g_mu.
std::map<const void*, int> g_fit;
int groups_per_cu(const void* fn) {
  auto it = g_fit.find(fn);
  if (it != g_fit.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kBlock, 0) !=
          hipSuccess ||
      nb < 1)
    nb = 1;
  g_fit[fn] = nb;
  return nb;
}

int get_scratch(int dev, hipStream_t stream, Scratch* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  const auto key = std::make_pair(dev, (void*)stream);
  auto it = g_cache.find(key);
  if (it != g_cache.end()) {
    *out = it->second;
    return LIBTOPK_OK;
  }
  Scratch s;
  if (getenv("LIBTOPK_TEST_FAIL_ALLOC")) return LIBTOPK_ERR_NOMEM;
  hipError_t e = hipMalloc(&s.base, kScratchBytes);
  if (e != hipSuccess) {
    debug_hip("hipMalloc(scratch)", e);
    (void)hipGetLastError();
    return LIBTOPK_ERR_NOMEM;
  }
  char* b = (char*)s.base;
  s.cand = (int*)b;
  b += kCandBytes;
  s.heads = (int*)b;
  b += kHeadBytes;
  s.kths = (int*)b;
  b += kHeadBytes;
  s.partials = (int64_t*)b;
  b += kPartBytes;
  s.spart = (uint64_t*)b;
  b += kStatBytes;
  s.kvcand = (uint64_t*)b;
  b += kKvCandBytes;
  s.kvheads = (uint64_t*)b;
  b += kKvHeadBytes;
  s.kvkths = (uint64_t*)b;
  b += kKvHeadBytes;
  s.acc = (uint64_t*)b;
  b += kAccBytes;
  s.rstate = (RadixState*)b;
  b += kStateBytes;
  s.ticket = (uint64_t*)b;
  s.epochs = std::make_shared<std::atomic<uint32_t>>(0u);
  s.seg_calls = std::make_shared<std::atomic<uint32_t>>(0u);
  // A kernel (not a memset) clears the histogram counters, the selection
  // state and the tickets (contiguous), ordered on the caller's stream
  // before the first real launch.  (Any value would do for the counters and
  // tickets, which carry epoch tags; zero is the tidy start.)
  const int zwords = (int)((kAccBytes + kStateBytes + kTicketBytes) / 4);
  hipLaunchKernelGGL(zero_words, dim3((zwords + 255) / 256), dim3(256), 0,
                     stream, (unsigned*)s.acc, zwords);
  e = hipGetLastError();
  if (e != hipSuccess) {
    debug_hip("zero_words launch", e);
    (void)hipFree(s.base);
    return LIBTOPK_ERR_HIP;
  }
  g_cache[key] = s;
  *out = s;
  return LIBTOPK_OK;
}

struct Plan {
  int64_t head, ntiles, covered;
  int grid;
};

// What a launch does with its tiles, for the choice of its grid.
enum GridKind {
  kGridTopk,    // top-k and key-value top-k (LDS ring, per-element lists)
  kGridReduce,  // sum, max, min and the statistics (register pipeline)
  kGridHist,    // histogram (an LDS atomic per element)
  kGridSelect,  // the sample, filter and digit passes of k > 128
};

// Stage-1 grid: up to `per_cu` workgroups per CU, fewer for smaller inputs,
// capped by the tiles there are.  Every workgroup ends with a device
// atomic on the launch's one ticket, and those serialise (about 12 ns
// each under load): on small inputs, where the workgroups finish together,
// 512 tickets alone take microseconds, so fewer workgroups with more tiles
// each win until the input is large.  The floors and tile ratios below are
// the measured best grids on 256 CUs (event-timed, uniform int32, n = 1e6,
// 4e6, 1.6e7, 3.2e7, 2^26 and 1e8):
//  * top-k: 192 at 1e6 (9.8 us against 10.5 at 244), 256 at 4e6 (13.3
//    against 15.5 at 512), 512 from 3.2e7;
//  * reductions and statistics: 64 at 1e6 (sum 4.5 us against 6.2), 128
//    at 4e6 (5.6 against 10.0), and never more than one per CU (sum of 1e8
//    55.9 us against 58.6 at 512; statistics 56.8 against 60.0);
//  * histogram: 128 at 1e6 (6.8 us against 7.9), 256 at 4e6 (9.6 against
//    11.8), 512 at 1e8;
//  * k > 128: 128 up to 4e6 (top-1000 of 4e6 31.8 us against 37.0), one
//    per CU beyond (top-1000 of 1e8 85.3 us against 87.5 at 512).
Plan plan(const int32_t* in, int64_t n, int cus, GridKind kind = kGridTopk,
          int per_cu = 2) {
  Plan pl;
  const uintptr_t a = (uintptr_t)in;
  int64_t head = (int64_t)(((16u - (a & 15u)) & 15u) / 4u);
  if (head > n) head = n;
  const int64_t vecs = (n - head) / 4;
  pl.head = head;
  pl.ntiles = vecs / (kBlock * kTileVec);
  pl.covered = pl.ntiles * kBlock * kTileVec * 4;
  int g = g_grid_override.load();
  if (g <= 0) {
    int64_t lo, hi, want;
    switch (kind) {
      case kGridReduce:
        lo = cus / 4, hi = cus, want = pl.ntiles / 8;
        break;
      case kGridHist:
        lo = cus / 2, hi = 2 * (int64_t)cus, want = pl.ntiles / 4;
        break;
      case kGridSelect:
        lo = cus / 2, hi = cus, want = pl.ntiles / 16;
        break;
      default:
        lo = 3 * (int64_t)cus / 4, hi = (int64_t)per_cu * cus,
        want = pl.ntiles / 16;
        break;
    }
    if (lo > hi) lo = hi;
    want = want < lo ? lo : (want > hi ? hi : want);
    g = (int)(want < 1 ? 1 : want);
  }
  if (g > kMaxGrid) g = kMaxGrid;
  int64_t cap = pl.ntiles > 0 ? pl.ntiles : 1;
  if (g > cap) g = (int)cap;
  pl.grid = g;
  return pl;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bn && y < x + an;
}

template <class P>
int launch_threads(const void* fn, int grid, int threads, P params,
                   hipStream_t stream) {
  void* args[] = {&params};
  const hipError_t e =
      hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
  if (e != hipSuccess) {
    debug_hip("kernel launch", e);
    (void)hipGetLastError();
    return LIBTOPK_ERR_HIP;
  }
  return LIBTOPK_OK;
}

template <class P>
int launch(const void* fn, int grid, P params, hipStream_t stream) {
  return launch_threads(fn, grid, kBlock, params, stream);
}

// List capacity: exactly k rounded up to 8 while that is small (the list
// then needs no guards); for k > 32, 32 slots (lists shorter than k, with
// the check of short_list_check).
const void* topk_fn(int k) {
  if (k <= 8) return (const void*)&topk_kernel<8, true, kTileVec>;
  if (k <= 16) return (const void*)&topk_kernel<16, true, kTileVec>;
  if (k <= 24) return (const void*)&topk_kernel<24, true, kTileVec>;
  if (k <= 32) return (const void*)&topk_kernel<32, true, kTileVec>;
  // k > 32: lists of 32 values, shorter than k (see short_list_check).
  return (const void*)&topk_kernel<32, false, kTileVec>;
}

template <bool F32>
const void* topk_kv_fn(int k) {
  if (k <= 8) return (const void*)&topk_kv_kernel<8, true, kTileVec, F32>;
  if (k <= 16) return (const void*)&topk_kv_kernel<16, true, kTileVec, F32>;
  if (k <= 24) return (const void*)&topk_kv_kernel<24, true, kTileVec, F32>;
  if (k <= 32) return (const void*)&topk_kv_kernel<32, true, kTileVec, F32>;
  // k > 32: lists of 32 keys, shorter than k (see kv_lost_check).
  return (const void*)&topk_kv_kernel<32, false, kTileVec, F32>;
}

// Both key-value entry points: values are 32-bit words (int32 or float32
// bits); F32 selects the float order.
int topk_kv(const int32_t* in, int64_t n, int32_t k, int32_t* out_v,
            int64_t* out_i, libtopk_stream_t stream, bool f32) {
  if (!in || !out_v || !out_i) return LIBTOPK_ERR_INVALID;
  if (((uintptr_t)in & 3u) || ((uintptr_t)out_v & 3u) ||
      ((uintptr_t)out_i & 7u))
    return LIBTOPK_ERR_INVALID;
  if (n < 1 || n >= kMaxN) return LIBTOPK_ERR_INVALID;
  if (k < 1 || (int64_t)k > n) return LIBTOPK_ERR_INVALID;
  if (k > LIBTOPK_MAX_K) return LIBTOPK_ERR_UNSUPPORTED;
  if (overlaps(in, (size_t)n * 4, out_v, (size_t)k * 4) ||
      overlaps(in, (size_t)n * 4, out_i, (size_t)k * 8) ||
      overlaps(out_v, (size_t)k * 4, out_i, (size_t)k * 8))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  // With 128-key lists (k > 64) the kernel's registers leave room for one
  // workgroup per CU: a grid of two per CU would run in two rounds
  // (key-value top-100 of 1e8: 138 us against 110 us at one per CU).
  const void* fn = f32 ? topk_kv_fn<true>(k) : topk_kv_fn<false>(k);
  int cus, fit;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
    fit = groups_per_cu(fn);
  }
  const Plan pl = plan(in, n, cus, kGridTopk, fit < 2 ? fit : 2);
  TopkKvParams p;
  p.in = in;
  p.n = n;
  p.head = pl.head;
  p.ntiles = pl.ntiles;
  p.covered = pl.covered;
  p.k = k;
  p.grid = pl.grid;
  p.refresh = refresh_period(k);
  p.cand = sc.kvcand;
  p.heads = sc.kvheads;
  p.kths = sc.kvkths;
  p.ticket = sc.ticket;
  p.epoch = next_epoch(*sc.epochs);
  p.out_v = out_v;
  p.out_i = out_i;
  return launch(fn, pl.grid, p, s);
}

// Inputs from this size on are sampled for a filter threshold (the
// smallest the full sample can read; measured on top-1000 .. top-16384 of
// 3e5 .. 1e7 uniform int32, sampled calls are as fast as the digit passes
// or up to 4x faster).
constexpr int64_t kSampleMinN = (int64_t)kSampleGridMax * kSampleThreads * 4;

// The candidate buffer of radix selection (kCandCap int32) and, after it,
// the published sample lists and their lengths (kSampleGridMax *
// (kNeedMax + 1) int32), allocated
// once per (device, stream) on first use.
int get_rcand(int dev, hipStream_t stream, int** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& sc = g_cache[std::make_pair(dev, (void*)stream)];
  if (!sc.rcand) {
    if (getenv("LIBTOPK_TEST_FAIL_ALLOC")) return LIBTOPK_ERR_NOMEM;
    void* p = nullptr;
    const hipError_t e =
        hipMalloc(&p, (size_t)(kCandCap + kSampleGridMax * (kNeedMax + 1)) *
                          sizeof(int));
    if (e != hipSuccess) {
      debug_hip("hipMalloc(candidates)", e);
      (void)hipGetLastError();
      return LIBTOPK_ERR_NOMEM;
    }
    sc.rcand = (int*)p;
  }
  *out = sc.rcand;
  return LIBTOPK_OK;
}

// The segmented top-k's scratch for inputs of up to n elements: lists of
// the mid-length, medium and huge segments, the units of the huge ones
// with their candidates, maxima and k-th values, four counters, one ticket
// per huge segment plus one, and the plan.  Sized from n (valid offsets
// list at most n / (kSegReg + 1) mid-length, n / (kSegShort + 1) medium
// and n / (kSegWhole + 1) huge segments, and at most n / kSegUnit + huge
// units); grown on demand, the stream
// synchronised before the old area is freed.
struct SegScratch {
  int* med;
  int* mid;
  SegHuge* huge;
  SegUnit* units;
  int* cand;
  int* heads;
  int* kths;
  uint64_t* ctr;
  uint64_t* ticket;
  SegPlan* plan;
  int med_cap, mid_cap, huge_cap, unit_cap;
};

void seg_layout(void* base, int64_t n, SegScratch* s, size_t* bytes) {
  const int64_t nn = n < ((int64_t)1 << 20) ? ((int64_t)1 << 20) : n;
  s->med_cap = (int)(nn / (kSegShort + 1) + 1);
  s->mid_cap = (int)(nn / (kSegReg + 1) + 1);
  s->huge_cap = (int)(nn / (kSegWhole + 1) + 1);
  s->unit_cap = (int)(nn / kSegUnit + s->huge_cap + 1);
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) & ~(size_t)255;
    return (char*)base + o;
  };
  // 1 KiB of slack after the per-unit arrays: stage 2 copies them to LDS in
  // whole KiB chunks.
  s->cand = (int*)take((size_t)s->unit_cap * kMaxK * 4 + 1024);
  s->heads = (int*)take((size_t)s->unit_cap * 4 + 1024);
  s->kths = (int*)take((size_t)s->unit_cap * 4 + 1024);
  s->units = (SegUnit*)take((size_t)s->unit_cap * sizeof(SegUnit));
  s->huge = (SegHuge*)take((size_t)s->huge_cap * sizeof(SegHuge));
  s->med = (int*)take((size_t)s->med_cap * 4);
  s->mid = (int*)take((size_t)s->mid_cap * 4);
  s->plan = (SegPlan*)take(sizeof(SegPlan));
  s->ctr = (uint64_t*)take(4 * 8 + (size_t)(1 + s->huge_cap) * 8);
  s->ticket = s->ctr + 4;
  *bytes = off;
}

int get_seg(int dev, hipStream_t stream, int64_t n, SegScratch* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  Scratch& sc = g_cache[std::make_pair(dev, (void*)stream)];
  size_t bytes = 0;
  if (sc.seg_base && n <= sc.seg_n) {
    seg_layout(sc.seg_base, sc.seg_n, out, &bytes);
    return LIBTOPK_OK;
  }
  if (getenv("LIBTOPK_TEST_FAIL_ALLOC")) return LIBTOPK_ERR_NOMEM;
  const int64_t want = n < ((int64_t)1 << 20) ? ((int64_t)1 << 20) : n;
  seg_layout(nullptr, want, out, &bytes);
  if (sc.seg_base) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(sc.seg_base);
    sc.seg_base = nullptr;
    sc.seg_n = 0;
  }
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    debug_hip("hipMalloc(segments)", e);
    (void)hipGetLastError();
    return LIBTOPK_ERR_NOMEM;
  }
  seg_layout(p, want, out, &bytes);
  // Counters and tickets carry epoch tags; zero is the tidy start.
  const int zwords = (int)((4 + 1 + out->huge_cap) * 2);
  hipLaunchKernelGGL(zero_words, dim3((zwords + 255) / 256), dim3(256), 0,
                     stream, (unsigned*)out->ctr, zwords);
  e = hipGetLastError();
  if (e != hipSuccess) {
    debug_hip("zero_words launch", e);
    (void)hipFree(p);
    return LIBTOPK_ERR_HIP;
  }
  sc.seg_base = p;
  sc.seg_n = want;
  return LIBTOPK_OK;
}

template <int KCAP, bool FIT>
const void* seg_long_fn_of() {
  return (const void*)&seg_long_kernel<KCAP, FIT, kTileVec>;
}
const void* seg_long_fn(int k) {
  if (k <= 8) return seg_long_fn_of<8, true>();
  if (k <= 16) return seg_long_fn_of<16, true>();
  if (k <= 24) return seg_long_fn_of<24, true>();
  if (k <= 32) return seg_long_fn_of<32, true>();
  return seg_long_fn_of<32, false>();
}

// Top-k for LIBTOPK_MAX_K < k <= LIBTOPK_MAX_K_SELECT: four digit passes of
// radix selection (the second of which usually also splits the bucket off
// into the candidate buffer), a gather pass and a one-workgroup sort, all
// stream-ordered launches on the caller's stream.
int topk_select(const int32_t* in, int64_t n, int32_t k, int32_t* out,
                hipStream_t s, int dev, const Scratch& sc, const Plan& pl) {
  int* rcand = nullptr;
  int rc = get_rcand(dev, s, &rcand);
  if (rc != LIBTOPK_OK) return rc;
  SelectParams sp;
  sp.in = in;
  sp.n = n;
  sp.head = pl.head;
  sp.ntiles = pl.ntiles;
  sp.covered = pl.covered;
  sp.grid = pl.grid;
  sp.k = k;
  sp.st = sc.rstate;
  sp.cand = rcand;
  sp.out = out;
  sp.acc = sc.acc;
  sp.ticket = sc.ticket;
  // Large inputs: a sample sets a threshold, and a filter pass copies
  // every value above it aside; one workgroup selects from a small copy,
  // the selection passes from a larger one (or, if the copy cannot hold the
  // top-k, from the input).
  bool filtered = false;
  const int64_t nvec = (n - pl.head) / 4;
  bool sampled = n >= kSampleMinN &&
                 nvec >= (int64_t)kSampleGridMax * kSampleThreads;
  // need = the sample's share of k, plus four standard deviations and 4.
  // The largest sample (grid workgroups of 4096 values) for which each
  // workgroup's list (need values) fits kNeedMax and all of them the last
  // workgroup's kUnionSlots; none at all if even one workgroup's sample
  // asks too much (k too large for n).
  int grid = kSampleGridMax, need = 0;
  while (sampled) {
    const double ks = (double)k * (4.0 * kSampleThreads * grid) / (double)n;
    need = (int)std::ceil(ks + 4.0 * std::sqrt(ks) + 4.0);
    if (need <= kNeedMax && grid * need <= kUnionSlots) break;
    if (grid == 1) sampled = false;
    grid /= 2;
  }
  if (sampled) {
    SampleParams q;
    q.body = reinterpret_cast<const v4i*>(in + pl.head);
    q.nvec = nvec;
    q.grid = grid;
    q.need = need;
    // nvec < 2^31 and S >= kSampleThreads, so i * step < nvec * 2^32 fits.
    q.step = (uint64_t)(((unsigned __int128)nvec << 32) /
                        (uint64_t)((int64_t)grid * kSampleThreads));
    q.st = sc.rstate;
    q.samp = rcand + kCandCap;
    q.samp_cnt = q.samp + kSampleGridMax * kNeedMax;
    q.ticket = sc.ticket;
    q.epoch = next_epoch(*sc.epochs);
    rc = launch_threads((const void*)&sample_kernel, grid, kSampleThreads, q,
                        s);
    if (rc != LIBTOPK_OK) return rc;
    sp.epoch = next_epoch(*sc.epochs);
    rc = launch((const void*)&filter_kernel<kTileVec>, pl.grid, sp, s);
    if (rc != LIBTOPK_OK) return rc;
    filtered = true;
  }
  for (int pass = 0; pass < 4; ++pass) {
    sp.dshift = 24 - 8 * pass;
    sp.first = pass == 0 && !filtered;  // the filter wrote the first state
    sp.epoch = next_epoch(*sc.epochs);
    rc = launch((const void*)&select_pass_kernel<kTileVec>, pl.grid, sp, s);
    if (rc != LIBTOPK_OK) return rc;
  }
  sp.epoch = next_epoch(*sc.epochs);
  rc = launch((const void*)&gather_kernel<kTileVec>, pl.grid, sp, s);
  if (rc != LIBTOPK_OK) return rc;
  return launch_threads((const void*)&select_finish_kernel, 1, kFinThreads,
                        sp, s);
}

const void* reduce_fn(int op) {
  if (op == kOpSum) return (const void*)&reduce_kernel<kOpSum, kTileVec>;
  if (op == kOpMax) return (const void*)&reduce_kernel<kOpMax, kTileVec>;
  return (const void*)&reduce_kernel<kOpMin, kTileVec>;
}

// Workgroups of one kernel that fit on a CU at once (registers, LDS), from
// the runtime's occupancy calculator; at least 1.
int resident_blocks(const void* fn) {
  static std::mutex mu;
  static std::map<const void*, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(fn);
  if (it != cache.end()) return it->second;
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, kBlock, 0) !=
          hipSuccess || b < 1) {
    (void)hipGetLastError();
    b = 1;
  }
  cache[fn] = b;
  return b;
}

// Rows of at most this many elements go one wave per row, the whole row in
// registers (topk_rows_kernel); longer rows stream through topk_kernel.
constexpr int64_t kShortRow = 4096;
// Workgroups per launch of topk_kernel on many rows (later rows go in
// further launches).
constexpr int64_t kMaxLaunchBlocks = (int64_t)1 << 20;

// Elements per lane V: the row length rounded up to 64 V, V from
// {4, 8, 16, 32, 64}.  Rows of exactly 64 V elements that all start on a
// 16-byte boundary take the vector-load variant.
template <int V>
const void* rows_fn_v(bool full) {
  return full ? (const void*)&topk_rows_kernel<V, true>
              : (const void*)&topk_rows_kernel<V, false>;
}

const void* rows_fn(const int32_t* in, int64_t n, int64_t ld) {
  // Rows of at most 64 elements: one per lane, sorted across the wave.
  if (n <= kWave) return (const void*)&topk_rows_kernel<1, false>;
  const int v = n <= 256 ? 4 : n <= 512 ? 8 : n <= 1024 ? 16 : n <= 2048 ? 32
                                                                        : 64;
  const bool full = n == 64 * v && ((uintptr_t)in & 15u) == 0 && ld % 4 == 0;
  switch (v) {
    case 4: return rows_fn_v<4>(full);
    case 8: return rows_fn_v<8>(full);
    case 16: return rows_fn_v<16>(full);
    case 32: return rows_fn_v<32>(full);
    default: return rows_fn_v<64>(full);
  }
}

// Workgroups per row for rows longer than kShortRow: enough workgroups in
// all to give every CU two, but never more than a row has tiles, and few
// enough rows x workgroups for the per-block scratch.  Many rows: one
// workgroup per row, whose own top-k is the row's result.
int row_grid(int64_t rows, int64_t cols, int cus) {
  int target = g_grid_override.load();
  if (target <= 0) target = 2 * cus;
  const int64_t tiles = (cols / 4) / (kBlock * kTileVec);
  if (rows >= target || rows > kMaxGrid || tiles < 2) return 1;
  int64_t g = (target + rows - 1) / rows;
  if (g > tiles) g = tiles;
  if (g > kMaxGrid / rows) g = kMaxGrid / rows;
  return g < 1 ? 1 : (int)g;
}

// ---- scratch of the allocation-free top-k -----------------------------------
// topk_i32_noalloc keeps the stage-1 candidates, block maxima, k-th values
// and tickets of the register-list top-k in one file-scope device array
// instead of the per-stream scratch, so that a call never allocates.  The
// array is sized for the largest grid and list (kMaxGrid x kMaxK), so every
// k <= kMaxK and every n fits.  Each device holds its own copy at its own
// address until the process ends.
struct NoAllocScratch {
  int cand[kMaxGrid * kMaxK];
  int heads[kMaxGrid];
  int kths[kMaxGrid];
  uint64_t ticket[kMaxGrid];  // epoch-tagged (see Tagged in wave.hpp)
};
constexpr size_t kNoAllocBytes = sizeof(NoAllocScratch);
static_assert(kNoAllocBytes == LIBTOPK_NOALLOC_SCRATCH_BYTES,
              "the header states the array's size");

}  // namespace

// The array itself.  In host code its name is only a stand-in for the
// device symbol: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

// Per device: the address of `scratch` and the epochs of its launches.
struct NoAllocState {
  NoAllocScratch* s = nullptr;
  std::atomic<uint32_t> epochs{0u};
};
std::mutex g_noalloc_mu;
std::map<int, std::unique_ptr<NoAllocState>> g_noalloc;

// The device address of `scratch` on device `dev` (current), looked up once
// per device, and its epoch counter.  The first lookup also clears the
// tickets with a fill kernel on the caller's stream (they carry epoch tags,
// so any value would do; zero is the tidy start).  Nothing is allocated on
// the device (the host keeps one small record per device).
int noalloc_scratch(int dev, hipStream_t stream, NoAllocScratch** out,
                    std::atomic<uint32_t>** epochs) {
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  auto it = g_noalloc.find(dev);
  if (it != g_noalloc.end()) {
    *out = it->second->s;
    *epochs = &it->second->epochs;
    return LIBTOPK_OK;
  }
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) {
    debug_hip("hipGetSymbolAddress(scratch)", e);
    (void)hipGetLastError();
    return LIBTOPK_ERR_HIP;
  }
  NoAllocScratch* s = (NoAllocScratch*)ptr;
  const int zwords = (int)(sizeof(s->ticket) / 4);
  hipLaunchKernelGGL(zero_words, dim3((zwords + 255) / 256), dim3(256), 0,
                     stream, (unsigned*)s->ticket, zwords);
  e = hipGetLastError();
  if (e != hipSuccess) {
    debug_hip("zero_words launch", e);
    return LIBTOPK_ERR_HIP;
  }
  std::unique_ptr<NoAllocState> st(new NoAllocState);
  st->s = s;
  *out = s;
  *epochs = &st->epochs;
  g_noalloc[dev] = std::move(st);
  return LIBTOPK_OK;
}

}  // namespace

extern "C" {

int topk_i32_noalloc(const int32_t* in, int64_t n, int32_t k, int32_t* out,
                     libtopk_stream_t stream) {
  if (!in || !out) return LIBTOPK_ERR_INVALID;
  if (((uintptr_t)in & 3u) || ((uintptr_t)out & 3u)) return LIBTOPK_ERR_INVALID;
  if (n < 1 || n > kMaxN) return LIBTOPK_ERR_INVALID;
  if (k < 1 || (int64_t)k > n) return LIBTOPK_ERR_INVALID;
  // Radix selection (k > LIBTOPK_MAX_K) needs megabytes of candidates: not
  // in the fixed array.
  if (k > LIBTOPK_MAX_K) return LIBTOPK_ERR_UNSUPPORTED;
  if (overlaps(in, (size_t)n * 4, out, (size_t)k * 4))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  NoAllocScratch* sc = nullptr;
  std::atomic<uint32_t>* epochs = nullptr;
  rc = noalloc_scratch(dev, s, &sc, &epochs);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  const Plan pl = plan(in, n, cus);
  TopkParams p;
  p.in = in;
  p.n = n;
  p.ld = n;  // one row
  p.k = k;
  p.grid = pl.grid;
  p.refresh = refresh_period(k);
  p.cand = sc->cand;
  p.heads = sc->heads;
  p.kths = sc->kths;
  p.ticket = sc->ticket;
  p.epoch = next_epoch(*epochs);
  p.out = out;
  return launch(topk_fn(k), pl.grid, p, s);
}

int topk_i32(const int32_t* in, int64_t n, int32_t k, int32_t* out,
             libtopk_stream_t stream) {
  if (!in || !out) return LIBTOPK_ERR_INVALID;
  if (((uintptr_t)in & 3u) || ((uintptr_t)out & 3u)) return LIBTOPK_ERR_INVALID;
  if (n < 1 || n > kMaxN) return LIBTOPK_ERR_INVALID;
  if (k < 1 || (int64_t)k > n) return LIBTOPK_ERR_INVALID;
  if (k > LIBTOPK_MAX_K_SELECT) return LIBTOPK_ERR_UNSUPPORTED;
  if (overlaps(in, (size_t)n * 4, out, (size_t)k * 4))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  if (k > LIBTOPK_MAX_K)
    return topk_select(in, n, k, out, s, dev, sc,
                       plan(in, n, cus, kGridSelect));
  const Plan pl = plan(in, n, cus);
  TopkParams p;
  p.in = in;
  p.n = n;
  p.ld = n;  // one row
  p.k = k;
  p.grid = pl.grid;
  p.refresh = refresh_period(k);
  p.cand = sc.cand;
  p.heads = sc.heads;
  p.kths = sc.kths;
  p.ticket = sc.ticket;
  p.epoch = next_epoch(*sc.epochs);
  p.out = out;
  return launch(topk_fn(k), pl.grid, p, s);
}

int reduce_i32(const int32_t* in, int64_t n, int32_t op, int64_t* out_i64,
               libtopk_stream_t stream) {
  if (!out_i64 || ((uintptr_t)out_i64 & 7u)) return LIBTOPK_ERR_INVALID;
  if (n < 0 || n > kMaxN) return LIBTOPK_ERR_INVALID;
  if (n > 0 && (!in || ((uintptr_t)in & 3u))) return LIBTOPK_ERR_INVALID;
  if (op < LIBTOPK_SUM || op > LIBTOPK_MIN) return LIBTOPK_ERR_INVALID;
  if (n > 0 && overlaps(in, (size_t)n * 4, out_i64, 8))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  // n == 0: a one-block launch with nothing to read writes the identity.
  static const int32_t kDummy = 0;
  const Plan pl = plan(n > 0 ? in : &kDummy, n, cus, kGridReduce);
  ReduceParams p;
  p.in = in;
  p.n = n;
  p.head = pl.head;
  p.ntiles = pl.ntiles;
  p.covered = pl.covered;
  p.grid = pl.grid;
  p.partials = sc.partials;
  p.ticket = sc.ticket;
  p.epoch = next_epoch(*sc.epochs);
  p.out = out_i64;
  return launch(reduce_fn(op), pl.grid, p, s);
}

int topk_kv_i32(const int32_t* in, int64_t n, int32_t k, int32_t* out_values,
                int64_t* out_indices, libtopk_stream_t stream) {
  return topk_kv(in, n, k, out_values, out_indices, stream, false);
}

int topk_kv_f32(const float* in, int64_t n, int32_t k, float* out_values,
                int64_t* out_indices, libtopk_stream_t stream) {
  return topk_kv(reinterpret_cast<const int32_t*>(in), n, k,
                 reinterpret_cast<int32_t*>(out_values), out_indices, stream,
                 true);
}

int reduce_stats_i32(const int32_t* in, int64_t n, int64_t* out,
                     libtopk_stream_t stream) {
  if (!out || ((uintptr_t)out & 7u)) return LIBTOPK_ERR_INVALID;
  if (n < 0 || n > kMaxN) return LIBTOPK_ERR_INVALID;
  if (n > 0 && (!in || ((uintptr_t)in & 3u))) return LIBTOPK_ERR_INVALID;
  if (n > 0 && overlaps(in, (size_t)n * 4, out, 6 * 8))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  // n == 0: a one-block launch with nothing to read writes the identities.
  static const int32_t kDummy = 0;
  const Plan pl = plan(n > 0 ? in : &kDummy, n, cus, kGridReduce);
  StatsParams p;
  p.in = in;
  p.n = n;
  p.head = pl.head;
  p.ntiles = pl.ntiles;
  p.covered = pl.covered;
  p.grid = pl.grid;
  p.partials = sc.spart;
  p.ticket = sc.ticket;
  p.epoch = next_epoch(*sc.epochs);
  p.out = out;
  return launch((const void*)&stats_kernel<kTileVec>, pl.grid, p, s);
}

int topk_batched_i32(const int32_t* in, int64_t rows, int64_t cols,
                     int64_t ld, int32_t k, int32_t* out,
                     libtopk_stream_t stream) {
  if (rows < 0 || cols < 1 || cols > kMaxN || ld < cols)
    return LIBTOPK_ERR_INVALID;
  if (k < 1 || (int64_t)k > cols) return LIBTOPK_ERR_INVALID;
  if (k > LIBTOPK_MAX_K) return LIBTOPK_ERR_UNSUPPORTED;
  if (rows == 0) return LIBTOPK_OK;
  if (!in || !out) return LIBTOPK_ERR_INVALID;
  if (((uintptr_t)in & 3u) || ((uintptr_t)out & 3u)) return LIBTOPK_ERR_INVALID;
  // The input spans (rows - 1) * ld + cols elements: keep byte sizes far
  // from overflow.
  const int64_t kSpanMax = (int64_t)1 << 60;
  if (rows - 1 > (kSpanMax - cols) / ld || rows > kSpanMax / k)
    return LIBTOPK_ERR_INVALID;
  const size_t in_bytes = (size_t)((rows - 1) * ld + cols) * 4;
  if (overlaps(in, in_bytes, out, (size_t)(rows * k) * 4))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  if (cols <= kShortRow) {
    RowsParams p;
    p.in = in;
    p.rows = rows;
    p.ld = ld;
    p.n = (int)cols;
    p.k = k;
    p.out = out;
    // Exactly as many workgroups as fit on the device at once: each wave
    // then walks its share of the rows to the end, with no second, partly
    // filled round of workgroups.
    const void* fn = rows_fn(in, cols, ld);
    const int64_t want = (rows + kWaves - 1) / kWaves;
    const int64_t slots = (int64_t)resident_blocks(fn) * cus;
    const int grid = (int)(want < slots ? want : slots);
    return launch(fn, grid, p, s);
  }
  const int gr = row_grid(rows, cols, cus);
  TopkParams p;
  p.n = cols;
  p.ld = ld;
  p.k = k;
  p.grid = gr;
  p.refresh = refresh_period(k);
  p.cand = sc.cand;
  p.heads = sc.heads;
  p.kths = sc.kths;
  p.ticket = sc.ticket;
  const int64_t per_launch = kMaxLaunchBlocks / gr;
  for (int64_t r0 = 0; r0 < rows; r0 += per_launch) {
    const int64_t nr = rows - r0 < per_launch ? rows - r0 : per_launch;
    p.in = in + r0 * ld;
    p.out = out + r0 * k;
    p.epoch = next_epoch(*sc.epochs);
    rc = launch(topk_fn(k), (int)(nr * gr), p, s);
    if (rc != LIBTOPK_OK) return rc;
  }
  return LIBTOPK_OK;
}

int topk_merge_i32(const int32_t* lists, int64_t m, int32_t len, int32_t k,
                   int32_t* out, libtopk_stream_t stream) {
  if (!lists || !out) return LIBTOPK_ERR_INVALID;
  if (((uintptr_t)lists & 3u) || ((uintptr_t)out & 3u))
    return LIBTOPK_ERR_INVALID;
  if (m < 1 || m > (int64_t)kMaxGrid * kMaxGrid || len < 1)
    return LIBTOPK_ERR_INVALID;
  if (k < 1 || (int64_t)k > m * len) return LIBTOPK_ERR_INVALID;
  if (k > LIBTOPK_MAX_K) return LIBTOPK_ERR_UNSUPPORTED;
  if (overlaps(lists, (size_t)(m * len) * 4, out, (size_t)k * 4))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  MergeParams p;
  p.lists = lists;
  p.m = m;
  p.len = len;
  p.k = k;
  p.groups = (int)((m + kMaxGrid - 1) / kMaxGrid);
  p.cand = sc.cand;
  p.ticket = sc.ticket;
  p.epoch = next_epoch(*sc.epochs);
  p.out = out;
  return launch((const void*)&topk_merge_kernel, p.groups, p, s);
}

int topk_segmented_i32(const int32_t* in, int64_t n, const int64_t* offsets,
                       int64_t nseg, int32_t k, int32_t* out, int32_t* counts,
                       libtopk_stream_t stream) {
  if (n < 0 || n > kMaxN || nseg < 0 || nseg > (int64_t)INT32_MAX - 1)
    return LIBTOPK_ERR_INVALID;
  if (k < 1) return LIBTOPK_ERR_INVALID;
  if (k > LIBTOPK_MAX_K) return LIBTOPK_ERR_UNSUPPORTED;
  if (nseg == 0) return LIBTOPK_OK;
  if (!offsets || ((uintptr_t)offsets & 7u)) return LIBTOPK_ERR_INVALID;
  if (!out || ((uintptr_t)out & 3u)) return LIBTOPK_ERR_INVALID;
  if (counts && ((uintptr_t)counts & 3u)) return LIBTOPK_ERR_INVALID;
  if (n > 0 && (!in || ((uintptr_t)in & 3u))) return LIBTOPK_ERR_INVALID;
  const size_t out_b = (size_t)(nseg * k) * 4, off_b = (size_t)(nseg + 1) * 8;
  if (overlaps(out, out_b, offsets, off_b) ||
      (n > 0 && overlaps(out, out_b, in, (size_t)n * 4)))
    return LIBTOPK_ERR_INVALID;
  if (counts && (overlaps(counts, (size_t)nseg * 4, out, out_b) ||
                 overlaps(counts, (size_t)nseg * 4, offsets, off_b) ||
                 (n > 0 && overlaps(counts, (size_t)nseg * 4, in,
                                    (size_t)n * 4))))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  SegScratch ss;
  rc = get_seg(dev, s, n, &ss);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  SegParams p;
  p.in = in;
  p.n = n;
  p.in_mis = (int)(((uintptr_t)in & 15u) >> 2);
  p.offsets = offsets;
  p.nseg = nseg;
  p.k = k;
  p.refresh = refresh_period(k);
  p.out = out;
  p.counts = counts;
  p.med = ss.med;
  p.med_cap = ss.med_cap;
  p.mid = ss.mid;
  p.mid_cap = ss.mid_cap;
  p.huge = ss.huge;
  p.huge_cap = ss.huge_cap;
  p.units = ss.units;
  p.unit_cap = ss.unit_cap;
  p.cand = ss.cand;
  p.heads = ss.heads;
  p.kths = ss.kths;
  p.ctr = ss.ctr;
  p.ticket = ss.ticket;
  p.plan = ss.plan;
  p.seg_tag = next_epoch(*sc.seg_calls);
  // 1. One wave per segment: the short ones done, the others listed and
  // planned.
  // Many short segments on average: the lean short kernel (see
  // seg_short_kernel).
  const bool lean = n < kSegReg * nseg;
  const void* sfn = lean ? (const void*)&seg_short_kernel<true>
                         : (const void*)&seg_short_kernel<false>;
  const int64_t want = (nseg + kWaves - 1) / kWaves;
  int64_t slots = (int64_t)resident_blocks(sfn) * cus;
  // Few segments (fewer than 8 per wave at one workgroup per CU): every
  // workgroup's ticket (they serialise) costs more than its segments gain
  // from more waves, so one workgroup per CU (log-uniform lengths in
  // [16, 2^18] over 1e8, 3,967 segments: 122 -> 115 us; 5,000 segments of
  // 20,000: 149 -> 133 us).  With more, more waves hide the segments'
  // latency (20,000 segments of 1,000 .. 4,096 elements: 64 us, 95 with
  // the cap).
  if (nseg < 32 * (int64_t)cus && slots > cus) slots = cus;
  p.epoch = next_epoch(*sc.epochs);
  rc = launch(sfn, (int)(want < slots ? want : slots), p, s);
  if (rc != LIBTOPK_OK) return rc;
  // 2. Persistent workgroups over the plan's work items.
  const void* lfn = seg_long_fn(k);
  p.epoch = next_epoch(*sc.epochs);
  return launch(lfn, resident_blocks(lfn) * cus, p, s);
}

int histogram_i32(const int32_t* in, int64_t n, int32_t lo, int32_t shift,
                  int32_t nbins, int64_t* out, libtopk_stream_t stream) {
  if (!out || ((uintptr_t)out & 7u)) return LIBTOPK_ERR_INVALID;
  if (n < 0 || n > kMaxN) return LIBTOPK_ERR_INVALID;
  if (n > 0 && (!in || ((uintptr_t)in & 3u))) return LIBTOPK_ERR_INVALID;
  if (shift < 0 || shift > 31 || nbins < 1 || nbins > LIBTOPK_MAX_BINS)
    return LIBTOPK_ERR_INVALID;
  if (n > 0 && overlaps(in, (size_t)n * 4, out, (size_t)nbins * 8))
    return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  Scratch sc;
  rc = get_scratch(dev, s, &sc);
  if (rc != LIBTOPK_OK) return rc;
  int cus;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  // n == 0: a one-block launch with nothing to read writes zero counts.
  static const int32_t kDummy = 0;
  const Plan pl = plan(n > 0 ? in : &kDummy, n, cus, kGridHist);
  HistParams p;
  p.in = in;
  p.n = n;
  p.head = pl.head;
  p.ntiles = pl.ntiles;
  p.covered = pl.covered;
  p.grid = pl.grid;
  p.lo = lo;
  p.shift = shift;
  p.nbins = nbins;
  p.out = out;
  p.acc = sc.acc;
  p.ticket = sc.ticket;
  p.epoch = next_epoch(*sc.epochs);
  return launch((const void*)&hist_kernel<kTileVec>, pl.grid, p, s);
}

int libtopk_debug_scramble(libtopk_stream_t stream, int32_t which,
                           uint64_t seed) {
  if (which != 0 && which != 1) return LIBTOPK_ERR_INVALID;
  int dev = 0;
  int rc = current_device(&dev);
  if (rc != LIBTOPK_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  uint64_t* words[3];
  int counts[3];
  int parts = 0;
  if (which == 0) {
    Scratch sc;
    rc = get_scratch(dev, s, &sc);
    if (rc != LIBTOPK_OK) return rc;
    words[0] = sc.ticket;
    counts[0] = kMaxGrid;
    words[1] = sc.acc;
    counts[1] = kMaxBins;
    parts = 2;
    {
      std::lock_guard<std::mutex> lock(g_mu);
      const Scratch& cur = g_cache[std::make_pair(dev, (void*)s)];
      if (cur.seg_base) {
        // the segmented top-k's counters and tickets
        SegScratch ss;
        size_t bytes = 0;
        seg_layout(cur.seg_base, cur.seg_n, &ss, &bytes);
        words[2] = ss.ctr;
        counts[2] = 4 + 1 + ss.huge_cap;
        parts = 3;
      }
    }
  } else {
    NoAllocScratch* sc = nullptr;
    std::atomic<uint32_t>* epochs = nullptr;
    rc = noalloc_scratch(dev, s, &sc, &epochs);
    if (rc != LIBTOPK_OK) return rc;
    words[0] = sc->ticket;
    counts[0] = kMaxGrid;
    parts = 1;
  }
  for (int i = 0; i < parts; ++i) {
    hipLaunchKernelGGL(scramble_words, dim3((counts[i] + 255) / 256),
                       dim3(256), 0, s, words[i], counts[i],
                       seed + 0x632be59bd9b4e019ull * (uint64_t)i);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      debug_hip("scramble_words launch", e);
      return LIBTOPK_ERR_HIP;
    }
  }
  return LIBTOPK_OK;
}

const char* libtopk_strerror(int status) {
  switch (status) {
    case LIBTOPK_OK: return "success";
    case LIBTOPK_ERR_INVALID: return "invalid argument";
    case LIBTOPK_ERR_UNSUPPORTED: return "k above the supported maximum";
    case LIBTOPK_ERR_NOMEM: return "scratch allocation failed";
    case LIBTOPK_ERR_HIP: return "no HIP device, or a HIP call failed";
    default: return "unknown status";
  }
}

int libtopk_max_k(void) { return LIBTOPK_MAX_K; }

int libtopk_set_grid(int32_t blocks) {
  if (blocks < 0 || blocks > kMaxGrid) return LIBTOPK_ERR_INVALID;
  g_grid_override.store(blocks);
  return LIBTOPK_OK;
}

int32_t libtopk_grid_for(int64_t n) {
  if (n < 1) return 0;
  int cus = 256;
  int dev = 0;
  if (current_device(&dev) == LIBTOPK_OK) {
    std::lock_guard<std::mutex> lock(g_mu);
    cus = compute_units(dev);
  }
  // The grid depends on the alignment only through the head peel (< 4
  // elements); report it for a 16-byte-aligned input.
  return plan((const int32_t*)(uintptr_t)0x1000, n, cus).grid;
}

void libtopk_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int prev = -1;
  (void)hipGetDevice(&prev);
  for (auto& kv : g_cache) {
    if (hipSetDevice(kv.first.first) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(kv.second.base);
      if (kv.second.rcand) (void)hipFree(kv.second.rcand);
      if (kv.second.seg_base) (void)hipFree(kv.second.seg_base);
    }
  }
  g_cache.clear();
  if (prev >= 0) (void)hipSetDevice(prev);
  (void)hipGetLastError();
}

}  // extern "C"
