// Segmented Top-K: the k largest values of every segment of one array,
// segments of any lengths given by offsets in device memory.
//
// Sources:
//   [TopK] "CUDA并行优化实战：从TopK问题剖析共享内存与规约算法设计"
//          §6 (the two-stage pattern as a building block: candidate
//          selection per user, whose candidate lists differ in length;
//          several TopK results merged again) and §2 (each segment is
//          reduced by the two stages: per-thread lists, a block merge, and
//          for a long segment a second stage over its blocks' candidates).
//
// Segment s is in[offsets[s] .. offsets[s+1]) (clamped to [0, n]; an end
// before the start is an empty segment).  Its result is out[s*k ..
// s*k + k): its min(k, len) largest values in descending order, then
// INT_MIN in the slots a short segment cannot fill; counts[s] = min(k, len).
//
// gfx950 design.  The offsets live on the device, so the host cannot plan
// per segment; two launches plan and work on the device instead:
//  1. seg_short_kernel, one wave per segment (segments dealt to the waves
//     in order).  A segment of at most kSegReg elements is read into the
//     wave's registers (V elements per lane, V picked by its length) and
//     finished there by the short-row machinery of topk_rows_kernel.hpp;
//     so are segments up to kSegShort elements, unless the segments are
//     many and short on average: then those are listed as "mid-length" for
//     a wave of the next kernel each (see seg_short_kernel).  Longer
//     segments are only listed: up to kSegWhole elements as
//     "medium" (one workgroup will stream the whole segment), beyond that
//     as "huge".  The last workgroup to finish (epoch-tagged ticket) cuts
//     each huge segment into units of about kSegUnit elements (whole tiles,
//     16-byte aligned from the second unit on, at most kMaxGrid of them)
//     and writes the work plan.
//  2. seg_long_kernel, persistent workgroups: first the mid-length
//     segments, one wave each, then work items from an epoch-tagged
//     counter: the huge units, then the medium segments.
//     A workgroup streams its item with the stage-1 machinery of
//     topk_kernel (workgroup_topk).  A medium segment's top-k is its
//     result.  A huge unit's top-k goes to scratch with its max and k-th;
//     the last unit of a segment to finish (per-segment ticket) merges the
//     segment's units by topk_kernel's stage 2.
// Offsets out of order cannot make either kernel read or write outside the
// buffers: lists and units are capped by the scratch sizes, and a segment
// whose work did not fit is left unwritten (its result is then
// unspecified, as the interface says).
#pragma once

#include "hist_kernel.hpp"  // wave_scan_incl
#include "topk_kernel.hpp"
#include "topk_rows_kernel.hpp"

namespace ltk {

constexpr int64_t kSegShort = 4096;         // one wave, in registers
constexpr int64_t kSegReg = 1024;           // ... in seg_short_kernel<true>
constexpr int64_t kSegWhole = 1 << 17;      // one workgroup, whole segment
constexpr int64_t kSegUnit = 1 << 18;       // a huge segment's units
constexpr int kSegStageMed = 64;            // per-wave LDS staging of the
constexpr int kSegStageHuge = 16;           // listed segments
constexpr int64_t kSegTile = kBlock * 16;   // elements in one stage-1 tile

struct SegUnit {   // one unit of a huge segment
  int64_t start;   // first element
  int32_t len;
  int32_t j;       // the huge segment it belongs to
};
struct SegHuge {   // one huge segment
  int32_t seg;     // its index
  int32_t base;    // its first unit
  int32_t units;   // how many
  int32_t pad;
};
struct SegPlan {   // written by seg_short_kernel's last workgroup
  int32_t m_med;   // medium segments listed
  int32_t units;   // units of the huge segments
  int32_t total;   // work items of seg_long_kernel: units + m_med
  int32_t m_mid;   // mid-length segments listed (one wave each)
};

struct SegParams {
  const int* in;
  int64_t n;
  int in_mis;               // (in & 15) / 4: elements before a 16-byte line
  const int64_t* offsets;   // [nseg + 1]
  int64_t nseg;
  int k;
  int refresh;              // bound refresh period of the stage-1 stream
  int* out;                 // [nseg * k]
  int* counts;              // [nseg] or null
  int* med;                 // [med_cap] medium segment indices
  int med_cap;
  int* mid;                 // [mid_cap] mid-length segment indices
  int mid_cap;
  SegHuge* huge;            // [huge_cap]
  int huge_cap;
  SegUnit* units;           // [unit_cap]
  int unit_cap;
  int* cand;                // [unit_cap * k] per unit: its top-k
  int* heads;               // [unit_cap] per unit: its max
  int* kths;                // [unit_cap] per unit: its k-th
  uint64_t* ctr;            // [4] tagged with seg_tag: medium, huge,
                            // work, mid-length
  uint32_t seg_tag;         // this call's: one more than the previous
                            // segmented call's on the same scratch
  uint64_t* ticket;         // [1 + huge_cap]: seg_short_kernel's, then one
                            // per huge segment
  SegPlan* plan;
  uint32_t epoch;           // this launch's
};

// Segment s's bounds, clamped into [0, n] with the end not before the start.
__device__ __forceinline__ void seg_bounds(const SegParams& p, int64_t s,
                                           int64_t& a, int64_t& b) {
  a = p.offsets[s];
  b = p.offsets[s + 1];
  a = a < 0 ? 0 : (a > p.n ? p.n : a);
  b = b < a ? a : (b > p.n ? p.n : b);
}

// The top-k of a short segment (1 <= len <= 64 V, kk = min(k, len)) in the
// wave's registers: lane l holds elements l, l + 64, ... (loads clamped to
// the segment, padding INT_MIN).
template <int V>
__device__ __forceinline__ void seg_short_topk(const int* src, int len,
                                               int kk, int* dst,
                                               RowsWaveLds& L) {
  int nn = len;
  asm volatile("" : "+s"(nn));  // keep the clamped addresses in the loop
  int x[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int idx = lane() + kWave * j;
    const int v = __builtin_nontemporal_load(src + (idx < nn ? idx : nn - 1));
    x[j] = idx < nn ? v : kI32Min;
  }
  row_topk<V, false>(x, len, kk, dst, L);
}

// Issue the loads of a segment of at most 256 elements (four per lane,
// clamped to the segment) without waiting for them: x holds the raw
// values, to be masked (seg_mask4) where they are used.  Nothing is read
// for an empty or longer segment.
__device__ __forceinline__ void seg_prefetch4(const int* in, int64_t a,
                                              int64_t b, int (&x)[4]) {
  const int64_t len = b - a;
  if (len > 0 && len <= 4 * kWave) {
    const int nn = (int)len;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = lane() + kWave * j;
      x[j] = __builtin_nontemporal_load(in + a + (idx < nn ? idx : nn - 1));
    }
  }
}

__device__ __forceinline__ void seg_mask4(int (&x)[4], int n) {
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = lane() + kWave * j < n ? x[j] : kI32Min;
}

typedef Tagged<32> SegCount;

// Append a wave's n staged segment indices to a device list (entry i at
// dst[i * stride], i < cap) with one tagged atomic (lane 0), then the
// entries by the lanes.  Wave-uniform.
__device__ __forceinline__ void seg_flush(uint64_t* ctr, uint32_t tag,
                                          const int* stage, int n, int* dst,
                                          int stride, int cap) {
  __builtin_amdgcn_wave_barrier();
  uint64_t base = 0;
  if (lane() == 0) base = SegCount::add(ctr, (uint64_t)n, tag);
  base = ((uint64_t)uni((unsigned)(base >> 32)) << 32) | uni((unsigned)base);
  for (int i = lane(); i < n; i += kWave)
    if (base + i < (uint64_t)cap) st_agent(dst + (base + i) * stride, stage[i]);
  __builtin_amdgcn_wave_barrier();
}

// LEAN (chosen by the host for inputs of many short segments: an average
// below kSegReg elements): segments of kSegReg .. kSegShort elements are
// listed for seg_long_kernel instead of held in registers here, so this
// kernel needs less than half the registers and runs 5 waves per SIMD
// instead of 2, which hide the memory latency of the many segments each
// wave visits in turn; segments of at most 64 elements are sorted across
// the wave directly (1e6 segments of 30 elements: 992 us, 567 with the
// lean instance, 404 with the direct sort).  Otherwise every segment up
// to kSegShort elements is finished here.
template <bool LEAN>
__global__ __launch_bounds__(kBlock) void seg_short_kernel(SegParams p) {
  __shared__ RowsWaveLds lds[kWaves];
  __shared__ int mstage[kWaves][kSegStageMed];
  __shared__ int hstage[kWaves][kSegStageHuge];
  __shared__ int dstage[kWaves][kSegStageMed];
  __shared__ int scan[kWaves];
  __shared__ int staged[3][kWaves];
  __shared__ uint64_t lbase[3];
  __shared__ int is_last;
  const int w = threadIdx.x / kWave;
  RowsWaveLds& L = lds[w];
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  const int k = p.k;
  // Staged medium, huge and mid-length segments (uniform).
  int mcnt = 0, hcnt = 0, dcnt = 0;
  // Software pipeline over the wave's segments s, s + W, s + 2W, ...: while
  // segment s is worked on, the bounds of s + 2W and, when it has at most
  // 256 elements, the data of s + W are in flight.
  int64_t s = uni((int)(blockIdx.x * kWaves + w));
  int64_t a0 = 0, b0 = 0, a1 = 0, b1 = 0;
  if (s < p.nseg) seg_bounds(p, s, a0, b0);
  if (s + nwaves < p.nseg) seg_bounds(p, s + nwaves, a1, b1);
  int x0[4] = {kI32Min, kI32Min, kI32Min, kI32Min};
  seg_prefetch4(p.in, a0, b0, x0);
  for (; s < p.nseg; s += nwaves) {
    int64_t a2 = 0, b2 = 0;
    if (s + 2 * nwaves < p.nseg) seg_bounds(p, s + 2 * nwaves, a2, b2);
    int x1[4] = {kI32Min, kI32Min, kI32Min, kI32Min};
    seg_prefetch4(p.in, a1, b1, x1);
    const int64_t a = a0, b = b0;
    const int64_t len = b - a;
    if (len > kSegShort) {
      // Listed in the wave's LDS stage; a full stage goes out at once.
      if (len > kSegWhole) {
        if (lane() == 0) hstage[w][hcnt] = (int)s;
        if (++hcnt == kSegStageHuge) {
          seg_flush(p.ctr + 1, p.seg_tag, hstage[w], hcnt, &p.huge[0].seg,
                    4, p.huge_cap);
          hcnt = 0;
        }
      } else {
        if (lane() == 0) mstage[w][mcnt] = (int)s;
        if (++mcnt == kSegStageMed) {
          seg_flush(p.ctr, p.seg_tag, mstage[w], mcnt, p.med, 1, p.med_cap);
          mcnt = 0;
        }
      }
    } else if (LEAN && len > kSegReg) {
      // Mid-length: one wave of seg_long_kernel takes it (this kernel keeps
      // the registers of segments up to kSegReg only, for occupancy).
      if (lane() == 0) dstage[w][dcnt] = (int)s;
      if (++dcnt == kSegStageMed) {
        seg_flush(p.ctr + 3, p.seg_tag, dstage[w], dcnt, p.mid, 1, p.mid_cap);
        dcnt = 0;
      }
    } else {
      const int n = (int)len;
      const int kk = n < k ? n : k;
      int* dst = p.out + s * k;
      if (n > 0) {
        const int* src = p.in + a;
        if (n <= 256) {
          seg_mask4(x0, n);
          if (LEAN && n <= kWave)
            tiny_row_topk(x0[0], n, kk, dst);
          else
            row_topk<4, false>(x0, n, kk, dst, L);
        } else if (n <= 512) {
          seg_short_topk<8>(src, n, kk, dst, L);
        } else if (LEAN || n <= 1024) {
          seg_short_topk<16>(src, n, kk, dst, L);
        } else if (n <= 2048) {
          seg_short_topk<32>(src, n, kk, dst, L);
        } else {
          seg_short_topk<64>(src, n, kk, dst, L);
        }
      }
      for (int i = kk + lane(); i < k; i += kWave) dst[i] = kI32Min;
      if (p.counts && lane() == 0) p.counts[s] = kk;
    }
    a0 = a1;
    b0 = b1;
    a1 = a2;
    b1 = b2;
#pragma unroll
    for (int j = 0; j < 4; ++j) x0[j] = x1[j];
  }
  // What the waves still hold goes out with one atomic per list for the
  // whole workgroup.
  if (lane() == 0) {
    staged[0][w] = mcnt;
    staged[1][w] = hcnt;
    staged[2][w] = dcnt;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    // List 0 counts in ctr[0], list 1 in ctr[1], list 2 in ctr[3].
    const int l = threadIdx.x;
    int tot = 0;
    for (int v = 0; v < kWaves; ++v) tot += staged[l][v];
    lbase[l] = tot ? SegCount::add(p.ctr + (l == 2 ? 3 : l), (uint64_t)tot,
                                   p.seg_tag)
                   : 0;
  }
  __syncthreads();
  {
    uint64_t mb = lbase[0], hb = lbase[1], db = lbase[2];
    for (int v = 0; v < w; ++v) {
      mb += staged[0][v];
      hb += staged[1][v];
      db += staged[2][v];
    }
    for (int i = lane(); i < mcnt; i += kWave)
      if (mb + i < (uint64_t)p.med_cap) st_agent(p.med + mb + i, mstage[w][i]);
    for (int i = lane(); i < hcnt; i += kWave)
      if (hb + i < (uint64_t)p.huge_cap)
        st_agent(&p.huge[hb + i].seg, hstage[w][i]);
    for (int i = lane(); i < dcnt; i += kWave)
      if (db + i < (uint64_t)p.mid_cap) st_agent(p.mid + db + i, dstage[w][i]);
  }

  // ---- the last workgroup plans the long segments -----------------------
  if (!last_to_finish(p.ticket, gridDim.x, p.epoch, &is_last)) return;
  const int tid = threadIdx.x;
  int m_med = (int)min(SegCount::count(ld_agent(p.ctr), p.seg_tag),
                       (uint64_t)p.med_cap);
  int m_huge = (int)min(SegCount::count(ld_agent(p.ctr + 1), p.seg_tag),
                        (uint64_t)p.huge_cap);
  const int m_mid = (int)min(SegCount::count(ld_agent(p.ctr + 3), p.seg_tag),
                             (uint64_t)p.mid_cap);
  __syncthreads();  // every thread has read the counts
  if (tid == 0) {
    st_agent(p.ctr, SegCount::armed(p.seg_tag + 1u));
    st_agent(p.ctr + 1, SegCount::armed(p.seg_tag + 1u));
    st_agent(p.ctr + 3, SegCount::armed(p.seg_tag + 1u));
  }
  // Units of each huge segment: c0 = ceil(len / kSegUnit) capped at
  // kMaxGrid, chunk = len / c0 rounded up to whole tiles.  Unit 0 starts
  // at the segment's start; unit c >= 1 at a0 + c * chunk, where a0 is the
  // first element at or after the start on a 16-byte boundary, so every
  // unit but the first streams aligned tiles and only the last has a tail.
  int base = 0;  // units so far (uniform)
  for (int j0 = 0; j0 < m_huge; j0 += kBlock) {
    const int j = j0 + tid;
    int units = 0;
    int s = 0;
    int64_t a = 0, b = 0, a0 = 0, chunk = 1;
    if (j < m_huge) {
      s = ld_agent(&p.huge[j].seg);
      seg_bounds(p, s, a, b);
      const int64_t len = b - a;
      int64_t c0 = (len + kSegUnit - 1) / kSegUnit;
      if (c0 > kMaxGrid) c0 = kMaxGrid;
      chunk = (len + c0 - 1) / c0;
      chunk = (chunk + kSegTile - 1) / kSegTile * kSegTile;
      a0 = a + ((4 - ((p.in_mis + a) & 3)) & 3);
      // ceil((b - a0) / chunk) units, at most c0
      units = a0 + chunk >= b ? 1 : (int)((b - a0 + chunk - 1) / chunk);
    }
    // Exclusive scan of the unit counts over the workgroup.
    const int incl_w = wave_scan_incl(units);
    if (lane() == kWave - 1) scan[w] = incl_w;
    __syncthreads();
    int before = base;
    for (int v = 0; v < w; ++v) before += scan[v];
    before += incl_w - units;
    int tot = 0;
    for (int v = 0; v < kWaves; ++v) tot += scan[v];
    __syncthreads();  // scan[] is rewritten by the next round
    if (j < m_huge) {
      // Units past the scratch are dropped (only offsets out of order can
      // ask for that many); the segment then never completes.
      SegHuge h;
      h.seg = s;
      h.base = before;
      h.units = units;
      h.pad = 0;
      p.huge[j] = h;
      for (int c = 0; c < units; ++c) {
        const int u = before + c;
        if (u >= p.unit_cap) break;
        SegUnit e;
        e.start = c == 0 ? a : a0 + c * chunk;
        const int64_t end = a0 + (c + 1) * chunk;
        e.len = (int32_t)((end < b ? end : b) - e.start);
        e.j = j;
        p.units[u] = e;
      }
    }
    base += tot;
  }
  if (tid == 0) {
    SegPlan pl;
    pl.m_med = m_med;
    pl.units = base < p.unit_cap ? base : p.unit_cap;
    pl.total = pl.units + m_med;
    pl.m_mid = m_mid;
    *p.plan = pl;
  }
}

template <int KCAP, bool FIT, int U>
__global__ __launch_bounds__(kBlock) void seg_long_kernel(SegParams p) {
  __shared__ TopkShared<KCAP> sh;
  __shared__ v4i ring_lds[kWaves][kRing][U][kWave];
  __shared__ int item_sh;
  static_assert(sizeof(ring_lds) >= sizeof(Stage2Lds), "ring too small");
  const SegPlan plan = *p.plan;
  const int k = p.k;
  const int G = gridDim.x;
  // Mid-length segments first, one wave each, in registers as in the short
  // kernel; the ring's LDS holds the waves' candidate buffers meanwhile.
  static_assert(sizeof(ring_lds) >= kWaves * sizeof(RowsWaveLds),
                "ring holds the waves' buffers");
  if (plan.m_mid > 0) {
    RowsWaveLds* rl = reinterpret_cast<RowsWaveLds*>(&ring_lds[0][0][0][0]);
    const int w = uni((int)(threadIdx.x / kWave));
    for (int64_t i = (int64_t)blockIdx.x * kWaves + w; i < plan.m_mid;
         i += (int64_t)G * kWaves) {
      const int s = uni(p.mid[i]);
      int64_t a, b;
      seg_bounds(p, s, a, b);
      const int n = uni((int)(b - a));  // in (kSegReg, kSegShort]
      const int kk = n < k ? n : k;
      int* dst = p.out + (int64_t)s * k;
      if (n <= 2048)
        seg_short_topk<32>(p.in + a, n, kk, dst, rl[w]);
      else
        seg_short_topk<64>(p.in + a, n, kk, dst, rl[w]);
      for (int j = kk + lane(); j < k; j += kWave) dst[j] = kI32Min;
      if (p.counts && lane() == 0) p.counts[s] = kk;
    }
    __syncthreads();  // the ring is the items' again
  }
  // Work items: workgroup b starts with item b, then takes items G, G + 1,
  // ... from a counter (G = gridDim.x).  Every workgroup that started ends
  // with one grab past the end; the last grab of all arms the counter for
  // the next call.
  const int64_t started = min((int64_t)G, (int64_t)plan.total);
  const uint64_t grabs =
      (uint64_t)(plan.total > G ? plan.total - G : 0) + (uint64_t)started;
  int item = blockIdx.x;
  for (;; ) {
    if (item >= plan.total) break;
    // Take the next item now; its index is first needed after this one.
    uint64_t c = 0;
    if (threadIdx.x == 0) c = SegCount::add(p.ctr + 2, 1, p.seg_tag);
    if (item < plan.units) {
      const SegUnit u = p.units[item];
      const SegHuge h = p.huge[u.j];
      workgroup_topk<KCAP, FIT, U>(p.in + u.start, u.len, 0, 1, k, p.refresh,
                                   p.cand + (int64_t)item * k,
                                   p.heads + item, p.kths + item, sh,
                                   ring_lds);
      if (last_to_finish(p.ticket + 1 + u.j, h.units, p.epoch, &sh.is_last)) {
        // The segment's last unit: stage 2 over its units' candidates.
        Stage2Lds& s2 = *reinterpret_cast<Stage2Lds*>(&ring_lds[0][0][0][0]);
        const int nu = h.units;
        const bool all_in_lds = nu * k <= kDirectCand;
        const CandView cv{p.cand + (int64_t)h.base * k, k, k};
        stage2_init(sh, s2);
        stage2_fill_blocks(p.heads + h.base, p.kths + h.base, cv.cand, nu,
                           nu * k, all_in_lds, sh, s2);
        const Stage2Bound r = stage2_bound(cv, nu, k, all_in_lds, sh, s2);
        stage2_finish(cv, k, r, p.out + (int64_t)h.seg * k, sh, s2);
        if (p.counts && threadIdx.x == 0) p.counts[h.seg] = k;
      }
    } else {
      const int s = p.med[item - plan.units];
      int64_t a, b;
      seg_bounds(p, s, a, b);
      workgroup_topk<KCAP, FIT, U>(p.in + a, b - a, 0, 1, k, p.refresh,
                                   p.out + (int64_t)s * k, nullptr, nullptr,
                                   sh, ring_lds);
      if (p.counts && threadIdx.x == 0) p.counts[s] = k;
    }
    __syncthreads();  // the item's LDS reads are done; item_sh is free
    if (threadIdx.x == 0) {
      if (c == grabs - 1) st_agent(p.ctr + 2, SegCount::armed(p.seg_tag + 1u));
      item_sh = (int)min((uint64_t)G + c, (uint64_t)plan.total);
    }
    __syncthreads();
    item = item_sh;
  }
}

}  // namespace ltk
