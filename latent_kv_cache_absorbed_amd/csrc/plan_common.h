// The split-KV planner rule on the device, shared by the planner kernel and by the decode kernel's
// fused-plan prologue (the host computes the same rule in plan_host, api.cpp).
//
//   L_b   = clamp(seq_lens[b], 0, capacity)
//   auto:   chunk(T) = the smallest multiple of page with sum_b ceil(L_b / chunk) <= T
//           (roundup(max_b L_b, page) when none is); with T1 = one work group per CU (base_units)
//           and T2 = the resident work groups over the chip (target_units, a multiple of T1),
//           chunk = max(chunk(T2), min(chunk(T1), kMinChunkPages * page));    n_b = ceil(L_b / chunk)
//   forced: chunk_b = max(page, roundup(ceil(L_b / splits), page));        n_b = ceil(L_b / chunk_b)
//   either chunk is capped at kUnitPages pages
//   units of sequence b are first_b .. first_b + n_b - 1 (first_b = exclusive prefix sum of n_b),
//   unit first_b + s covers tokens [s * chunk_b, min(L_b, (s + 1) * chunk_b)).
//   combine tasks of b: none for one split, one for an empty sequence, else ceil(n_b / kCombineChunk);
//   b is a "multi" sequence (its chunk results are merged again) when it has more than one task.
#ifndef LD_PLAN_COMMON_H
#define LD_PLAN_COMMON_H

#include <hip/hip_runtime.h>

#include "ld_internal.h"

namespace ld {
namespace {

constexpr int kCachedLens = 16;  // page counts per lane of the searching wave kept in registers

__device__ __forceinline__ int plan_clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Automatic chunk (tokens), or 0 with forced splits.  Called by all 64 lanes of one wave; every
// lane returns the same value.  The smallest chunk is found by bisection on the page count (the
// unit count only falls as the chunk grows; ceil(L / (k * page)) = ceil(ceil(L / page) / k)), with
// the page counts of the first 64 * kCachedLens sequences held in registers.
__device__ __forceinline__ int plan_auto_chunk(const PlanArgs& a, int lane) {
  if (a.forced_splits > 0) return 0;
  const int page = a.page_size;
  auto pages_of = [&](int b) { return (unsigned)((plan_clampi(a.seq_lens[b], 0, a.capacity) + page - 1) / page); };
  unsigned pg[kCachedLens];
  unsigned mx = 0, sum = 0;
  const int kk = min(kCachedLens, (a.batch + 63) / 64);  // cached rows in use (uniform)
  // every load is issued before any is used (indices past the batch read sequence 0 and are masked)
  int raw[kCachedLens];
#pragma unroll
  for (int k = 0; k < kCachedLens; ++k) {
    const int b = lane + 64 * k;
    raw[k] = a.seq_lens[b < a.batch ? b : 0];
  }
#pragma unroll
  for (int k = 0; k < kCachedLens; ++k) {
    const int b = lane + 64 * k;
    pg[k] = (k < kk && b < a.batch) ? (unsigned)((plan_clampi(raw[k], 0, a.capacity) + page - 1) / page) : 0u;
    mx = max(mx, pg[k]);
    sum = min(sum + pg[k], 1u << 30);
  }
  for (int b = lane + 64 * kCachedLens; b < a.batch; b += 64) {
    const unsigned pb = pages_of(b);
    mx = max(mx, pb);
    sum = min(sum + pb, 1u << 30);
  }
  for (int off = 32; off > 0; off >>= 1) {
    mx = max(mx, (unsigned)__shfl_xor((int)mx, off));
    sum = min(sum + (unsigned)__shfl_xor((int)sum, off), 1u << 30);
  }
  auto count = [&](unsigned k) {  // units for a chunk of k pages, saturated at 2^30
    unsigned cnt = 0;
#pragma unroll
    for (int j = 0; j < kCachedLens; ++j)
      if (j < kk) cnt += (pg[j] + k - 1) / k;
    for (int b = lane + 64 * kCachedLens; b < a.batch; b += 64) cnt = min(cnt + (pages_of(b) + k - 1) / k, 1u << 30);
    for (int off = 32; off > 0; off >>= 1) cnt = min(cnt + (unsigned)__shfl_xor((int)cnt, off), 1u << 30);
    return cnt;
  };
  // sum_b ceil(P_b / k) >= sum_b P_b / k, so no k below ceil(sum / target) qualifies; for
  // balanced lengths that bound usually does
  auto chunk_pages = [&](unsigned tu) {
    unsigned lo = max(1u, (sum + tu - 1) / tu), hi = max(mx, 1u);
    if (lo >= hi || count(lo) <= tu) {
      hi = lo = min(lo, hi);
    } else {
      lo = lo + 1;
    }
    while (lo < hi) {  // uniform across the wave
      const unsigned mid = (lo + hi) >> 1;
      if (count(mid) <= tu)
        hi = mid;
      else
        lo = mid + 1;
    }
    return min(lo, (unsigned)kUnitPages);
  };
  const unsigned c1 = chunk_pages((unsigned)a.base_units);
  if (a.target_units == a.base_units) return (int)c1 * page;
  const unsigned c2 = chunk_pages((unsigned)a.target_units);
  return (int)max(c2, min(c1, (unsigned)kMinChunkPages)) * page;
}

// One sequence's share of the plan: clamped length, chunk, units, combine tasks, multi flag.
struct SeqPlan {
  int L, ck, n, nc, mc;
};

// raw_len: seq_lens[b] as stored (read by the caller)
__device__ __forceinline__ SeqPlan plan_seq_len(const PlanArgs& a, int chunk, int b, int raw_len) {
  SeqPlan s{0, chunk, 0, 0, 0};
  if (b >= a.batch) return s;
  const int page = a.page_size;
  s.L = plan_clampi(raw_len, 0, a.capacity);
  if (a.forced_splits > 0) {
    const int per = (s.L + a.forced_splits - 1) / a.forced_splits;
    s.ck = (per + page - 1) / page * page;
    if (s.ck < page) s.ck = page;
    if (s.ck > kUnitPages * page) s.ck = kUnitPages * page;
  }
  s.n = (s.L + s.ck - 1) / s.ck;
  s.nc = s.n == 1 ? 0 : (s.n == 0 ? 1 : (s.n + kCombineChunk - 1) / kCombineChunk);
  s.mc = s.nc > 1 ? 1 : 0;
  return s;
}

__device__ __forceinline__ SeqPlan plan_seq(const PlanArgs& a, int chunk, int b) {
  return plan_seq_len(a, chunk, b, b < a.batch ? a.seq_lens[b] : 0);
}

}  // namespace
}  // namespace ld

#endif  // LD_PLAN_COMMON_H
