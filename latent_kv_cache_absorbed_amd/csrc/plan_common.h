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

// Inclusive scan over the 64 lanes of a fully active wave by DPP lane moves (VALU operands, no LDS
// round trip): shifts by 1, 2, 4 and 8 lanes inside each 16-lane row give every lane its row's
// prefix, then lane 15 of rows 0 and 2 is broadcast into rows 1 and 3, and lane 31 into rows 2 and
// 3.  A lane with no source lane, or a row left out by the row mask, takes 0, so `op` must be
// associative with 0 as its identity on the values it sees: sums and maxima of non-negative counts.
template <typename Op>
__device__ __forceinline__ int wave_scan_dpp(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true));   // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true));   // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true));   // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true));   // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15 into rows 1, 3
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31 into rows 2, 3
  return v;
}
// sum saturated at 2^30 (operands at most 2^30, so the unsigned sum cannot wrap)
__device__ __forceinline__ int sat_add(int x, int y) { return (int)min((unsigned)x + (unsigned)y, 1u << 30); }
// wave-wide results (uniform): saturated sum, maximum, plain sum of non-negative counts
__device__ __forceinline__ int wave_sum_sat(int v) {
  return __builtin_amdgcn_readlane(wave_scan_dpp(v, [](int x, int y) { return sat_add(x, y); }), 63);
}
__device__ __forceinline__ int wave_max(int v) {
  return __builtin_amdgcn_readlane(wave_scan_dpp(v, [](int x, int y) { return max(x, y); }), 63);
}
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_scan_dpp(v, [](int x, int y) { return x + y; }), 63);
}

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
  mx = (unsigned)wave_max((int)mx);
  sum = (unsigned)wave_sum_sat((int)sum);
  auto count = [&](unsigned k) {  // units for a chunk of k pages, saturated at 2^30
    unsigned cnt = 0;
#pragma unroll
    for (int j = 0; j < kCachedLens; ++j)
      if (j < kk) cnt += (pg[j] + k - 1) / k;
    for (int b = lane + 64 * kCachedLens; b < a.batch; b += 64) cnt = min(cnt + (pages_of(b) + k - 1) / k, 1u << 30);
    return (unsigned)wave_sum_sat((int)cnt);
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

// Fused plan.  Wave 0 of every work group applies the planner rule (plan_common.h) to seq_lens:
// the unit count, then the unit this work group takes (same XCD-blocked mapping as with a stored
// plan), then that unit's sequence, split and token range, which it leaves in u[0..4] (u[0] = -1:
// no unit).  The plan arrays the combine reads are written on the way: each sequence's entries and
// tasks by the first work group of its first unit, the unit record by the unit's first work group,
// and the header, the entries of empty sequences (which have no unit) and the zeroed combine
// arrival counters by work group 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  return wave_scan_dpp(v, [](int x, int y) { return x + y; });
}

__device__ __forceinline__ void fused_plan_unit(const DecodeArgs& a, int x, int xcd, int yy, int sb, int* u) {
  const PlanArgs& P = a.plan;
  const int lane = threadIdx.x & 63;
  // the lengths of the first 64 * kFusedLens sequences are read once, into registers
  constexpr int kFusedLens = 4;
  int len[kFusedLens];
#pragma unroll
  for (int k = 0; k < kFusedLens; ++k) {
    const int bb = lane + 64 * k;
    len[k] = (64 * k < P.batch && bb < P.batch) ? P.seq_lens[bb] : 0;
  }
  auto seq = [&](int chunk_, int base) {
    const int bb = base + lane;
    const int k = base >> 6;
    int raw = 0;
#pragma unroll
    for (int j = 0; j < kFusedLens; ++j)
      if (j == k) raw = len[j];
    if (k >= kFusedLens && bb < P.batch) raw = P.seq_lens[bb];
    return plan_seq_len(P, chunk_, bb, raw);
  };
  const int chunk = plan_auto_chunk(P, lane);
  // the plan of the first 64 sequences is kept; every later block of 64 is derived again where needed
  const SeqPlan sp0 = seq(chunk, 0);
  int tn = 0, tc = 0, tm = 0;
  for (int base = 0; base < P.batch; base += 64) {
    const SeqPlan sp = base == 0 ? sp0 : seq(chunk, base);
    tn = sat_add(tn, sp.n);
    tc = sat_add(tc, sp.nc);
    tm += sp.mc;
  }
  tn = wave_sum_sat(tn);
  tc = wave_sum_sat(tc);
  tm = wave_sum(tm);
  const int nunits = min(tn, P.max_units);
  if (x == 0) {
    if (lane == 0) {
      P.header[0] = nunits;
      P.header[1] = chunk;
      P.header[2] = min(tc, P.max_tasks);
      P.header[3] = min(tm, P.max_multi);
    }
    for (int i = lane; i < P.ccount_n; i += 64) P.ccount[i] = 0;  // combine arrival counters
    // empty sequences: one combine task each, which writes zeros
    int cn = 0, cc = 0;
    for (int base = 0; base < P.batch; base += 64) {
      const int b = base + lane;
      const SeqPlan sp = base == 0 ? sp0 : seq(chunk, base);
      const int in = wave_incl_scan(sp.n), ic = wave_incl_scan(sp.nc);
      if (b < P.batch && sp.n == 0) {
        const int ftask = cc + ic - sp.nc;
        P.seqs[4 * b] = 0;
        P.seqs[4 * b + 1] = cn + in;
        P.seqs[4 * b + 2] = ftask;
        P.seqs[4 * b + 3] = 1;
        if (ftask < P.max_tasks) reinterpret_cast<int4*>(P.tasks)[ftask] = make_int4(b, 0, cn + in, 0);
      }
      cn += __builtin_amdgcn_readlane(in, 63);
      cc += __builtin_amdgcn_readlane(ic, 63);
    }
  }
  const int per = (nunits + 7) >> 3;
  const int unit = xcd * per + yy;
  if (yy >= per || unit >= nunits) {
    if (lane == 0) u[0] = -1;
    return;
  }
  // the sequence holding the unit: first_b <= unit < first_b + n_b
  int cn = 0, cc = 0, cm = 0;
  int b = -1, first = 0, ftask = 0, mi = 0, L = 0, ck = 1, n = 0, nc = 0, mc = 0;
  for (int base = 0; base < P.batch; base += 64) {
    const SeqPlan sp = base == 0 ? sp0 : seq(chunk, base);
    const int in = wave_incl_scan(sp.n), ic = wave_incl_scan(sp.nc), im = wave_incl_scan(sp.mc);
    const int f = cn + in - sp.n;
    const unsigned long long hit = __ballot(base + lane < P.batch && unit >= f && unit < f + sp.n);
    if (hit) {
      const int src = __ffsll(hit) - 1;
      b = base + src;
      first = __builtin_amdgcn_readlane(f, src);
      ftask = __builtin_amdgcn_readlane(cc + ic - sp.nc, src);
      mi = __builtin_amdgcn_readlane(cm + im - sp.mc, src);
      L = __builtin_amdgcn_readlane(sp.L, src);
      ck = __builtin_amdgcn_readlane(sp.ck, src);
      n = __builtin_amdgcn_readlane(sp.n, src);
      nc = __builtin_amdgcn_readlane(sp.nc, src);
      mc = __builtin_amdgcn_readlane(sp.mc, src);
      break;
    }
    cn += __builtin_amdgcn_readlane(in, 63);
    cc += __builtin_amdgcn_readlane(ic, 63);
    cm += __builtin_amdgcn_readlane(im, 63);
  }
  if (b < 0) {  // unreachable: the units are counted from the same lengths
    if (lane == 0) u[0] = -1;
    return;
  }
  const int s = unit - first;
  const int t_begin = s * ck;
  const int t_end = min(L, (s + 1) * ck);
  if (lane == 0) {
    u[0] = unit;
    u[1] = b;
    u[2] = t_begin;
    u[3] = t_end;
    u[4] = n;
  }
  if (sb != 0) return;
  if (lane == 0) P.units[unit] = Unit{b, t_begin, t_end, s};
  if (s != 0) return;
  if (lane == 0) {
    P.seqs[4 * b] = n;
    P.seqs[4 * b + 1] = first;
    P.seqs[4 * b + 2] = ftask;
    P.seqs[4 * b + 3] = nc;
    if (mc && mi < P.max_multi) P.multi[mi] = b;
  }
  for (int c = lane; c < nc; c += 64) {
    if (ftask + c < P.max_tasks) reinterpret_cast<int4*>(P.tasks)[ftask + c] = make_int4(b, c, first, n);
  }
}

}  // namespace
}  // namespace ld

#endif  // LD_PLAN_COMMON_H
