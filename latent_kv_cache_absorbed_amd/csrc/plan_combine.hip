// Split-KV planner and log-sum-exp combine kernels (gfx950).
//
// The planner rule is stated in plan_common.h (identical to plan_host in api.cpp, which tests
// compare against).
//
// Combine rule for a row split into n parts with normalised partial outputs o_s and
// log-sum-exps lse_s:  lse = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ld_internal.h"
#include "plan_common.h"

namespace ld {
namespace {

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

constexpr int kOwnUnits = 8;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int scan[kPlanThreads];
  __shared__ int scan2[kPlanThreads];
  __shared__ int scan3[kPlanThreads];
  __shared__ int s_chunk;
  __shared__ int s_carry;
  __shared__ int s_carry2;
  __shared__ int s_carry3;
  __shared__ int s_nlong;
  __shared__ int long_b[kPlanThreads], long_n[kPlanThreads], long_first[kPlanThreads], long_L[kPlanThreads],
      long_ck[kPlanThreads];
  const int tid = threadIdx.x;

  if (tid == 0) {
    s_carry = 0;
    s_carry2 = 0;
    s_carry3 = 0;
    s_chunk = 0;
  }
  if (tid < 64) {
    const int c = plan_auto_chunk(a, tid);
    if (tid == 0) s_chunk = c;
  }
  for (int i = tid; i < a.ccount_n; i += blockDim.x) a.ccount[i] = 0;
  __syncthreads();
  const int chunk = s_chunk;

  for (int base = 0; base < a.batch; base += blockDim.x) {
    const int b = base + tid;
    // combine tasks of this sequence: none for one split (the decode kernel writes the output),
    // one for an empty sequence (it writes zeros), else one per chunk of kCombineChunk splits
    const SeqPlan sp = plan_seq(a, chunk, b);
    const int L = sp.L, ck = sp.ck, n = sp.n, nc = sp.nc, mc = sp.mc;
    scan[tid] = n;
    scan2[tid] = nc;
    scan3[tid] = mc;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      const int v2 = tid >= off ? scan2[tid - off] : 0;
      const int v3 = tid >= off ? scan3[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      scan2[tid] += v2;
      scan3[tid] += v3;
      __syncthreads();
    }
    const int first = s_carry + scan[tid] - n;
    const int ftask = s_carry2 + scan2[tid] - nc;
    const int mi = s_carry3 + scan3[tid] - mc;
    auto write_unit = [&](int bb, int s, int f, int LL, int c) {
      const int u = f + s;
      if (u < a.max_units) {
        Unit rec;
        rec.b = bb;
        rec.t_begin = s * c;
        rec.t_end = min(LL, (s + 1) * c);
        rec.split = s;
        a.units[u] = rec;
      }
    };
    // each thread writes the first kOwnUnits units of its sequence; the units beyond those (long
    // sequences split many ways) are written by the whole work group, one such sequence at a time
    if (tid == 0) s_nlong = 0;
    __syncthreads();
    if (b < a.batch) {
      a.seqs[4 * b] = n;
      a.seqs[4 * b + 1] = first;
      a.seqs[4 * b + 2] = ftask;
      a.seqs[4 * b + 3] = nc;
      for (int c = 0; c < nc; ++c)
        if (ftask + c < a.max_tasks) {
          reinterpret_cast<int4*>(a.tasks)[ftask + c] = make_int4(b, c, first, n);
        }
      if (mc && mi < a.max_multi) a.multi[mi] = b;
      for (int s = 0; s < n && s < kOwnUnits; ++s) write_unit(b, s, first, L, ck);
      if (n > kOwnUnits) {
        const int slot = atomicAdd(&s_nlong, 1);
        long_b[slot] = b;
        long_n[slot] = n;
        long_first[slot] = first;
        long_L[slot] = L;
        long_ck[slot] = ck;
      }
    }
    __syncthreads();
    for (int i = 0; i < s_nlong; ++i)
      for (int s = kOwnUnits + tid; s < long_n[i]; s += blockDim.x) write_unit(long_b[i], s, long_first[i], long_L[i], long_ck[i]);
    __syncthreads();
    if (tid == blockDim.x - 1) {
      s_carry += scan[tid];
      s_carry2 += scan2[tid];
      s_carry3 += scan3[tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.header[0] = min(s_carry, a.max_units);
    a.header[1] = chunk;
    a.header[2] = min(s_carry2, a.max_tasks);
    a.header[3] = min(s_carry3, a.max_multi);
  }
}

// Merge the split partials of every sequence whose split count is not 1.  The partials are in
// the decode kernel's fragment order: slot block (unit, set, 32-head block) holds 32 heads x d_v
// values as [column block][piece][lane][value], where a piece is the 8 (bf16) or 4 (f32)
// consecutive accumulator registers of one lane: register i of lane l holds head l % 32 and
// column 32 * cb + 8 * (i / 4) + 4 * (l / 32) + i % 4.
//
// A combine task is (sequence, chunk of at most kCombineChunk splits).  Work group (x, t) takes
// task t and 256 piece positions: one 64-lane piece group per wave, one 1 KB load per split, all
// of a chunk's loads issued together.  A sequence merged in one chunk is finished there; the
// chunk results of longer ones are merged in chunk order by the last of their tasks to finish.
constexpr int kCombineThreads = 256;

struct PieceGroup {
  int j, cb, hb, gs, lane, h, head_in_set;
  size_t blk_in_unit, blocks_per_unit, piece_off, pieces;
};

// plane: the piece position (0..63) within the group, by default this thread's lane
__device__ __forceinline__ PieceGroup piece_group(const DecodeArgs& a, int d_v, int pg, int plane = -1) {
  PieceGroup p;
  const int vals = a.part_bf16 ? 8 : 4;
  const int jn = 16 / vals;
  const int cbn = d_v / 32;
  int rest = pg;                       // pg = ((gs * HB + hb) * cbn + cb) * jn + j
  p.j = rest % jn;
  rest /= jn;
  p.cb = rest % cbn;
  rest /= cbn;
  p.hb = rest % a.hblocks;
  p.gs = rest / a.hblocks;
  p.lane = plane >= 0 ? plane : (int)(threadIdx.x & 63);
  p.h = p.lane >> 5;
  p.head_in_set = p.hb * 32 + (p.lane & 31);
  p.blk_in_unit = (size_t)p.gs * a.hblocks + p.hb;
  p.blocks_per_unit = (size_t)a.groups * a.hblocks;
  p.piece_off = ((size_t)(p.cb * jn + p.j) * 64 + p.lane) * vals;
  p.pieces = (size_t)a.xblocks * 256;
  return p;
}

// Output row of query set gs, head head_in_set: gs * heads_per_set + head; MLRA rows are (token,
// head, branch) with the branch innermost, its sets token * branches + branch
__device__ __forceinline__ int out_row(const DecodeArgs& a, int gs, int head_in_set) {
  if (!a.mlra) return gs * a.heads_per_set + head_in_set;
  const int qi = gs / a.cache_groups;
  return (qi * a.heads_per_set + head_in_set) * a.cache_groups + (gs - qi * a.cache_groups);
}

// out and lse of one piece position (lane) of sequence b
__device__ __forceinline__ void write_piece(const DecodeArgs& a, int d_v, const PieceGroup& p, int b,
                                            const float* o, float lse) {
  if (p.head_in_set >= a.heads_per_set) return;
  const int vals = a.part_bf16 ? 8 : 4;
  const int row = out_row(a, p.gs, p.head_in_set);
  const size_t orow = (size_t)b * a.rows + row;
  if (p.cb == 0 && p.j == 0 && p.h == 0) a.lse[orow] = lse;
  // value e of piece j is register i = vals * j + e: column 32 cb + 8 (i / 4) + 4 h + i % 4
  for (int q = 0; q < vals / 4; ++q) {
    const int i0 = vals * p.j + 4 * q;
    const int col = p.cb * 32 + 8 * (i0 / 4) + 4 * p.h;
    if (a.out_bf16) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t v = {(__bf16)o[4 * q], (__bf16)o[4 * q + 1], (__bf16)o[4 * q + 2], (__bf16)o[4 * q + 3]};
      *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(a.out) + orow * d_v + col) = v;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * d_v + col) =
          make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
  }
}

// Online merge of (lse, normalised piece) pairs in batches of kBatch: the loads of a batch are
// issued together (indexes past the last pair repeat it and get weight 0), then the running max,
// sum and weighted values are updated.  Pairs are taken in index order.
constexpr int kBatch = 8;

// e^x for merge weights (x <= 0): v_exp_f32 of x log2(e); the relative error of a weight is below
// 2^-22 (1 + |x|), and weights of large |x| are negligible beside the largest (which is 1)
__device__ __forceinline__ float wexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896340736f); }

// A NaN lse (a NaN reached that split's scores, e.g. through a NaN query) makes the merged row NaN,
// as the combine rule computes it; fmaxf would drop it, so it is recorded by poisoning `tot`, which
// every later rescale and merge carries along.
struct Merge {
  float M = -INFINITY, tot = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  template <int KB = kBatch>
  __device__ __forceinline__ void add(const float* ls, const float (*v)[8], int valid, int vals) {
    float bm = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (k < valid) {
        bm = fmaxf(bm, ls[k]);
        nan |= ls[k] != ls[k];
      }
    if (nan) tot = __builtin_nanf("");
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) return;
    const float r = (M == -INFINITY) ? 0.f : wexp(M - Mn);
    tot *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= r;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float w = k < valid ? wexp(ls[k] - Mn) : 0.f;
      tot += w;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < vals) o[e] += w * v[k][e];
    }
    M = Mn;
  }
  // the same over raw pieces as loaded: eight bf16 (bf16 = true) or four f32 per uint4, widened
  // here, so that a batch of loads in flight holds 4 registers a piece, not 8 (more work groups fit)
  template <int KB = kBatch>
  __device__ __forceinline__ void add_raw(const float* ls, const uint4* raw, int valid, bool bf16) {
    float bm = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (k < valid) {
        bm = fmaxf(bm, ls[k]);
        nan |= ls[k] != ls[k];
      }
    if (nan) tot = __builtin_nanf("");
    const float Mn = fmaxf(M, bm);
    if (Mn == -INFINITY) return;
    const float r = (M == -INFINITY) ? 0.f : wexp(M - Mn);
    tot *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= r;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float w = k < valid ? wexp(ls[k] - Mn) : 0.f;
      tot += w;
      const unsigned u[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
      if (bf16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[2 * q] += w * __builtin_bit_cast(float, u[q] << 16);
          o[2 * q + 1] += w * __builtin_bit_cast(float, u[q] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] += w * __builtin_bit_cast(float, u[q]);
      }
    }
    M = Mn;
  }
  // fold in another state (its pairs come after this one's)
  __device__ __forceinline__ void merge(float M2, float tot2, const float* o2) {
    if (tot2 != tot2) tot = __builtin_nanf("");
    const float Mn = fmaxf(M, M2);
    if (Mn == -INFINITY) return;
    const float r1 = (M == -INFINITY) ? 0.f : wexp(M - Mn);
    const float r2 = (M2 == -INFINITY) ? 0.f : wexp(M2 - Mn);
    tot = tot * r1 + tot2 * r2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * r1 + o2[e] * r2;
    M = Mn;
  }
  // normalised output and lse (0 and -inf when every lse was -inf; NaN when one was NaN)
  __device__ __forceinline__ float finish() {
    if (tot != tot) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_nanf("");
      return __builtin_nanf("");
    }
    if (M == -INFINITY) return -INFINITY;
    const float inv = 1.f / tot;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    return M + logf(tot);
  }
};

// The 4 waves of a work group hold 32 heads x 32 (f32) or 64 (bf16) consecutive columns of the
// output; a sequence finished here passes them through LDS so that every store writes 16 bytes of
// a row and each row segment is written whole (128 B per head).
__device__ __forceinline__ void write_tile(const DecodeArgs& a, int d_v, const PieceGroup& p, int b, const float* o,
                                          float lse, float* tile) {
  const int vals = a.part_bf16 ? 8 : 4;
  const int tcols = 8 * vals;  // 4 pieces of 16 / vals per 32-column block: 32 (f32) or 64 (bf16) columns
  const int row_l = p.lane & 31;
  // value e of piece j is register i = vals * j + e: column 32 cb + 8 (i / 4) + 4 h + i % 4
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < vals) {
      const int i = vals * p.j + e;
      const int colg = 32 * p.cb + 8 * (i / 4) + 4 * p.h + (i % 4);
      tile[row_l * (tcols + 1) + (colg % tcols)] = o[e];
    }
  }
  if (p.cb == 0 && p.j == 0 && p.h == 0 && p.head_in_set < a.heads_per_set) {
    const int row = out_row(a, p.gs, p.head_in_set);
    a.lse[(size_t)b * a.rows + row] = lse;
  }
  __syncthreads();
  // thread -> (row, 16-byte chunk): 32 rows x 8 chunks (bf16: 8 values, f32: 4 values)
  const int r = threadIdx.x >> 3, ch = threadIdx.x & 7;
  const int head_in_set = p.hb * 32 + r;
  const int col0 = (32 * p.cb) / tcols * tcols;  // first column of the tile
  if (head_in_set < a.heads_per_set) {
    const int row = out_row(a, p.gs, head_in_set);
    const size_t orow = (size_t)b * a.rows + row;
    const float* src = tile + r * (tcols + 1) + ch * (vals == 8 ? 8 : 4);
    if (a.out_bf16) {
      typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
      bf16x8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (__bf16)src[e];
      *reinterpret_cast<bf16x8_t*>(static_cast<__bf16*>(a.out) + orow * d_v + col0 + ch * 8) = v;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * d_v + col0 + ch * 4) =
          make_float4(src[0], src[1], src[2], src[3]);
    }
  }
}

__global__ __launch_bounds__(kCombineThreads) void combine_ws_kernel(DecodeArgs a, int d_v) {
  __shared__ float tile[32 * 65];
  const int t = blockIdx.y;
  // The task record carries what the merge needs (sequence, chunk, first unit, splits), so the
  // partials' loads wait for one round trip, not two; it is read together with the task count.
  const int ntask = a.header[2];
  const int4 task = reinterpret_cast<const int4*>(a.tasks)[t];
  const int b = task.x, c = task.y;
  if ((t >= ntask) | (b < 0)) return;  // (b >= 0 in every task; testing it keeps both loads before the branch)
  const int first = task.z;
  const int n = max(0, min(task.w, a.max_units - first));
  const int nc = task.w > kCombineChunk ? (task.w + kCombineChunk - 1) / kCombineChunk : 1;
  const int ftask = t - c;
  const int pg = 4 * blockIdx.x + (threadIdx.x >> 6);
  const PieceGroup p = piece_group(a, d_v, pg);
  const int vals = a.part_bf16 ? 8 : 4;
  const int s_lo = c * kCombineChunk;
  const int cnt = max(0, min(n - s_lo, kCombineChunk));  // splits of this chunk
  Merge m;
  // one batch of KB (lse, piece) pairs, loads issued together; indexes past the last repeat it
  auto batch = [&](auto kb, int k0) {
    constexpr int KB = decltype(kb)::value;
    float ls[KB];
    uint4 raw[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const size_t s = first + s_lo + min(k0 + k, cnt - 1);
      ls[k] = a.part_lse[(s * p.blocks_per_unit + p.blk_in_unit) * 32 + (p.lane & 31)];
      const size_t off = (s * p.blocks_per_unit + p.blk_in_unit) * (size_t)(32 * d_v) + p.piece_off;
      raw[k] = a.part_bf16 ? *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.part_out) + off)
                           : *reinterpret_cast<const uint4*>(static_cast<const float*>(a.part_out) + off);
    }
    m.add_raw<KB>(ls, raw, cnt - k0, a.part_bf16 != 0);
  };
  if (cnt <= 4) {
    if (cnt > 0) batch(std::integral_constant<int, 4>{}, 0);
  } else {
    for (int k0 = 0; k0 < cnt; k0 += kBatch) batch(std::integral_constant<int, kBatch>{}, k0);
  }
  if (nc <= 1) {
    const float lse = m.finish();
    write_tile(a, d_v, p, b, m.o, lse, tile);
    return;
  }
  // a chunk of a longer sequence: its merged result (f32, same piece order, with its lse)
  const float lse = m.finish();
  const size_t lo = (size_t)(ftask + c) * p.pieces + (size_t)pg * 64 + p.lane;
  float4* dst = reinterpret_cast<float4*>(a.l2_out + lo * vals);
  dst[0] = make_float4(m.o[0], m.o[1], m.o[2], m.o[3]);
  if (vals == 8) dst[1] = make_float4(m.o[4], m.o[5], m.o[6], m.o[7]);
  a.l2_lse[lo] = lse;
  // The last of the sequence's nc chunk tasks to finish (for this work group's piece positions)
  // merges the chunk results in chunk order.  Release: every wave's results are stored and fenced
  // before the arrival is counted; acquire: the last arriver fences before reading the others'.
  // It resets the counter for the next call (the planner zeroes it too).
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int* ctr = a.ccount + (size_t)ftask * a.xblocks + blockIdx.x;
    s_last = atomicAdd(ctr, 1) == nc - 1;
    if (s_last) *ctr = 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  Merge mm;
  constexpr int kB2 = 4;  // (chunk results are f32: eight registers a piece)
  for (int q0 = 0; q0 < nc; q0 += kB2) {
    float ls[kB2], v[kB2][8];
#pragma unroll
    for (int k = 0; k < kB2; ++k) {
      const size_t l2 = (size_t)(ftask + min(q0 + k, nc - 1)) * p.pieces + (size_t)pg * 64 + p.lane;
      ls[k] = a.l2_lse[l2];
      const float4* src = reinterpret_cast<const float4*>(a.l2_out + l2 * vals);
      const float4 x0 = src[0];
      const float4 x1 = vals == 8 ? src[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[k][0] = x0.x, v[k][1] = x0.y, v[k][2] = x0.z, v[k][3] = x0.w;
      v[k][4] = x1.x, v[k][5] = x1.y, v[k][6] = x1.z, v[k][7] = x1.w;
    }
    mm.add<kB2>(ls, v, nc - q0, vals);
  }
  write_piece(a, d_v, p, b, mm.o, mm.finish());
}

// Batches of a few long sequences (many splits each): work group (x, b) merges part x % kSeqLanes
// (kSeqPos piece positions) of piece group x / kSeqLanes of sequence b in one launch, so that one
// sequence's merge spreads over kSeqLanes times as many work groups as it has piece groups (256 for
// one 128-head MLA row set: every CU).  Its kSeqWaves waves take the sequence's chunks of
// kCombineChunk splits round-robin; the kSeqLanes lanes of a piece position (l, l + kSeqPos, ..)
// fold one part of every chunk each, issuing that part's loads at once and folding them in one step,
// and then merge their states.  The states of the waves then meet in LDS in two rounds (four waves
// fold four states each, then the first wave folds those four) and the first wave writes the result.
constexpr int kSeqWaves = 16;
constexpr int kSeqLanes = 2;                          // lanes per piece position (4: no faster)
constexpr int kSeqPart = kCombineChunk / kSeqLanes;   // splits of a chunk one lane folds
constexpr int kSeqPos = 64 / kSeqLanes;               // piece positions per work group

__global__ __launch_bounds__(kSeqWaves * 64) void combine_seq_kernel(DecodeArgs a, int d_v) {
  __shared__ float st_m[kSeqWaves][64], st_t[kSeqWaves][64], st_o[kSeqWaves][8][64];
  const int b = blockIdx.y;
  const int n_all = a.seqs[4 * b];
  if (n_all == 1) return;  // the decode kernel wrote this sequence's output
  const int first = a.seqs[4 * b + 1];
  const int n = max(0, min(n_all, a.max_units - first));
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int part = lane / kSeqPos;  // which part of each chunk this lane folds
  const PieceGroup p = piece_group(a, d_v, blockIdx.x / kSeqLanes,
                                   (blockIdx.x % kSeqLanes) * kSeqPos + lane % kSeqPos);
  Merge m;
  for (int c0 = wave * kCombineChunk; c0 < n; c0 += kSeqWaves * kCombineChunk) {
    const int s0 = c0 + part * kSeqPart;
    const int cnt = min(n - s0, kSeqPart);  // none for the later parts of a short last chunk
    if (cnt <= 0) continue;
    // every load of the part is issued before any is used (raw pieces: 16 bytes each)
    float ls[kSeqPart];
    uint4 raw[kSeqPart];
#pragma unroll
    for (int k = 0; k < kSeqPart; ++k) {
      const size_t s = first + s0 + min(k, cnt - 1);
      ls[k] = a.part_lse[(s * p.blocks_per_unit + p.blk_in_unit) * 32 + (p.lane & 31)];
      const size_t off = (s * p.blocks_per_unit + p.blk_in_unit) * (size_t)(32 * d_v) + p.piece_off;
      raw[k] = a.part_bf16 ? *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.part_out) + off)
                           : *reinterpret_cast<const uint4*>(static_cast<const float*>(a.part_out) + off);
    }
    // one online-merge step over the part chunk, each piece converted as it is folded in
    float bm = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int k = 0; k < kSeqPart; ++k)
      if (k < cnt) {
        bm = fmaxf(bm, ls[k]);
        nan |= ls[k] != ls[k];
      }
    if (nan) m.tot = __builtin_nanf("");
    const float Mn = fmaxf(m.M, bm);
    if (Mn != -INFINITY) {
      const float r = (m.M == -INFINITY) ? 0.f : wexp(m.M - Mn);
      m.tot *= r;
#pragma unroll
      for (int e = 0; e < 8; ++e) m.o[e] *= r;
#pragma unroll
      for (int k = 0; k < kSeqPart; ++k) {
        const float w = k < cnt ? wexp(ls[k] - Mn) : 0.f;
        m.tot += w;
        const uint4 x = raw[k];
        if (a.part_bf16) {
          typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
          const bf16x8_t y = __builtin_bit_cast(bf16x8_t, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) m.o[e] += w * (float)y[e];
        } else {
          m.o[0] += w * __builtin_bit_cast(float, x.x);
          m.o[1] += w * __builtin_bit_cast(float, x.y);
          m.o[2] += w * __builtin_bit_cast(float, x.z);
          m.o[3] += w * __builtin_bit_cast(float, x.w);
        }
      }
      m.M = Mn;
    }
  }
  // the parts of this piece position's chunks (lanes l, l ^ kSeqPos, ..) meet; the lanes of the
  // first part carry the result on
#pragma unroll
  for (int off = 32; off >= kSeqPos; off >>= 1) {
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(m.o[e], off);
    const float M2 = __shfl_xor(m.M, off), t2 = __shfl_xor(m.tot, off);
    m.merge(M2, t2, o2);
  }
  st_m[wave][lane] = m.M;
  st_t[wave][lane] = m.tot;
#pragma unroll
  for (int e = 0; e < 8; ++e) st_o[wave][e][lane] = m.o[e];
  __syncthreads();
  // the states meet in two rounds: waves 0..3 fold in waves w + 4, w + 8, w + 12, then wave 0 folds
  // in waves 1..3 (wave w's chunks are w, w + kSeqWaves, ...; the merge is a sum, so the order
  // changes only the rounding)
  auto fold = [&](int w) {
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = st_o[w][e][lane];
    m.merge(st_m[w][lane], st_t[w][lane], o2);
  };
  if (wave < 4) {
    fold(wave + 4);
    fold(wave + 8);
    fold(wave + 12);
  }
  __syncthreads();
  if (wave >= 1 && wave < 4) {
    st_m[wave][lane] = m.M;
    st_t[wave][lane] = m.tot;
#pragma unroll
    for (int e = 0; e < 8; ++e) st_o[wave][e][lane] = m.o[e];
  }
  __syncthreads();
  if (wave != 0 || part != 0) return;
  fold(1);
  fold(2);
  fold(3);
  const float lse = m.finish();
  write_piece(a, d_v, p, b, m.o, lse);
}

__global__ __launch_bounds__(kCombineThreads) void combine_rows_kernel(int num_rows, int d_v, int max_splits,
                                                                       const float* part_out, const float* part_lse,
                                                                       const int32_t* nsplits, int out_bf16,
                                                                       void* out, float* lse_out,
                                                                       int rows_per_block) {
  const int c4n = d_v >> 2;
  const int r0 = blockIdx.x * rows_per_block;
  for (int idx = threadIdx.x; idx < rows_per_block * c4n; idx += blockDim.x) {
    const int r = r0 + idx / c4n;
    if (r >= num_rows) break;
    const int c = (idx % c4n) * 4;
    const int n = clampi(nsplits[r], 0, max_splits);
    const float* ls = part_lse + (size_t)r * max_splits;
    float M = -INFINITY;
    bool nan = false;
    for (int s = 0; s < n; ++s) {
      M = fmaxf(M, ls[s]);
      nan |= ls[s] != ls[s];
    }
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = -INFINITY;
    if (nan) {  // a NaN lse makes the row NaN (fmaxf above skips it)
      const float q = __builtin_nanf("");
      o = make_float4(q, q, q, q);
      lse = q;
    } else if (M != -INFINITY) {
      float tot = 0.f;
      for (int s = 0; s < n; ++s) tot += expf(ls[s] - M);
      lse = M + logf(tot);
      for (int s = 0; s < n; ++s) {
        const float w = expf(ls[s] - lse);
        const float4 v = *reinterpret_cast<const float4*>(part_out + ((size_t)r * max_splits + s) * d_v + c);
        o.x += w * v.x;
        o.y += w * v.y;
        o.z += w * v.z;
        o.w += w * v.w;
      }
    }
    if (c == 0) lse_out[r] = lse;
    if (out_bf16) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t v = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
      *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(out) + (size_t)r * d_v + c) = v;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)r * d_v + c) = o;
    }
  }
}

}  // namespace

int launch_plan(const PlanArgs& a, void* stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

int launch_combine_ws(const DecodeArgs& a, int32_t d_v, void* stream) {
  if (a.batch == 0 || a.rows == 0) return 0;
  if (a.batch <= kSeqCombineMaxBatch) {
    // a few sequences, so (when split) many splits each: one launch, one wide work group per
    // (piece group, sequence)
    hipLaunchKernelGGL(combine_seq_kernel, dim3(a.xblocks * 4 * kSeqLanes, a.batch), dim3(kSeqWaves * 64), 0,
                       static_cast<hipStream_t>(stream), a, d_v);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL(combine_ws_kernel, dim3(a.xblocks, a.max_tasks), dim3(kCombineThreads), 0,
                     static_cast<hipStream_t>(stream), a, d_v);
  return (int)hipGetLastError();
}

int launch_combine_rows(int32_t num_rows, int32_t d_v, int32_t max_splits, const float* part_out,
                        const float* part_lse, const int32_t* nsplits, int32_t out_bf16, void* out, float* lse,
                        void* stream) {
  if (num_rows == 0) return 0;
  const int rpb = d_v >= 256 ? 4 : 16;
  const dim3 grid((num_rows + rpb - 1) / rpb);
  hipLaunchKernelGGL(combine_rows_kernel, grid, dim3(kCombineThreads), 0, static_cast<hipStream_t>(stream), num_rows,
                     d_v, max_splits, part_out, part_lse, nsplits, out_bf16, out, lse, rpb);
  return (int)hipGetLastError();
}

}  // namespace ld
