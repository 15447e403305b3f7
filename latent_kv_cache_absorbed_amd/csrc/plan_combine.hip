// Split-KV planner and log-sum-exp combine kernels (gfx950).
//
// Planner rule (identical to plan_host in api.cpp, which tests compare against):
//   L_b   = clamp(seq_lens[b], 0, capacity)
//   auto:   chunk = max(page, roundup(ceil(sum_b L_b / target_units), page)); n_b = ceil(L_b / chunk)
//   forced: chunk_b = max(page, roundup(ceil(L_b / splits), page));        n_b = ceil(L_b / chunk_b)
//   units of sequence b are first_b .. first_b + n_b - 1 (first_b = exclusive prefix sum of n_b),
//   unit first_b + s covers tokens [s * chunk_b, min(L_b, (s + 1) * chunk_b)).
//
// Combine rule for a row split into n parts with normalised partial outputs o_s and
// log-sum-exps lse_s:  lse = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s.
#include <hip/hip_runtime.h>

#include "ld_internal.h"

namespace ld {
namespace {

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

constexpr int kOwnUnits = 8;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ long long red[kPlanThreads / 64];
  __shared__ int scan[kPlanThreads];
  __shared__ int s_chunk;
  __shared__ int s_carry;
  __shared__ int s_nlong;
  __shared__ int long_b[kPlanThreads], long_n[kPlanThreads], long_first[kPlanThreads], long_L[kPlanThreads],
      long_ck[kPlanThreads];
  const int tid = threadIdx.x;
  const int page = a.page_size;

  long long part = 0;
  for (int b = tid; b < a.batch; b += blockDim.x) part += clampi(a.seq_lens[b], 0, a.capacity);
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) red[tid >> 6] = part;
  __syncthreads();
  if (tid == 0) {
    long long total = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total += red[w];
    int chunk = 0;
    if (a.forced_splits <= 0) {
      const long long per = (total + a.target_units - 1) / a.target_units;
      long long c = (per + page - 1) / page * page;
      if (c < page) c = page;
      chunk = (int)(c > 0x7fffffffLL ? 0x7fffffff : c);
    }
    s_chunk = chunk;
    s_carry = 0;
  }
  __syncthreads();
  const int chunk = s_chunk;

  for (int base = 0; base < a.batch; base += blockDim.x) {
    const int b = base + tid;
    int L = 0, ck = chunk, n = 0;
    if (b < a.batch) {
      L = clampi(a.seq_lens[b], 0, a.capacity);
      if (a.forced_splits > 0) {
        const int per = (L + a.forced_splits - 1) / a.forced_splits;
        ck = (per + page - 1) / page * page;
        if (ck < page) ck = page;
      }
      n = (L + ck - 1) / ck;
    }
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = s_carry + scan[tid] - n;
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
      a.seqs[2 * b] = n;
      a.seqs[2 * b + 1] = first;
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
    if (tid == blockDim.x - 1) s_carry += scan[tid];
    __syncthreads();
  }
  if (tid == 0) {
    a.header[0] = min(s_carry, a.max_units);
    a.header[1] = chunk;
  }
}

// Merge the split partials of every sequence whose split count is not 1.  The partials are in
// the decode kernel's fragment order: slot block (unit, set, 32-head block) holds 32 heads x d_v
// values as [column block][piece][lane][value], where a piece is the 8 (bf16) or 4 (f32)
// consecutive accumulator registers of one lane: register i of lane l holds head l % 32 and
// column 32 * cb + 8 * (i / 4) + 4 * (l / 32) + i % 4.
// A work group takes 64 consecutive piece positions of one sequence (one 1 KB load per split) and
// its four waves split the sequence's splits between them; the waves' sums are added in LDS in a
// fixed order, so the result does not depend on timing.
constexpr int kCombineThreads = 256;
constexpr int kCombineWaves = kCombineThreads / 64;
constexpr int kCombineFewSplits = 8;  // at most this many splits: one wave merges a piece group alone

__global__ __launch_bounds__(kCombineThreads) void combine_ws_kernel(DecodeArgs a, int d_v) {
  __shared__ float red_m[kCombineWaves][64];
  __shared__ float red_o[kCombineWaves][8][64];
  const int b = blockIdx.y;
  int n = a.seqs[2 * b];
  if (n == 1) return;
  const int first = a.seqs[2 * b + 1];
  n = max(0, min(n, a.max_units - first));  // the planner never exceeds the workspace; stay inside it regardless
  const int vals = a.part_bf16 ? 8 : 4;     // values per piece
  const int jn = 16 / vals;                 // pieces per lane and column block
  const int cbn = d_v / 32;
  const int HB = a.hblocks;
  const int G = a.groups;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // piece position p = blockIdx.x * 64 + lane (the piece count per unit is a multiple of 64)
  int rest = blockIdx.x;
  const int j = rest % jn;
  rest /= jn;
  const int cb = rest % cbn;
  rest /= cbn;
  const int hb = rest % HB;
  const int gs = rest / HB;
  const int head_in_set = hb * 32 + (lane & 31);
  const int h = lane >> 5;
  const size_t blk_in_unit = (size_t)gs * HB + hb;
  const size_t blocks_per_unit = (size_t)G * HB;
  auto lse_of = [&](int s) { return a.part_lse[((first + s) * blocks_per_unit + blk_in_unit) * 32 + (lane & 31)]; };

  const size_t piece_off = ((size_t)(cb * jn + j) * 64 + lane) * vals;
  // this wave's share (splits s0, s0 + step, ...) of the weighted sum, loads unrolled for overlap
  auto accumulate = [&](int s0, int step, float lse, float* o) {
#pragma unroll 8
    for (int s = s0; s < n; s += step) {
      const float w = expf(lse_of(s) - lse);
      const size_t off = ((first + s) * blocks_per_unit + blk_in_unit) * (size_t)(32 * d_v) + piece_off;
      if (a.part_bf16) {
        typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
        const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(static_cast<const __bf16*>(a.part_out) + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += w * (float)v[e];
      } else {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.part_out) + off);
        o[0] += w * v.x;
        o[1] += w * v.y;
        o[2] += w * v.z;
        o[3] += w * v.w;
      }
    }
  };
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse;
  if (n <= kCombineFewSplits) {
    // few splits: one wave does the whole piece group, no cross-wave reduction
    if (wave != 0) return;
    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, lse_of(s));
    float tot = 0.f;
    if (M != -INFINITY)
      for (int s = 0; s < n; ++s) tot += expf(lse_of(s) - M);
    lse = (M == -INFINITY) ? -INFINITY : M + logf(tot);
    if (M != -INFINITY) accumulate(0, 1, lse, o);
    if (head_in_set >= a.heads_per_set) return;
  } else {
    // combined lse of this lane's head
    float M = -INFINITY;
#pragma unroll 4
    for (int s = wave; s < n; s += kCombineWaves) M = fmaxf(M, lse_of(s));
    red_m[wave][lane] = M;
    __syncthreads();
    M = red_m[0][lane];
#pragma unroll
    for (int w = 1; w < kCombineWaves; ++w) M = fmaxf(M, red_m[w][lane]);
    __syncthreads();
    float tot = 0.f;
#pragma unroll 4
    for (int s = wave; s < n; s += kCombineWaves) tot += expf(lse_of(s) - M);
    red_m[wave][lane] = tot;
    __syncthreads();
    tot = 0.f;
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) tot += red_m[w][lane];
    lse = M + logf(tot);  // n > kCombineFewSplits >= 1 non-empty splits: M is finite
    accumulate(wave, kCombineWaves, lse, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[wave][e][lane] = o[e];
    __syncthreads();
    if (wave != 0 || head_in_set >= a.heads_per_set) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = red_o[0][e][lane];
#pragma unroll
      for (int w = 1; w < kCombineWaves; ++w) t += red_o[w][e][lane];
      o[e] = t;
    }
  }
  const int row = a.mlra ? head_in_set * G + gs : gs * a.heads_per_set + head_in_set;
  const size_t orow = (size_t)b * a.rows + row;
  if (cb == 0 && j == 0 && h == 0) a.lse[orow] = lse;
  // value e of piece j is register i = vals * j + e: column 32 cb + 8 (i / 4) + 4 h + i % 4
  for (int q = 0; q < vals / 4; ++q) {
    const int i0 = vals * j + 4 * q;
    const int c = cb * 32 + 8 * (i0 / 4) + 4 * h;
    if (a.out_bf16) {
      typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
      bf16x4_t v = {(__bf16)o[4 * q], (__bf16)o[4 * q + 1], (__bf16)o[4 * q + 2], (__bf16)o[4 * q + 3]};
      *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(a.out) + orow * d_v + c) = v;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow * d_v + c) =
          make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
  }
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
    for (int s = 0; s < n; ++s) M = fmaxf(M, ls[s]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = -INFINITY;
    if (M != -INFINITY) {
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
  const int pieces = a.groups * a.hblocks * (d_v / 32) * (a.part_bf16 ? 2 : 4) * 64;
  const dim3 grid(pieces / 64, a.batch);
  hipLaunchKernelGGL(combine_ws_kernel, grid, dim3(kCombineThreads), 0, static_cast<hipStream_t>(stream), a, d_v);
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
