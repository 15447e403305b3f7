// Per-head projections around the absorbed decode step (gfx950): C[m, h, n] = sum_k W[h, n, k] A[m, h, k]
// with bf16 operands and fp32 accumulation (v_mfma_f32_32x32x16_bf16).  See ld_head_projection in
// include/latent_decode.h for the operation and its sources.
//
// One wave computes a 32-column tile n0 .. n0+31 of one head for every row m, two 32-row tiles at a
// time, as C^T tiles (weights as the A operand), so each lane stores four consecutive columns at once.  Both operands are read straight from memory as MFMA fragments: the activation row m holds
// its K values contiguously and so does the weight row n (W[h] is stored [N, K]), so every lane
// loads 16 contiguous bytes per k-step.  The weights, which dominate the bytes (H*N*K), are read
// once per pair of row tiles; the operands of eight k-steps are loaded before their MFMAs issue.
#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "ld_internal.h"

namespace ld {
namespace {

constexpr int kProjThreads = 256;
constexpr int kKChunk = 8;  // k-steps whose operands are loaded together

__device__ __forceinline__ bf16x8_t load_frag(const __bf16* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// KS waves of a work group share one (head, 32-column tile) and split its k-steps KS ways; with
// KS = 1 the four waves take four tiles.  Partial sums meet in LDS; the first wave adds them.
template <int OUT_BF16, int KS>
__global__ __launch_bounds__(kProjThreads) void head_projection_kernel(ProjArgs a) {
  constexpr int WAVES = kProjThreads / 64;
  __shared__ floatx16 part[KS > 1 ? (KS - 1) * 2 * 64 : 1];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ntiles = a.n / 32;
  const long long gw = (long long)blockIdx.x * (WAVES / KS) + wave / KS;   // the tile of this wave
  const int kq = wave % KS;                                                  // its share of the k-steps
  const bool live = gw < (long long)a.heads * ntiles;                        // uniform per tile
  const long long gt = live ? gw : 0;
  const int h = (int)(gt / ntiles);
  const int n0 = (int)(gt % ntiles) * 32;
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int ksteps = a.k / 16;
  const int per = (ksteps + KS - 1) / KS;
  const int kb = min(kq * per, ksteps), ke = min(kb + per, ksteps);
  const __bf16* A = static_cast<const __bf16*>(a.a);
  const __bf16* wrow = static_cast<const __bf16*>(a.w) + ((size_t)h * a.n + n0 + col) * a.k + hh * 8;
  const bf16x8_t zero = __builtin_bit_cast(bf16x8_t, make_uint4(0u, 0u, 0u, 0u));
  for (int mt = 0; mt < a.m; mt += 64) {
    const bool two = mt + 32 < a.m;  // uniform: a second row tile
    const int r0 = mt + col, r1 = mt + 32 + col;
    const bool v0 = r0 < a.m, v1 = two && r1 < a.m;
    const __bf16* a0 = A + ((size_t)(v0 ? r0 : 0) * a.heads + h) * a.k + hh * 8;
    const __bf16* a1 = A + ((size_t)(v1 ? r1 : 0) * a.heads + h) * a.k + hh * 8;
    floatx16 acc0 = floatx16{}, acc1 = floatx16{};
    if (live) {
      for (int s0 = kb; s0 < ke; s0 += kKChunk) {
        bf16x8_t wf[kKChunk], f0[kKChunk], f1[kKChunk];
#pragma unroll
        for (int j = 0; j < kKChunk; ++j) {
          const int s = min(s0 + j, ke - 1);  // steps past the share repeat its last (not used)
          wf[j] = load_frag(wrow + s * 16);
          f0[j] = v0 ? load_frag(a0 + s * 16) : zero;
          f1[j] = v1 ? load_frag(a1 + s * 16) : zero;
        }
#pragma unroll
        for (int j = 0; j < kKChunk; ++j) {
          if (s0 + j < ke) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], f0[j], acc0, 0, 0, 0);
            if (two) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], f1[j], acc1, 0, 0, 0);
          }
        }
      }
    }
    if constexpr (KS > 1) {
      // partial sums of the k shares, added in share order by the tile's first wave; every wave
      // passes both barriers
      if (kq > 0) {
        part[((kq - 1) * 2 + 0) * 64 + lane] = acc0;
        part[((kq - 1) * 2 + 1) * 64 + lane] = acc1;
      }
      __syncthreads();
      if (kq == 0) {
#pragma unroll
        for (int q = 1; q < KS; ++q) {
          acc0 += part[((q - 1) * 2 + 0) * 64 + lane];
          acc1 += part[((q - 1) * 2 + 1) * 64 + lane];
        }
      }
    }
    // C^T tiles (the weight rows are the A operand): lane holds row m = mt + col (32 further for acc1)
    // and columns n0 + 8 (r / 4) + 4 hh + r % 4, so four consecutive registers are four consecutive
    // columns of one output row, written by one 8-byte (bf16) or 16-byte (f32) store
    if (live && kq == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t == 1 && !two) break;
        const int m = mt + 32 * t + col;
        if (m < a.m) {
          const floatx16& acc = t == 0 ? acc0 : acc1;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const size_t o = ((size_t)m * a.heads + h) * a.n + n0 + 8 * g + 4 * hh;
            if constexpr (OUT_BF16) {
              *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(a.c) + o) =
                  bf16x4_t{(__bf16)acc[4 * g], (__bf16)acc[4 * g + 1], (__bf16)acc[4 * g + 2], (__bf16)acc[4 * g + 3]};
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(a.c) + o) =
                  make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
            }
          }
        }
      }
    }
    if constexpr (KS > 1) __syncthreads();  // the partials are rewritten by the next row tiles
  }
}

}  // namespace

int launch_head_projection(const ProjArgs& a, int out_bf16, void* stream) {
  if (a.m == 0) return 0;
  constexpr int WAVES = kProjThreads / 64;
  const long long tiles = (long long)a.heads * (a.n / 32);
  // a long k is split over the four waves of a work group (one tile each), a short one is not
  const bool split = a.k / 16 >= 2 * kKChunk;
  const dim3 grid((unsigned)(split ? tiles : (tiles + WAVES - 1) / WAVES));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (split) {
    if (out_bf16)
      hipLaunchKernelGGL((head_projection_kernel<1, WAVES>), grid, dim3(kProjThreads), 0, s, a);
    else
      hipLaunchKernelGGL((head_projection_kernel<0, WAVES>), grid, dim3(kProjThreads), 0, s, a);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((head_projection_kernel<1, 1>), grid, dim3(kProjThreads), 0, s, a);
    else
      hipLaunchKernelGGL((head_projection_kernel<0, 1>), grid, dim3(kProjThreads), 0, s, a);
  }
  return (int)hipGetLastError();
}

}  // namespace ld
