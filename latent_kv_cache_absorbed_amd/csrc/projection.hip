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

#include <atomic>

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

// Staged form for k <= 512 (k % 64 == 0) and n % 64 == 0: a work group takes one head and 64 output
// columns; it copies the 64 weight rows w[h, n0 .. n0 + 63, :] and 64 activation rows a[m0 .. m0 + 63,
// h, :] whole into LDS with 1 KB global -> LDS copies (each row's 16-byte chunks land XOR-swizzled by
// the row's three low bits: chunk c of row r sits in slot c ^ (r & 7), so the eight rows an MFMA
// operand read touches in one cycle fall in distinct banks), then each of its four waves computes a
// 32 x 32 C^T tile (columns 32 (wave & 1) .., rows 32 (wave >> 1) ..) from LDS.  One load burst per work
// group, every byte fetched once by it; the weights stay in LDS across row tiles.
template <int OUT_BF16>
__global__ __launch_bounds__(kProjThreads) void head_projection_staged_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nblocks = a.n / 64;
  const int h = blockIdx.x / nblocks;
  const int n0 = (blockIdx.x % nblocks) * 64;
  const int RB = a.k * 2;                 // bytes of a row (all k)
  const int region = 64 * RB;             // LDS bytes of 64 rows
  char* const lw = smem;
  char* const la = smem + region;
  const int blocks = region / 1024;       // 1 KB copies per region
  // copy q of a region (lane i): region bytes [1024 q + 16 i, +16) = row r, slot p; it holds chunk
  // (p & ~7) | ((p & 7) ^ (r & 7)) of that row
  auto copy_region = [&](char* dst, const char* base, size_t row_stride, int rows_valid) {
    for (int q = wave; q < blocks; q += kProjThreads / 64) {
      const int off = q * 1024 + lane * 16;
      const int r = off / RB;
      const int p = (off % RB) >> 4;
      const int c = (p & ~7) | ((p & 7) ^ (r & 7));
      const unsigned voff = (unsigned)((size_t)min(r, rows_valid - 1) * row_stride) + (unsigned)(c << 4);
      dma16(base, voff, dst + q * 1024);
    }
  };
  const char* wbase = static_cast<const char*>(a.w) + ((size_t)h * a.n + n0) * (size_t)RB;
  copy_region(lw, wbase, (size_t)RB, 64);
  const int wn = wave & 1, wm = wave >> 1;
  const int col = lane & 31, hh = lane >> 5;
  const int nr = 32 * wn + col;           // this lane's weight row (A operand row) in the region
  for (int m0 = 0; m0 < a.m; m0 += 64) {
    const char* abase = static_cast<const char*>(a.a) + ((size_t)m0 * a.heads + h) * (size_t)RB;
    copy_region(la, abase, (size_t)a.heads * RB, min(64, a.m - m0));
    __syncthreads();                      // every copy has landed
    const int mr = 32 * wm + col;         // this lane's activation row (B operand column) in the region
    floatx16 acc = floatx16{};
    const int ksteps = a.k / 16;
    for (int s = 0; s < ksteps; ++s) {
      const int c = 2 * s + hh;           // chunk of k-step s held by this lane half
      const bf16x8_t wf = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(lw + nr * RB + (((c & ~7) | ((c & 7) ^ (nr & 7))) << 4)));
      const bf16x8_t af = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(la + mr * RB + (((c & ~7) | ((c & 7) ^ (mr & 7))) << 4)));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, af, acc, 0, 0, 0);
    }
    // C^T tile: lane holds row m0 + mr and columns n0 + 32 wn + 8 (r / 4) + 4 hh + r % 4
    const int m = m0 + mr;
    if (m < a.m) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const size_t o = ((size_t)m * a.heads + h) * a.n + n0 + 32 * wn + 8 * g + 4 * hh;
        if constexpr (OUT_BF16) {
          *reinterpret_cast<bf16x4_t*>(static_cast<__bf16*>(a.c) + o) =
              bf16x4_t{(__bf16)acc[4 * g], (__bf16)acc[4 * g + 1], (__bf16)acc[4 * g + 2], (__bf16)acc[4 * g + 3]};
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.c) + o) =
              make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
        }
      }
    }
    __syncthreads();                      // the activation rows are rewritten for the next row tile
  }
}

}  // namespace

int launch_head_projection(const ProjArgs& a, int out_bf16, void* stream) {
  if (a.m == 0) return 0;
  // staged form: k <= 512 (two 64-row regions of k * 2 bytes fit in LDS), 64-column blocks, and the
  // activation rows of a 64-row tile addressable by 32-bit offsets from the tile's first row
  if (a.k % 64 == 0 && a.k <= 512 && a.n % 64 == 0 && 64LL * a.heads * a.k * 2 < (1LL << 31)) {
    const dim3 grid((unsigned)((long long)a.heads * (a.n / 64)));
    const size_t lds = (size_t)2 * 64 * a.k * 2;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // more than 64 KB of dynamic LDS needs the kernel's limit raised, once per kernel and device (a
    // repeated call is harmless, so threads racing here are fine)
    static std::atomic<bool> raised[2][kMaxDevices] = {};
    const void* f = out_bf16 ? reinterpret_cast<const void*>(head_projection_staged_kernel<1>)
                             : reinterpret_cast<const void*>(head_projection_staged_kernel<0>);
    if (lds > 65536) {
      int dev = 0;
      const hipError_t ed = hipGetDevice(&dev);
      if (ed != hipSuccess) return (int)ed;
      std::atomic<bool>* flag = dev >= 0 && dev < kMaxDevices ? &raised[out_bf16 ? 1 : 0][dev] : nullptr;
      if (!flag || !flag->load(std::memory_order_relaxed)) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
        if (e != hipSuccess) return (int)e;
        if (flag) flag->store(true, std::memory_order_relaxed);
      }
    }
    if (out_bf16)
      hipLaunchKernelGGL((head_projection_staged_kernel<1>), grid, dim3(kProjThreads), lds, s, a);
    else
      hipLaunchKernelGGL((head_projection_staged_kernel<0>), grid, dim3(kProjThreads), lds, s, a);
    return (int)hipGetLastError();
  }
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
