// Append of one decode step's new token to the paged latent cache (gfx950).  See ld_cache_append
// in include/latent_decode.h for the operation and its sources.
//
// One work group per sequence.  The token goes to logical position L - 1 of a sequence of length L
// (page block_table[L-1 / page], slot (L-1) % page).  Its latent row (all groups) is copied into
// the cache dtype, or, for an fp8 cache, quantised with one scale per token: the work group's
// threads reduce the row's amax, scale = amax / 448 (fp32), every element becomes the E4M3 code
// nearest to latent / scale (fp32 division, clamped to +-448, ties to the even code).  The RoPE key
// is rotated by position L - 1: pair i turns by (L-1) * base^(-2i/d_rope), with the angle, its cosine
// and sine, and the rotation in fp64 (an angle of a million radians in fp32 would be off by
// tenths of a radian), then rounded to the cache dtype (bf16 for an fp8 cache's rope pool).
#include <hip/hip_runtime.h>

#include <cmath>

#include "ld_internal.h"

namespace ld {
namespace {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ float load_in(const void* p, size_t i, int in_bf16) {
  return in_bf16 ? (float)static_cast<const __bf16*>(p)[i] : static_cast<const float*>(p)[i];
}

// OCP E4M3 code of y (finite, |y| <= 448) by round to nearest, ties to even: the quantum of y's
// binade is 2^(e-3) (2^-9 below the smallest normal 2^-6), y / quantum is exact in fp32, and rintf
// rounds it to the nearest integer with ties to even; the rounded value is then encoded.
__device__ __forceinline__ unsigned e4m3_code(float y) {
  const unsigned sign = (__float_as_uint(y) >> 31) << 7;
  const float a = fabsf(y);
  const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // exponent of a normal fp32
  const float q = a < 0x1p-6f ? 0x1p-9f : ldexpf(1.f, e - 3);
  const float r = rintf(a / q) * q;
  unsigned code;
  if (r < 0x1p-6f) {
    code = (unsigned)(r * 512.f);                                   // subnormal: r = m * 2^-9
  } else {
    const int er = (int)((__float_as_uint(r) >> 23) & 0xFF) - 127;
    const unsigned m = (unsigned)((r * ldexpf(1.f, -er) - 1.f) * 8.f);
    code = ((unsigned)(er + 7) << 3) | m;
  }
  return code | sign;
}

template <int KV>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  __shared__ float red[kAppendThreads / 64];
  const int b = blockIdx.x;
  // A write goes only where the metadata says the token lives: a length outside [1, capacity] or a
  // page id outside the pool leaves the cache untouched (clamping would overwrite another slot,
  // possibly another sequence's).
  const int cap = a.max_pages * a.page_size;
  const int L = a.seq_lens[b];
  if (L < 1 || L > cap) return;
  const int pos = L - 1;
  const int page = a.block_table[(size_t)b * a.max_pages + pos / a.page_size];
  if (page < 0 || page >= a.num_pages) return;
  const size_t slot = (size_t)page * a.page_size + pos % a.page_size;
  const int D = a.d_lat;   // all groups
  const int DR = a.d_rope;
  const int tid = threadIdx.x;
  const size_t in_row = (size_t)b * D;

  if constexpr (KV == LD_FP8_E4M3) {
    float amax = 0.f;
    for (int i = tid; i < D; i += kAppendThreads) amax = fmaxf(amax, fabsf(load_in(a.c_new, in_row + i, a.in_bf16)));
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;
    unsigned char* codes = static_cast<unsigned char*>(a.k) + slot * D;
    for (int i = tid; i < D; i += kAppendThreads) {
      const float y = fminf(fmaxf(load_in(a.c_new, in_row + i, a.in_bf16) / scale, -448.f), 448.f);
      codes[i] = (unsigned char)e4m3_code(y);
    }
    if (tid == 0) a.scale[slot] = scale;
  } else {
    const size_t row = slot * (size_t)(D + DR);
    for (int i = tid; i < D; i += kAppendThreads) {
      const float v = load_in(a.c_new, in_row + i, a.in_bf16);
      if constexpr (KV == LD_BF16)
        static_cast<__bf16*>(a.k)[row + i] = (__bf16)v;
      else
        static_cast<float*>(a.k)[row + i] = v;
    }
  }

  for (int i = tid; i < DR / 2; i += kAppendThreads) {
    const double inv = pow((double)a.rope_base, -2.0 * i / DR);
    const double ang = (double)pos * inv;
    const double c = cos(ang), s = sin(ang);
    const double x0 = load_in(a.kr_new, (size_t)b * DR + 2 * i, a.in_bf16);
    const double x1 = load_in(a.kr_new, (size_t)b * DR + 2 * i + 1, a.in_bf16);
    const double y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
    if constexpr (KV == LD_FP8_E4M3) {
      __bf16* dst = static_cast<__bf16*>(a.rope) + slot * DR + 2 * i;
      dst[0] = (__bf16)(float)y0;
      dst[1] = (__bf16)(float)y1;
    } else if constexpr (KV == LD_BF16) {
      __bf16* dst = static_cast<__bf16*>(a.k) + slot * (size_t)(D + DR) + D + 2 * i;
      dst[0] = (__bf16)(float)y0;
      dst[1] = (__bf16)(float)y1;
    } else {
      float* dst = static_cast<float*>(a.k) + slot * (size_t)(D + DR) + D + 2 * i;
      dst[0] = (float)y0;
      dst[1] = (float)y1;
    }
  }
}

}  // namespace

int launch_append(const AppendArgs& a, int kv_dtype, void* stream) {
  if (a.batch == 0) return 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kv_dtype == LD_FP8_E4M3)
    hipLaunchKernelGGL(append_kernel<LD_FP8_E4M3>, dim3(a.batch), dim3(kAppendThreads), 0, s, a);
  else if (kv_dtype == LD_BF16)
    hipLaunchKernelGGL(append_kernel<LD_BF16>, dim3(a.batch), dim3(kAppendThreads), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<LD_F32>, dim3(a.batch), dim3(kAppendThreads), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace ld
