// Device-side building blocks shared by the decode kernels (gfx950): MFMA operand layouts, the
// LDS row swizzle, global->LDS stage copies, waits and barriers, cross-lane helpers, and the exact
// fp8 E4M3 -> bf16 conversion.  Included by the kernel sources only.
#ifndef LD_DECODE_COMMON_H
#define LD_DECODE_COMMON_H

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ld_internal.h"

namespace ld {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

enum KvT : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

constexpr float kLn2 = 0.69314718055994530942f;
// The running max is raised only when a stage's max exceeds it by more than this (log2 units),
// so O is rescaled rarely; scores then stay <= 2^8 above the stale max, far from overflow.
constexpr float kRescaleSlack = 8.f;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i%4 of the
// 8-byte loads of lanes 4k + i/4, k = 0..3 (so four lanes that load four consecutive
// elements of four rows hand every lane one column of those rows).
__device__ __forceinline__ bf16x4_t lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at
// their no-wait maxima).  Counts above the 6-bit field's 63 wait for 63 instead (a stricter wait).
template <int N0>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int N = N0 > 63 ? 63 : N0;
  static_assert(N >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Work-group barrier that orders LDS only.  __syncthreads() also fences global memory, which
// makes every wave drain all in-flight global->LDS copies (vmcnt 0) and defeats the stage
// pipeline; here the caller waits for exactly the copies it needs (wait_vmcnt) first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The pipelined kernels (decode_pipe.hip, decode_pipe_fp8.hip) use a fixed softmax reference per
// unit: p = 2^(s - r) may reach 2^kRefSlack before the unit is run again with the exact max, far
// below the fp32 / bf16 range, so sums of up to 2^20 stages x 32 tokens of such values stay finite.
constexpr float kRefSlack = 64.f;

// P.V MFMA accumulating into AGPRs.  The pipelined kernels' score MFMAs are compiler builtins with
// their results in VGPRs (the softmax reads them), and one function holds one MFMA register form,
// so the P.V MFMAs, whose accumulators sit in the AGPRs, are written out.
__device__ __forceinline__ void mfma_pv(floatx16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same MFMA for an A operand computed by VALU instructions just before it (the fp8 values
// converted to bf16): the compiler inserts no wait states ahead of an inline-asm MFMA, so the
// VALU-write -> MFMA-read distance the hardware needs is written out.
__device__ __forceinline__ void mfma_pv_valu_a(floatx16& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states after the last P.V MFMA before its accumulators are read or rewritten.
__device__ __forceinline__ void mfma_pv_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// 16-byte global -> LDS copy per lane; the LDS destination of lane i is lds + 16 i.
__device__ __forceinline__ void dma16(const char* base, unsigned voff, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(base + voff, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
}

// The same copy written out (global_load_lds_dwordx4; M0 holds the wave's LDS address).  The
// compiler models the builtin copy as a flat access that may also count in lgkmcnt, and then waits
// for every LDS read in flight (lgkmcnt(0)) before each use of any of them, which exposes the LDS
// latency of every MFMA operand; the written-out copy leaves its LDS-read waits exact.  The copy
// counts in vmcnt only, and nothing of it is visible to the compiler: a kernel that uses it waits for
// its copies itself (wait_vmcnt, then a barrier) before any wave reads the stage, and uses M0 for
// nothing else.  lds_wave_base must be a direct pointer into a __shared__ array (so that its LDS
// address folds to a constant plus an offset); dma16_asm_at takes that LDS address as a number.
__device__ __forceinline__ void dma16_asm_at(const char* base, unsigned voff, unsigned lds) {
  const unsigned long long b = (unsigned long long)(uintptr_t)base;
  const unsigned long long bs = ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) << 32) |
                                (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved; the kernels using this copy use it for nothing else
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
               :
               : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(bs)
               : "memory", "m0");
#pragma clang diagnostic pop
}
__device__ __forceinline__ void dma16_asm(const char* base, unsigned voff, char* lds_wave_base) {
  dma16_asm_at(base, voff, (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)(lds_wave_base));
}

// ------------------------------------------------------------------------------------------
// MFMA traits: fp32 caches use v_mfma_f32_32x32x2_f32 (one element per lane and k-step),
// bf16 and fp8 caches use v_mfma_f32_32x32x16_bf16 (eight elements per lane and k-step).
// A operand: lane l holds row l%32, k = (l/32)*EPL + [0, EPL).  B operand: k likewise,
// column l%32.  C: lane l holds column l%32, rows 8*(i/4) + 4*(l/32) + i%4 for i < 16.
// ------------------------------------------------------------------------------------------
template <int KV>
struct Mma;

template <>
struct Mma<KV_BF16> {
  using CT = __bf16;
  using Frag = bf16x8_t;
  static constexpr int KSTEP = 16;
  static constexpr int EPL = 8;
  static constexpr int PSTEPS = 2;  // k-steps over a 32-token stage in P.V
  // token held by C register i of lane half h
  static __device__ __forceinline__ int token_of(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }
  // token that S row r stands for (swap bits 2 and 3)
  static __device__ __forceinline__ int row_token(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
  static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma<KV_FP8> : Mma<KV_BF16> {};

template <>
struct Mma<KV_F32> {
  using CT = float;
  using Frag = float;
  static constexpr int KSTEP = 2;
  static constexpr int EPL = 1;
  static constexpr int PSTEPS = 16;
  static __device__ __forceinline__ int token_of(int i, int h) { return 2 * i + h; }
  static __device__ __forceinline__ int row_token(int r) { return (r & 24) | ((r & 3) << 1) | ((r >> 2) & 1); }
  static __device__ __forceinline__ floatx16 mma(Frag a, Frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Value of lane l ^ 32 (the other half of the wave), through v_permlane32_swap (a VALU op)
// rather than an LDS round trip: swapping a copy of x with itself leaves lanes 32..63 of the
// first result holding lanes 0..31 of x, and lanes 0..31 of the second holding lanes 32..63.
__device__ __forceinline__ float xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (__lane_id() < 32) ? r[1] : r[0]);
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Chunk swizzle of an LDS row: the low bits (mask m, at most four bits) of the 16-byte chunk
// index are XORed with a key of the row's token t, key bits = (t2^t3, t0, t1, t3^t0).  The key
// is a bijection on every 16 consecutive rows, and its bits 2 and 3 take four distinct values on
// every 4 consecutive rows.  So neither the S-operand reads (16 lanes of a cycle cover 16
// distinct rows mod 16, one chunk each) nor the transposed V reads (4 consecutive rows x 4
// chunks per 16 lanes) hit a bank twice, whether the LDS serves 16 lanes a cycle over 64 banks
// or 8 lanes over 32 banks.
__host__ __device__ constexpr int swz_mask(int rb) {
  return rb >= 256 ? 15 : rb >= 128 ? 7 : rb >= 64 ? 3 : rb >= 32 ? 1 : 0;
}
__device__ __forceinline__ int swz_key(int t) {
  return (((t >> 2) ^ (t >> 3)) & 1) | ((t & 1) << 1) | (((t >> 1) & 1) << 2) | ((((t >> 3) ^ t) & 1) << 3);
}
__device__ __forceinline__ int lds_off(int t, int rb, int m, int byte_in_row) {
  const int c = byte_in_row >> 4;
  return t * rb + ((((c & m) ^ (swz_key(t) & m)) | (c & ~m)) << 4) + (byte_in_row & 15);
}

// fp8 E4M3 (OCP) -> bf16, exact: v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes
// straight to two bf16 (every E4M3 value is a bf16 value).  (Converting through
// v_cvt_pk_f32_fp8 and repacking the f32 halves was mis-combined by the compiler into a copy
// of one half, so the direct conversion is used.)
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(unsigned lo, unsigned hi) {
  const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return make_uint4(__builtin_bit_cast(unsigned, a0), __builtin_bit_cast(unsigned, a1),
                    __builtin_bit_cast(unsigned, b0), __builtin_bit_cast(unsigned, b1));
}

// One region of a stage: kTile rows of RB bytes (swizzle mask MSK), filled by 1 KB DMA blocks.
// Block q covers region bytes [1024q, 1024q + 1024); lane i lands at byte 1024q + 16i.  Blocks
// are dealt to the NW waves round-robin across all regions of a stage (FIRST is this region's
// first block in that order), so every wave issues the floor or the ceiling of blocks / NW.
// Global source: stage token t's row starts at rows + min(t, tlast) * row_bytes (rows past the
// unit's end repeat its last row), and logical LDS row byte b comes from byte col(b) of it.  The
// address is formed as a wave-uniform 64-bit base plus a 32-bit per-lane offset, which the copy
// instruction takes as an SGPR pair and one VGPR.
template <int RB, int MSK, int NW, int FIRST, class ColFn, bool ASM = false>
__device__ __forceinline__ void dma_region(char* region, int wave, int lane, const char* rows, int row_bytes, int tlast,
                                           ColFn col, std::integral_constant<bool, ASM> = {}) {
  constexpr int blocks = kTile * RB / 1024;
  constexpr int iters = (blocks + NW - 1) / NW;
  constexpr int shift = FIRST % NW;
  constexpr int CPR = RB / 16;  // 16-byte chunks per row
  const int q0 = wave >= shift ? wave - shift : wave - shift + NW;
#pragma unroll
  for (int i = 0; i < iters; ++i) {
    const int q = q0 + i * NW;
    if (blocks % NW == 0 || q < blocks) {
      const int t_first = (q * 1024) / RB;                                    // wave-uniform
      const int t = RB >= 1024 ? t_first : t_first + lane / CPR;              // this lane's row
      const int cp = RB >= 1024 ? ((q * 1024) % RB) / 16 + lane : lane % CPR;  // physical chunk in it
      const int c = (cp & ~MSK) | ((cp & MSK) ^ (swz_key(t) & MSK));           // logical chunk it holds
      const int tu = min(t_first, tlast);
      unsigned voff = (unsigned)((min(t, tlast) - tu) * row_bytes + col(c << 4));
      asm volatile("" : "+v"(voff));  // computed here, not hoisted as a 64-bit address per block
      if constexpr (ASM)
        dma16_asm(rows + (size_t)tu * row_bytes, voff, region + q * 1024);
      else
        dma16(rows + (size_t)tu * row_bytes, voff, region + q * 1024);
    }
  }
}

}  // namespace
}  // namespace ld

#endif  // LD_DECODE_COMMON_H
