// Decode-attention kernels for gfx950 (CDNA4): one query token per sequence against a paged,
// shrunk KV cache.  See include/latent_decode.h for the operation and its sources.
//
// Work decomposition.  A work unit is (sequence b, token chunk [t_begin, t_end)) from the
// split-KV planner.  A "set" is a group of query heads that score against the same cached
// rows: all H heads for MLA, one latent group for GLA, one branch for MLRA, one kv head for
// GQA/GTA, all heads for MQA.  A work group handles NSETS sets of one unit; each of its
// WAVES waves owns one set and 32 of that set's heads.  Per 32-token stage the work group
// copies the rows it needs into LDS once (asynchronous global->LDS DMA, double-buffered, so
// stage n+1 streams in while stage n is computed), and every wave reads them from there:
//
//   S^T[token, head] = K_stage . Q^T           (v_mfma_f32_32x32x16_bf16; Q stays in VGPRs)
//   online softmax over the token axis         (each lane owns one head: 16 scores here and
//                                               16 in the lane 32 apart)
//   O^T[col, head]  += V_stage^T . P^T          (same MFMA; P never leaves registers; the V^T
//                                               operand comes from ds_read_b64_tr_b16)
//
// The rows of the S MFMA are a fixed permutation of the stage's tokens, chosen so that the
// score layout the MFMA writes is exactly the P^T operand layout the PV MFMA reads.
//
// LDS layout of one stage buffer (row-major, 16-byte chunks XOR-swizzled per row):
//   latent region [32][NSETS*DL]  (GQA/MQA/GTA: the K rows of the NSETS kv heads)
//   rope region   [32][DR]        (latent variants)
//   V region      [32][NSETS*DL]  (GQA/MQA only)
//   scales        [32] f32        (fp8 cache only)
// An fp8 cache is staged through registers (codes -> bf16, exact) instead of DMA.
#include <hip/hip_runtime.h>

#include "ld_internal.h"

namespace ld {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
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

// 16-byte global -> LDS copy per lane; the LDS destination of lane i is lds + 16 i.
__device__ __forceinline__ void dma16(const void* gsrc, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_wave_base), 16, 0, 0);
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

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Chunk swizzle of an LDS row of `rb` bytes: the low bits of the 16-byte chunk index are XORed
// with key(t) = 2*(t%4) + bit 3 of t.  The 8 storage rows one S-operand read serves per cycle
// ({0,1,2,3,8,9,10,11} + 4j, see row_token) get 8 distinct keys, and the 4 consecutive rows a
// transposed V read touches get keys that differ above bit 0, so neither read pattern has bank
// conflicts.
__host__ __device__ constexpr int swz_mask(int rb) { return rb >= 128 ? 7 : rb >= 64 ? 3 : rb >= 32 ? 1 : 0; }
__device__ __forceinline__ int swz_key(int t) { return ((t & 3) << 1) | ((t >> 3) & 1); }
__device__ __forceinline__ int lds_off(int t, int rb, int byte_in_row) {
  const int m = swz_mask(rb);
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

// ------------------------------------------------------------------------------------------
// compile-time shape of one kernel instance
// ------------------------------------------------------------------------------------------
template <int KV, int DL, int DR, int KIND, int NSETS, int WAVES>
struct Cfg {
  using M = Mma<KV>;
  using CT = typename M::CT;
  static constexpr int ES = sizeof(CT);                       // LDS element bytes (fp8 staged as bf16)
  static constexpr int GES = (KV == KV_FP8) ? 1 : ES;         // global latent element bytes
  static constexpr int THREADS = WAVES * kWaveSize;
  static constexpr int DK = DL + DR;                          // score dims per set
  static constexpr int KS = DK / M::KSTEP;                    // k-steps of S
  static constexpr int CB = DL / 32;                          // 32-column blocks of O
  static constexpr int LW = NSETS * DL * ES;                  // latent / K row bytes in LDS
  static constexpr int RW = DR * ES;                          // rope row bytes in LDS
  static constexpr int VW = (KIND == KIND_SHARED) ? NSETS * DL * ES : 0;
  static constexpr int LAT_OFF = 0;
  static constexpr int ROPE_OFF = kTile * LW;
  static constexpr int V_OFF = ROPE_OFF + kTile * RW;
  static constexpr int SC_OFF = V_OFF + kTile * VW;
  static constexpr int BUF = SC_OFF + ((KV == KV_FP8) ? kTile * 4 : 0);
  static constexpr int BUF_AL = (BUF + 127) / 128 * 128;
  static constexpr int LDS_BYTES = 2 * BUF_AL;
  static constexpr int VRB = (KIND == KIND_SHARED) ? VW : LW;   // row bytes of the V source region
  static constexpr int V_REG = (KIND == KIND_SHARED) ? V_OFF : LAT_OFF;
  static constexpr int FP8_ITEMS = kTile * NSETS * DL / 16;      // 16-code pieces of an fp8 stage
  static constexpr int FP8_PER_THREAD = (KV == KV_FP8) ? (FP8_ITEMS + THREADS - 1) / THREADS : 1;
  static_assert(DK % M::KSTEP == 0 && DL % 32 == 0, "unsupported dims");
  static_assert(pow2(LW) && LW >= 32 && (DR == 0 || (pow2(RW) && RW >= 32)), "row sizes must be powers of two");
  static_assert((kTile * LW) % 1024 == 0 && (kTile * RW) % 1024 == 0, "regions must be whole DMA blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// One region of a stage: kTile rows of RB bytes, filled by 1 KB DMA blocks.  Block q (of
// kTile*RB/1024) covers region bytes [1024q, 1024q + 1024); lane i lands at byte 1024q + 16i.
// `src_row(t)` is the global address of stage token t's row, `src_col(byte)` the byte offset in
// that row of a logical LDS row byte.
template <int RB, class RowFn, class ColFn>
__device__ __forceinline__ void dma_region(char* region, int wave, int nwaves, int lane, RowFn src_row,
                                           ColFn src_col) {
  constexpr int blocks = kTile * RB / 1024;
  constexpr int m = swz_mask(RB);
  for (int q = wave; q < blocks; q += nwaves) {
    const int o = q * 1024 + lane * 16;
    const int t = o >> ilog2(RB);
    const int cp = (o & (RB - 1)) >> 4;                       // physical chunk in the row
    const int c = (cp & ~m) | ((cp & m) ^ (swz_key(t) & m));  // logical chunk it must hold
    dma16(src_row(t) + src_col(c << 4), region + q * 1024);
  }
}

// ------------------------------------------------------------------------------------------
// the decode kernel
// ------------------------------------------------------------------------------------------
template <int KV, int DL, int DR, int KIND, int NSETS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(DecodeArgs a) {
  using C = Cfg<KV, DL, DR, KIND, NSETS, WAVES>;
  using M = typename C::M;
  using CT = typename C::CT;
  using Frag = typename M::Frag;
  constexpr int ES = C::ES;
  constexpr int HB = WAVES / NSETS;  // 32-head blocks per set
  extern __shared__ __attribute__((aligned(16))) char smem[];

  // XCD-aware mapping: all work groups of one unit land on the same XCD (ids = unit mod 8)
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int y = x >> 3;
  const int sb = y % a.wg_per_unit;
  const int unit = (y / a.wg_per_unit) * 8 + xcd;
  if (unit >= a.header[0]) return;
  const Unit u = a.units[unit];
  const int b = u.b;
  const int t_begin = u.t_begin;
  const int t_end = u.t_end;
  const int nsplit = a.seqs[2 * b];

  const int set0 = sb * NSETS;
  const int G = a.groups;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int s = wave / HB;          // wave-uniform
  const int hb = wave - s * HB;
  const int gs = set0 + s;
  const int head_in_set = hb * 32 + col;
  const bool valid = head_in_set < a.heads_per_set;
  const int head = (a.mlra ? 0 : gs * a.heads_per_set) + (valid ? head_in_set : 0);
  const int row = a.mlra ? head * G + gs : head;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  const int page_size = a.page_size;

  // global row geometry (bytes): latent variants store [G latents | rope] per token (fp8: codes
  // only, the rope key lives in its own pool); GQA/MQA/GTA store [G kv heads][DL] per token
  const int grow_bytes = (KIND == KIND_LATENT) ? (G * DL * C::GES + (KV == KV_FP8 ? 0 : DR * ES)) : G * DL * ES;
  const char* kbase = static_cast<const char*>(a.k);

  // ---- issue the copies of one stage into buffer `buf`
  uint4 pre[C::FP8_PER_THREAD];
  float pre_sc = 0.f;
  auto issue_stage = [&](int stage0, char* buf) {
    // every token of a stage lies in one page (stages are page aligned and page_size % 32 == 0)
    const int page = clampi(bt_row[stage0 / page_size], 0, a.num_pages - 1);
    const size_t r0 = (size_t)page * page_size + (stage0 % page_size);
    const int tlast = t_end - 1 - stage0;                  // rows past the unit's end repeat its last row
    if constexpr (KV != KV_FP8) {
      dma_region<C::LW>(buf + C::LAT_OFF, wave, WAVES, lane,
                        [&](int t) { return kbase + (r0 + min(t, tlast)) * (size_t)grow_bytes; },
                        [&](int cb) {
                          const int s2 = cb / (DL * ES);
                          return (set0 + s2) * DL * ES + (cb - s2 * DL * ES);
                        });
    } else {
      // codes -> registers now; converted and written after this stage's compute
#pragma unroll
      for (int r = 0; r < C::FP8_PER_THREAD; ++r) {
        const int i = threadIdx.x + r * C::THREADS;
        if (i < C::FP8_ITEMS) {
          const int t = i / (NSETS * DL / 16);
          const int k16 = i - t * (NSETS * DL / 16);
          const int s2 = (k16 * 16) / DL;
          const int w = k16 * 16 - s2 * DL;
          pre[r] = *reinterpret_cast<const uint4*>(kbase + (r0 + min(t, tlast)) * (size_t)grow_bytes +
                                                   (size_t)(set0 + s2) * DL + w);
        }
      }
      if (threadIdx.x < kTile) pre_sc = a.kscale[r0 + min((int)threadIdx.x, tlast)];
    }
    if constexpr (KIND == KIND_LATENT && DR > 0) {
      if constexpr (KV == KV_FP8) {
        const char* rbase = static_cast<const char*>(a.rope);
        dma_region<C::RW>(buf + C::ROPE_OFF, wave, WAVES, lane,
                          [&](int t) { return rbase + (r0 + min(t, tlast)) * (size_t)(DR * 2); },
                          [&](int cb) { return cb; });
      } else {
        dma_region<C::RW>(buf + C::ROPE_OFF, wave, WAVES, lane,
                          [&](int t) { return kbase + (r0 + min(t, tlast)) * (size_t)grow_bytes; },
                          [&](int cb) { return G * DL * ES + cb; });
      }
    }
    if constexpr (KIND == KIND_SHARED) {
      const char* vbase_g = static_cast<const char*>(a.v);
      dma_region<C::VW>(buf + C::V_OFF, wave, WAVES, lane,
                        [&](int t) { return vbase_g + (r0 + min(t, tlast)) * (size_t)grow_bytes; },
                        [&](int cb) {
                          const int s2 = cb / (DL * ES);
                          return (set0 + s2) * DL * ES + (cb - s2 * DL * ES);
                        });
    }
  };
  // fp8: convert the prefetched codes and write them (and the scales) into buffer `buf`
  auto finish_stage = [&](char* buf) {
    if constexpr (KV == KV_FP8) {
#pragma unroll
      for (int r = 0; r < C::FP8_PER_THREAD; ++r) {
        const int i = threadIdx.x + r * C::THREADS;
        if (i < C::FP8_ITEMS) {
          const int t = i / (NSETS * DL / 16);
          const int k16 = i - t * (NSETS * DL / 16);
          char* rowp = buf + C::LAT_OFF;
          *reinterpret_cast<uint4*>(rowp + lds_off(t, C::LW, k16 * 32)) = e4m3x8_to_bf16x8(pre[r].x, pre[r].y);
          *reinterpret_cast<uint4*>(rowp + lds_off(t, C::LW, k16 * 32 + 16)) = e4m3x8_to_bf16x8(pre[r].z, pre[r].w);
        }
      }
      if (threadIdx.x < kTile) reinterpret_cast<float*>(buf + C::SC_OFF)[threadIdx.x] = pre_sc;
    }
    (void)buf;
  };

  // ---- this lane's query fragments (B operand of S^T = K . Q^T)
  Frag qf[C::KS];
  {
    const size_t qrow = a.mlra ? ((size_t)b * a.heads + head) * G + gs : (size_t)b * a.heads + head;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = ks * M::KSTEP + h * M::EPL;
      const CT* src;
      if (KIND != KIND_LATENT || ks * M::KSTEP < DL)
        src = static_cast<const CT*>(a.q_lat) + qrow * DL + d0;
      else
        src = static_cast<const CT*>(a.q_rope) + qrow * DR + (d0 - DL);
      if constexpr (M::EPL == 8) {
        uint4 v = valid ? *reinterpret_cast<const uint4*>(src) : make_uint4(0u, 0u, 0u, 0u);
        qf[ks] = __builtin_bit_cast(Frag, v);
      } else {
        qf[ks] = valid ? *src : 0.f;
      }
    }
  }

  floatx16 acc[C::CB];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb) acc[cb] = floatx16{};
  float m_run = -INFINITY;  // running (possibly stale, see kRescaleSlack) max of this head's log2 scores
  float l_run = 0.f;        // running sum of 2^(score - m_run)

  const int tr = M::row_token(col);  // stage token this lane's S row stands for

  // Per-lane LDS byte offsets (bf16 path).  S operand: 16-byte chunk (2ks + h) of row tr; the
  // low three chunk bits depend on ks only through ks & 3.
  int klat[4] = {0, 0, 0, 0}, krope[4] = {0, 0, 0, 0};
  int vtr[2][2] = {{0, 0}, {0, 0}};
  if constexpr (M::EPL == 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      klat[q] = lds_off(tr, C::LW, (2 * q + h) * 16);
      if constexpr (DR > 0) krope[q] = lds_off(tr, C::RW, (2 * q + h) * 16);
    }
    // V^T operand via transposed reads.  Lane group g = lane/16 serves columns 16*(g%2) + (lane%16)
    // of a 32-column block and tokens 8*(g/2) + 4*rb + [0, 4) of a 16-token k-step; its source
    // lane L = lane%16 loads columns 4*(L%4) .. +3 of token 8*(g/2) + 4*rb + L/4.
    const int g16 = lane >> 4;
    const int L16 = lane & 15;
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int tt = 8 * (g16 >> 1) + 4 * rb + (L16 >> 2);
        vtr[c1][rb] = lds_off(tt, C::VRB, (4 * c1 + 2 * (g16 & 1)) * 16 + (L16 & 3) * 8);
      }
  }

  // ---- prologue: stage 0
  const int nstage = (t_end - t_begin + kTile - 1) / kTile;
  issue_stage(t_begin, smem);
  finish_stage(smem);

  for (int n = 0; n < nstage; ++n) {
    const int stage0 = t_begin + n * kTile;
    char* cur = smem + (n & 1) * C::BUF_AL;
    char* nxt = smem + ((n + 1) & 1) * C::BUF_AL;
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of stage n have landed (all counters zero)
    __syncthreads();                 // ... and everyone's; everyone is done with stage n-1's buffer
    if (n + 1 < nstage) issue_stage(stage0 + kTile, nxt);

    // ---- S^T for this wave's set: rows = stage tokens (permuted), columns = 32 heads
    floatx16 sl = floatx16{};
    floatx16 sr = floatx16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      Frag af;
      const bool lat = KIND != KIND_LATENT || ks * M::KSTEP < DL;
      if constexpr (M::EPL == 8) {
        const int c0 = lat ? (s * DL) / 8 + 2 * ks : 2 * (ks - DL / 16);   // even chunk, lane bit excluded
        const char* p = lat ? cur + C::LAT_OFF + klat[(c0 >> 1) & 3] + 16 * (c0 & ~7)
                            : cur + C::ROPE_OFF + krope[(c0 >> 1) & 3] + 16 * (c0 & ~7);
        af = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(p));
      } else {
        const int d0 = ks * M::KSTEP + h;
        const char* p = lat ? cur + C::LAT_OFF + lds_off(tr, C::LW, (s * DL + d0) * ES)
                            : cur + C::ROPE_OFF + lds_off(tr, C::RW > 0 ? C::RW : 32, (d0 - DL) * ES);
        af = *reinterpret_cast<const float*>(p);
      }
      if (KV == KV_FP8 && !lat)
        sr = M::mma(af, qf[ks], sr);
      else
        sl = M::mma(af, qf[ks], sl);
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the operand reads in flight
    }

    // ---- online softmax (log2 domain) over this lane's 16 tokens and its partner's 16
    float sv[16];
    float tok_scale[16];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tt = M::token_of(i, h);
      float v;
      if constexpr (KV == KV_FP8) {
        tok_scale[i] = reinterpret_cast<const float*>(cur + C::SC_OFF)[tt];
        v = (tok_scale[i] * sl[i] + sr[i]) * a.scale_log2;
      } else {
        tok_scale[i] = 1.f;
        v = sl[i] * a.scale_log2;
      }
      v = (stage0 + tt < t_end) ? v : -INFINITY;
      sv[i] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // raise the running max only when this stage's max exceeds it by more than the slack
    const bool raise = mt > m_run + kRescaleSlack;
    const float m_new = raise ? mt : m_run;
    const float alpha = raise ? exp2f(m_run - m_new) : 1.f;   // 0 on the first stage
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = exp2f(sv[i] - m_use);
      psum += sv[i];
    }
    psum += __shfl_xor(psum, 32);
    if (n > 0 && __any(alpha != 1.f)) {   // rare; O is still zero on the first stage
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- P^T fragments (B operand of the PV MFMA); fp8 folds the token scale in here
    Frag pf[M::PSTEPS];
    if constexpr (M::EPL == 8) {
#pragma unroll
      for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
        bf16x8_t f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (__bf16)(sv[8 * p2 + j] * tok_scale[8 * p2 + j]);
        pf[p2] = f;
      }
    } else {
#pragma unroll
      for (int p2 = 0; p2 < M::PSTEPS; ++p2) pf[p2] = sv[p2] * tok_scale[p2];
    }

    // ---- O^T += V^T . P^T
    const char* vsrc = cur + C::V_REG;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
      for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
        Frag af;
        if constexpr (M::EPL == 8) {
          const int cstat = 16 * p2 * C::VRB + 16 * ((s * DL) / 8 + ((4 * cb) & ~7));
          const bf16x4_t lo = lds_read_tr(vsrc + vtr[cb & 1][0] + cstat);
          const bf16x4_t hi = lds_read_tr(vsrc + vtr[cb & 1][1] + cstat);
          af = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          const int tt = 2 * p2 + h;
          af = *reinterpret_cast<const float*>(vsrc + lds_off(tt, C::VRB, (s * DL + cb * 32 + col) * ES));
        }
        acc[cb] = M::mma(af, pf[p2], acc[cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if (n + 1 < nstage) finish_stage(nxt);
  }

  // ---- epilogue: normalise; final output for unsplit sequences, partials otherwise
  const float inv_l = 1.f / l_run;
  const float lse_v = (m_run + log2f(l_run)) * kLn2;
  if (!valid) return;
  if (nsplit == 1) {
    const size_t orow = (size_t)b * a.rows + row;
    if (h == 0) a.lse[orow] = lse_v;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = cb * 32 + 8 * g4 + 4 * h;
        const float o0 = acc[cb][4 * g4 + 0] * inv_l, o1 = acc[cb][4 * g4 + 1] * inv_l;
        const float o2 = acc[cb][4 * g4 + 2] * inv_l, o3 = acc[cb][4 * g4 + 3] * inv_l;
        if (a.out_bf16) {
          __bf16* dst = static_cast<__bf16*>(a.out) + orow * DL + c;
          bf16x4_t v = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
          *reinterpret_cast<bf16x4_t*>(dst) = v;
        } else {
          float* dst = static_cast<float*>(a.out) + orow * DL + c;
          *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  } else {
    const size_t prow = (size_t)unit * a.rows + row;
    if (h == 0) a.part_lse[prow] = lse_v;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = cb * 32 + 8 * g4 + 4 * h;
        float* dst = a.part_out + prow * DL + c;
        *reinterpret_cast<float4*>(dst) =
            make_float4(acc[cb][4 * g4] * inv_l, acc[cb][4 * g4 + 1] * inv_l, acc[cb][4 * g4 + 2] * inv_l,
                        acc[cb][4 * g4 + 3] * inv_l);
      }
    }
  }
}

template <int KV, int DL, int DR, int KIND, int NSETS, int WAVES>
int run(const DecodeArgs& a, void* stream) {
  using C = Cfg<KV, DL, DR, KIND, NSETS, WAVES>;
  if (a.nsets != NSETS || a.nsets * a.hblocks != WAVES) return -1;
  auto fn = decode_kernel<KV, DL, DR, KIND, NSETS, WAVES>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     C::LDS_BYTES);
  if (e != hipSuccess) return (int)e;
  const int units8 = (a.max_units + 7) / 8 * 8;
  const dim3 grid(units8 * a.wg_per_unit);
  hipLaunchKernelGGL(fn, grid, dim3(C::THREADS), C::LDS_BYTES, static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// the instantiated shapes: (kv dtype, d_latent, d_rope, kind, sets per work group, waves)
// ------------------------------------------------------------------------------------------
#define LD_SHAPES(X)                                                                                   \
  /* MLA: 128 / 64 / 32 heads */                                                                       \
  X(KV_BF16, 512, 64, KIND_LATENT, 1, 4) X(KV_BF16, 512, 64, KIND_LATENT, 1, 2)                         \
  X(KV_BF16, 512, 64, KIND_LATENT, 1, 1) X(KV_FP8, 512, 64, KIND_LATENT, 1, 4)                          \
  X(KV_FP8, 512, 64, KIND_LATENT, 1, 2) X(KV_FP8, 512, 64, KIND_LATENT, 1, 1)                           \
  /* GLA-2 (2 groups x 64 heads), GLA-4, one group */                                                  \
  X(KV_BF16, 256, 64, KIND_LATENT, 2, 4) X(KV_BF16, 256, 64, KIND_LATENT, 4, 4)                         \
  X(KV_BF16, 256, 64, KIND_LATENT, 1, 4) X(KV_FP8, 256, 64, KIND_LATENT, 2, 4)                          \
  X(KV_FP8, 256, 64, KIND_LATENT, 4, 4) X(KV_FP8, 256, 64, KIND_LATENT, 1, 4)                           \
  /* MLRA-4 (two branches of 128 heads per work group), one branch */                                  \
  X(KV_BF16, 128, 64, KIND_LATENT, 2, 8) X(KV_BF16, 128, 64, KIND_LATENT, 1, 4)                         \
  X(KV_FP8, 128, 64, KIND_LATENT, 2, 8) X(KV_FP8, 128, 64, KIND_LATENT, 1, 4)                           \
  /* small latent shapes: up to 32 heads per set */                                                    \
  X(KV_F32, 64, 16, KIND_LATENT, 1, 1) X(KV_F32, 64, 16, KIND_LATENT, 2, 2)                             \
  X(KV_F32, 64, 16, KIND_LATENT, 4, 4) X(KV_BF16, 64, 16, KIND_LATENT, 1, 1)                            \
  X(KV_BF16, 64, 16, KIND_LATENT, 2, 2) X(KV_BF16, 64, 16, KIND_LATENT, 4, 4)                           \
  X(KV_FP8, 64, 16, KIND_LATENT, 1, 1) X(KV_FP8, 64, 16, KIND_LATENT, 2, 2)                             \
  X(KV_FP8, 64, 16, KIND_LATENT, 4, 4)                                                                  \
  /* GQA: 4 kv heads (K and V) per work group; GTA: 8; MQA: one kv head */                     \
  X(KV_BF16, 128, 0, KIND_SHARED, 4, 4) X(KV_BF16, 128, 0, KIND_SHARED, 2, 2)                           \
  X(KV_BF16, 128, 0, KIND_SHARED, 1, 2) X(KV_BF16, 128, 0, KIND_SHARED, 1, 1)                           \
  X(KV_BF16, 128, 0, KIND_TIED, 8, 8) X(KV_BF16, 128, 0, KIND_TIED, 4, 4)                               \
  X(KV_BF16, 128, 0, KIND_TIED, 1, 2) X(KV_BF16, 128, 0, KIND_TIED, 1, 1)                               \
  X(KV_F32, 64, 0, KIND_SHARED, 4, 4) X(KV_F32, 64, 0, KIND_SHARED, 1, 1)                               \
  X(KV_F32, 64, 0, KIND_TIED, 4, 4) X(KV_F32, 64, 0, KIND_TIED, 1, 1)

int kv_code(const ld_problem& p) { return p.kv_dtype == LD_FP8_E4M3 ? KV_FP8 : p.kv_dtype == LD_BF16 ? KV_BF16 : KV_F32; }
int kind_code(const ld_problem& p) {
  if (p.variant <= LD_VARIANT_MLRA) return KIND_LATENT;
  return p.variant == LD_VARIANT_GTA ? KIND_TIED : KIND_SHARED;
}

}  // namespace

bool decode_instantiated(const ld_problem& p, int nsets, int waves) {
  const int kv = kv_code(p), kind = kind_code(p), dl = p.d_latent, dr = p.d_rope;
#define LD_MATCH(KV_, DL_, DR_, KIND_, NS_, W_) \
  if (kv == KV_ && dl == DL_ && dr == DR_ && kind == KIND_ && nsets == NS_ && waves == W_) return true;
  LD_SHAPES(LD_MATCH)
#undef LD_MATCH
  return false;
}

int launch_decode(const ld_problem& p, const DecodeArgs& a, void* stream) {
  const int kv = kv_code(p), kind = kind_code(p), dl = p.d_latent, dr = p.d_rope;
  const int nsets = a.nsets, waves = a.nsets * a.hblocks;
#define LD_RUN(KV_, DL_, DR_, KIND_, NS_, W_) \
  if (kv == KV_ && dl == DL_ && dr == DR_ && kind == KIND_ && nsets == NS_ && waves == W_) \
    return run<KV_, DL_, DR_, KIND_, NS_, W_>(a, stream);
  LD_SHAPES(LD_RUN)
#undef LD_RUN
  return -1;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

}  // namespace ld
