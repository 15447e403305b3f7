// Decode-attention kernels for gfx950 (CDNA4): one query token per sequence against a paged,
// shrunk KV cache.  See include/latent_decode.h for the operation and its sources.
//
// Work decomposition.  A work unit is (sequence b, token chunk [t_begin, t_end)) from the
// split-KV planner.  A "set" is a group of query heads that score against the same cached
// rows: all H heads for MLA, one latent group for GLA, one branch for MLRA, one kv head for
// GQA/GTA, all heads for MQA.  A work group handles `nsets` sets of one unit; each of its
// waves owns one set and 32 of that set's heads.  Per 32-token tile the work group stages
// the rows it needs in LDS once, and every wave reads them from there:
//
//   S^T[token, head] = K_tile . Q^T          (v_mfma_f32_32x32x16_bf16, Q stays in VGPRs)
//   online softmax over the token axis      (each lane owns one head: 16 scores + the
//                                            other 16 in the lane 32 apart)
//   O^T[col, head]  += V_tile^T . P^T         (the same MFMA; P never leaves registers)
//
// The rows of the S MFMA are a fixed permutation of the tile's tokens, chosen so that the
// score layout the MFMA writes is exactly the P^T operand layout the PV MFMA reads.
#include <hip/hip_runtime.h>

#include "ld_internal.h"

namespace ld {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i%4 of the
// 8-byte loads of lanes 4k + i/4, k = 0..3 (so four lanes that load four consecutive
// elements of four rows hand every lane one column of those rows).
__device__ __forceinline__ bf16x4_t lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

enum KvT : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

constexpr float kLn2 = 0.69314718055994530942f;

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
  static constexpr int PSTEPS = 2;  // k-steps over a 32-token tile in P.V
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

// 16-byte chunks of a staged row are XOR-swizzled by the token's low bits so that the 32
// rows one MFMA operand read touches fall into different LDS banks.
template <int NCHUNK>
struct Swz {
  static constexpr int M = (NCHUNK % 8 == 0) ? 7 : (NCHUNK % 4 == 0) ? 3 : (NCHUNK % 2 == 0) ? 1 : 0;
};

__device__ __forceinline__ int lds_byte(int t, int row_bytes, int byte_in_row, int swm) {
  const int c = byte_in_row >> 4;
  return t * row_bytes + (((c ^ (t & swm)) << 4) | (byte_in_row & 15));
}

// fp8 E4M3 (OCP) -> bf16, exact: 8 codes in, 8 bf16 out.  v_cvt_scalef32_pk_bf16_fp8 with
// scale 1 converts two codes straight to two bf16 (every E4M3 value is a bf16 value).  (Going
// through v_cvt_pk_f32_fp8 and repacking the f32 halves was mis-combined by the compiler into
// a copy of one half, so the direct conversion is used.)
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 codes) {
  const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, 1.0f, false);
  const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, 1.0f, true);
  const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, 1.0f, false);
  const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(unsigned, a0), __builtin_bit_cast(unsigned, a1),
                    __builtin_bit_cast(unsigned, b0), __builtin_bit_cast(unsigned, b1));
}

template <int KV, int DL, int DR, int KIND>
struct Cfg {
  using M = Mma<KV>;
  using CT = typename M::CT;
  static constexpr int DK = DL + DR;            // score dims per set
  static constexpr int KS = DK / M::KSTEP;      // k-steps of S
  static constexpr int CB = DL / 32;            // 32-column blocks of O
  static constexpr int ES = sizeof(CT);
  static_assert(DK % M::KSTEP == 0 && DL % 32 == 0, "unsupported dims");
};

// ------------------------------------------------------------------------------------------
// stage one 32-token tile of the work group's rows into LDS (zeros past t_end)
// ------------------------------------------------------------------------------------------
template <class C, int KV, int DL, int DR, int KIND>
__device__ __forceinline__ void stage_tile(const DecodeArgs& a, char* lds_k, char* lds_v, float* lds_s,
                                           const int32_t* bt_row, int tile0, int t_end, int set0, int nsets,
                                           int kw_bytes, int vw_bytes, int swm_k, int swm_v) {
  using CT = typename C::CT;
  const int G = a.groups;
  const int nck = kw_bytes >> 4;
  const int total = kTile * nck;
  const int lat_bytes = nsets * DL * (int)sizeof(CT);
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int t = idx / nck;
    const int c = idx - t * nck;
    const int tok = tile0 + t;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (tok < t_end) {
      const int page = clampi(bt_row[tok / a.page_size], 0, a.num_pages - 1);
      const size_t rowi = (size_t)page * a.page_size + (tok % a.page_size);
      const int byte0 = c << 4;
      if (byte0 < lat_bytes) {
        const int e0 = byte0 / (int)sizeof(CT);
        const int s = e0 / DL;
        const int w = e0 - s * DL;
        const int gs = set0 + s;
        if constexpr (KV == KV_FP8) {
          const uint8_t* src = static_cast<const uint8_t*>(a.k) + rowi * (size_t)(G * DL) + (size_t)gs * DL + w;
          val = e4m3x8_to_bf16x8(*reinterpret_cast<const uint2*>(src));
        } else if constexpr (KIND == KIND_LATENT) {
          const CT* src = static_cast<const CT*>(a.k) + rowi * (size_t)(G * DL + DR) + (size_t)gs * DL + w;
          val = *reinterpret_cast<const uint4*>(src);
        } else {
          const CT* src = static_cast<const CT*>(a.k) + (rowi * G + gs) * (size_t)DL + w;
          val = *reinterpret_cast<const uint4*>(src);
        }
      } else {
        if constexpr (DR > 0) {
          const int r = (byte0 - lat_bytes) / (int)sizeof(CT);
          if constexpr (KV == KV_FP8) {
            const __bf16* src = static_cast<const __bf16*>(a.rope) + rowi * (size_t)DR + r;
            val = *reinterpret_cast<const uint4*>(src);
          } else {
            const CT* src = static_cast<const CT*>(a.k) + rowi * (size_t)(G * DL + DR) + (size_t)G * DL + r;
            val = *reinterpret_cast<const uint4*>(src);
          }
        }
      }
    }
    *reinterpret_cast<uint4*>(lds_k + lds_byte(t, kw_bytes, c << 4, swm_k)) = val;
  }
  if constexpr (KIND == KIND_SHARED) {
    const int nv = vw_bytes >> 4;
    const int totv = kTile * nv;
    for (int idx = threadIdx.x; idx < totv; idx += blockDim.x) {
      const int t = idx / nv;
      const int c = idx - t * nv;
      const int tok = tile0 + t;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (tok < t_end) {
        const int page = clampi(bt_row[tok / a.page_size], 0, a.num_pages - 1);
        const size_t rowi = (size_t)page * a.page_size + (tok % a.page_size);
        const int e0 = (c << 4) / (int)sizeof(CT);
        const int s = e0 / DL;
        const int w = e0 - s * DL;
        const CT* src = static_cast<const CT*>(a.v) + (rowi * G + (set0 + s)) * (size_t)DL + w;
        val = *reinterpret_cast<const uint4*>(src);
      }
      *reinterpret_cast<uint4*>(lds_v + lds_byte(t, vw_bytes, c << 4, swm_v)) = val;
    }
  }
  if constexpr (KV == KV_FP8) {
    for (int t = threadIdx.x; t < kTile; t += blockDim.x) {
      const int tok = tile0 + t;
      float sc = 0.f;
      if (tok < t_end) {
        const int page = clampi(bt_row[tok / a.page_size], 0, a.num_pages - 1);
        sc = a.kscale[(size_t)page * a.page_size + (tok % a.page_size)];
      }
      lds_s[t] = sc;
    }
  }
}

// ------------------------------------------------------------------------------------------
// the decode kernel
// ------------------------------------------------------------------------------------------
template <int KV, int DL, int DR, int KIND, int NSETS, int MAXT>
__global__ __launch_bounds__(MAXT) void decode_kernel(DecodeArgs a) {
  using C = Cfg<KV, DL, DR, KIND>;
  using M = typename C::M;
  using CT = typename C::CT;
  using Frag = typename M::Frag;
  constexpr int ES = C::ES;
  constexpr int KW = (NSETS * DL + DR) * ES;                    // staged K row bytes
  constexpr int VW = (KIND == KIND_SHARED) ? NSETS * DL * ES : 0;  // staged V row bytes
  constexpr int SWM_K = Swz<KW / 16>::M;
  constexpr int SWM_V = Swz<(VW > 0 ? VW : 16) / 16>::M;
  constexpr int VROW = (KIND == KIND_SHARED) ? VW : KW;
  constexpr int SWM_VR = (KIND == KIND_SHARED) ? SWM_V : SWM_K;
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
  char* lds_k = smem;
  char* lds_v = smem + kTile * KW;
  float* lds_s = reinterpret_cast<float*>(smem + kTile * (KW + VW));

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int s = __builtin_amdgcn_readfirstlane(wave / a.hblocks);
  const int hb = __builtin_amdgcn_readfirstlane(wave - s * a.hblocks);
  const int gs = set0 + s;
  const int head_in_set = hb * 32 + col;
  const bool valid = head_in_set < a.heads_per_set;
  const int head = (a.mlra ? 0 : gs * a.heads_per_set) + (valid ? head_in_set : 0);
  const int row = a.mlra ? head * G + gs : head;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;

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
  float m_run = -INFINITY;  // running max of the log2-scaled scores of this lane's head
  float l_run = 0.f;        // running sum of 2^(score - m_run)

  const int tr = M::row_token(col);  // tile token this lane's S row stands for

  // Per-lane LDS byte offsets (bf16 path).  S operand: the 16-byte chunk (2ks + h) of row tr,
  // swizzled; its low three chunk bits depend on ks only through ks & 3.
  int kbase[4];
  int vbase[2][2];
  if constexpr (M::EPL == 8) {
    const int key = tr & SWM_K;
#pragma unroll
    for (int q = 0; q < 4; ++q) kbase[q] = tr * KW + 16 * (((2 * q + h) & SWM_K) ^ key) + 16 * ((2 * q + h) & ~SWM_K);
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
        const int chunk = 4 * c1 + 2 * (g16 & 1) + ((L16 & 3) >> 1);
        vbase[c1][rb] = tt * VROW + 16 * (((chunk & SWM_VR) ^ (tt & SWM_VR)) + (chunk & ~SWM_VR)) + 8 * (L16 & 1);
      }
  }

  for (int tile0 = t_begin; tile0 < t_end; tile0 += kTile) {
    __syncthreads();
    stage_tile<C, KV, DL, DR, KIND>(a, lds_k, lds_v, lds_s, bt_row, tile0, t_end, set0, NSETS, KW, VW, SWM_K, SWM_V);
    __syncthreads();

    // ---- S^T for this wave's set: rows = tile tokens (permuted), columns = 32 heads
    floatx16 sl = floatx16{};
    floatx16 sr = floatx16{};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      Frag af;
      if constexpr (M::EPL == 8) {
        // chunk index of this k-step's first half, without the lane bits
        const int c0 = (KIND != KIND_LATENT || ks * 16 < DL) ? (s * DL) / 8 + 2 * ks : (NSETS * DL) / 8 + 2 * (ks - DL / 16);
        const char* p = lds_k + kbase[(c0 >> 1) & 3] + 16 * (c0 & ~7);
        af = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(p));
      } else {
        const int d0 = ks * M::KSTEP + h * M::EPL;
        const int e = (KIND != KIND_LATENT || d0 < DL) ? s * DL + d0 : NSETS * DL + (d0 - DL);
        af = *reinterpret_cast<const float*>(lds_k + lds_byte(tr, KW, e * ES, SWM_K));
      }
      if (KV == KV_FP8 && ks * M::KSTEP >= DL)
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
        tok_scale[i] = lds_s[tt];
        v = (tok_scale[i] * sl[i] + sr[i]) * a.scale_log2;
      } else {
        tok_scale[i] = 1.f;
        v = sl[i] * a.scale_log2;
      }
      v = (tile0 + tt < t_end) ? v : -INFINITY;
      sv[i] = v;
      mt = fmaxf(mt, v);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = exp2f(sv[i] - m_use);
      ps += sv[i];
    }
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) acc[cb] *= alpha;
    }

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
    const char* vsrc = (KIND == KIND_SHARED) ? lds_v : lds_k;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
#pragma unroll
      for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
        Frag af;
        if constexpr (M::EPL == 8) {
          const int cstat = 16 * p2 * VROW + 16 * ((s * DL) / 8 + ((4 * cb) & ~7));
          const bf16x4_t lo = lds_read_tr(vsrc + vbase[cb & 1][0] + cstat);
          const bf16x4_t hi = lds_read_tr(vsrc + vbase[cb & 1][1] + cstat);
          af = bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          const int tt = 2 * p2 + h;
          af = *reinterpret_cast<const float*>(vsrc + lds_byte(tt, VROW, (s * DL + cb * 32 + col) * ES, SWM_VR));
        }
        acc[cb] = M::mma(af, pf[p2], acc[cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
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
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
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

template <int KV, int DL, int DR, int KIND, int NSETS, int MAXT>
int run(const DecodeArgs& a, void* stream) {
  using C = Cfg<KV, DL, DR, KIND>;
  const int threads = NSETS * a.hblocks * kWaveSize;
  if (a.nsets != NSETS || threads > MAXT || threads <= 0) return -1;
  constexpr int kw = (NSETS * DL + DR) * C::ES;
  constexpr int vw = (KIND == KIND_SHARED) ? NSETS * DL * C::ES : 0;
  const size_t lds = (size_t)kTile * (kw + vw) + (KV == KV_FP8 ? kTile * sizeof(float) : 0);
  if (lds > 160 * 1024) return -1;
  auto fn = decode_kernel<KV, DL, DR, KIND, NSETS, MAXT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return (int)e;
  const int units8 = (a.max_units + 7) / 8 * 8;
  const dim3 grid(units8 * a.wg_per_unit);
  hipLaunchKernelGGL(fn, grid, dim3(threads), lds, static_cast<hipStream_t>(stream), a);
  return (int)hipGetLastError();
}

}  // namespace

// The instantiated shapes (see kernel_shape in api.cpp, which picks nsets and the work-group size):
//   latent bf16/fp8: (d_latent, d_rope) = (512, 64) nsets 1; (256, 64) nsets 1, 2; (128, 64) nsets 1, 2;
//                    (64, 16) nsets 1, 2, 4
//   latent f32:      (64, 16) nsets 1, 2, 4
//   shared bf16/f32: head dim 128 or 64, nsets 1, 2, 4, 8 (f32 with head dim 128: nsets <= 4)
bool decode_supported(const ld_problem& p) {
  const bool latent = p.variant <= LD_VARIANT_MLRA;
  const int dl = p.d_latent, dr = p.d_rope;
  if (latent) {
    if (p.kv_dtype == LD_F32) return dl == 64 && dr == 16;
    return (dl == 512 && dr == 64) || (dl == 256 && dr == 64) || (dl == 128 && dr == 64) || (dl == 64 && dr == 16);
  }
  return dr == 0 && (dl == 128 || dl == 64) && p.kv_dtype != LD_FP8_E4M3;
}

int kernel_max_threads(const ld_problem& p) {
  const bool latent = p.variant <= LD_VARIANT_MLRA;
  if (latent && (p.d_latent == 512 || p.d_latent == 256)) return 256;
  if (!latent && p.kv_dtype == LD_F32 && p.d_latent == 128) return 256;
  return 512;
}

int kernel_max_sets(const ld_problem& p) {
  const bool latent = p.variant <= LD_VARIANT_MLRA;
  if (latent) {
    if (p.d_latent == 512) return 1;
    if (p.d_latent == 64) return 4;
    return 2;
  }
  return (p.kv_dtype == LD_F32 && p.d_latent == 128) ? 4 : 8;
}

template <int KV, int DL, int DR, int MAXT>
static int latent_sets(const DecodeArgs& a, void* stream) {
  switch (a.nsets) {
    case 1: return run<KV, DL, DR, KIND_LATENT, 1, MAXT>(a, stream);
    case 2: if constexpr (DL <= 256) return run<KV, DL, DR, KIND_LATENT, 2, MAXT>(a, stream); else return -1;
    case 4: if constexpr (DL <= 64) return run<KV, DL, DR, KIND_LATENT, 4, MAXT>(a, stream); else return -1;
    default: return -1;
  }
}

template <int KV>
static int dispatch_latent(const ld_problem& p, const DecodeArgs& a, void* stream) {
  const int dl = p.d_latent, dr = p.d_rope;
  if constexpr (KV == KV_F32) {
    if (dl == 64 && dr == 16) return latent_sets<KV, 64, 16, 512>(a, stream);
    return -1;
  } else {
    if (dl == 512 && dr == 64) return latent_sets<KV, 512, 64, 256>(a, stream);
    if (dl == 256 && dr == 64) return latent_sets<KV, 256, 64, 256>(a, stream);
    if (dl == 128 && dr == 64) return latent_sets<KV, 128, 64, 512>(a, stream);
    if (dl == 64 && dr == 16) return latent_sets<KV, 64, 16, 512>(a, stream);
    return -1;
  }
}

template <int KV, int KIND, int DL, int MAXT>
static int shared_sets(const DecodeArgs& a, void* stream) {
  switch (a.nsets) {
    case 1: return run<KV, DL, 0, KIND, 1, MAXT>(a, stream);
    case 2: return run<KV, DL, 0, KIND, 2, MAXT>(a, stream);
    case 4: return run<KV, DL, 0, KIND, 4, MAXT>(a, stream);
    case 8: if constexpr (!(KV == KV_F32 && DL == 128)) return run<KV, DL, 0, KIND, 8, MAXT>(a, stream); else return -1;
    default: return -1;
  }
}

template <int KV, int KIND>
static int dispatch_shared(const ld_problem& p, const DecodeArgs& a, void* stream) {
  if (p.d_latent == 128) {
    if constexpr (KV == KV_F32) return shared_sets<KV, KIND, 128, 256>(a, stream);
    else return shared_sets<KV, KIND, 128, 512>(a, stream);
  }
  if (p.d_latent == 64) return shared_sets<KV, KIND, 64, 512>(a, stream);
  return -1;
}

int launch_decode(const ld_problem& p, const DecodeArgs& a, void* stream) {
  const bool latent = p.variant <= LD_VARIANT_MLRA;
  if (latent) {
    if (p.kv_dtype == LD_FP8_E4M3) return dispatch_latent<KV_FP8>(p, a, stream);
    if (p.kv_dtype == LD_BF16) return dispatch_latent<KV_BF16>(p, a, stream);
    return dispatch_latent<KV_F32>(p, a, stream);
  }
  if (p.variant == LD_VARIANT_GTA) {
    if (p.kv_dtype == LD_BF16) return dispatch_shared<KV_BF16, KIND_TIED>(p, a, stream);
    return dispatch_shared<KV_F32, KIND_TIED>(p, a, stream);
  }
  if (p.kv_dtype == LD_BF16) return dispatch_shared<KV_BF16, KIND_SHARED>(p, a, stream);
  return dispatch_shared<KV_F32, KIND_SHARED>(p, a, stream);
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

}  // namespace ld
