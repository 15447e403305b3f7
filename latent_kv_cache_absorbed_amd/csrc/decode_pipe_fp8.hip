// Decode kernel for latent caches stored as fp8 E4M3 codes with a per-token scale: GLA with
// 256-dim latent groups and 64 heads per group ("Mamba核心作者新作…" (jsbsmhs.com), the GLA section and
// the FP8 serving test), every group of the cache in one work group (GLA-2: two groups, 128 heads;
// one group, 64 heads: a tensor-parallel share), gfx950.  See include/latent_decode.h for the
// operation and its sources.
//
// The stage is copied as stored: 32 rows of codes (G x 256 bytes), 32 rope keys (bf16) and 32
// scales, 20.6 KB for GLA-2 against 36.9 KB for a bf16 stage of the same rows, into six stage
// buffers.  Codes become bf16 when an MFMA operand is read (v_cvt_scalef32_pk_bf16_fp8 with scale
// 1 makes each pair of codes two bf16, exactly):
//   score operand (8 dims of one token per lane): one 16-byte read gives two k-steps' operands
//   value operand (8 tokens of one column per lane): ds_read_b64_tr_b8, which hands lane i of each
//     16 lanes byte i of the 8 rows that lane pairs (2e, 2e+1) point at
// The conversions are half-rate VALU work, as much as the MFMAs they feed, so the work group runs
// two waves per SIMD with split roles, and one wave's conversions overlap the other's MFMAs:
//   producer wave (per 32-head block of a group): Q in 80 VGPRs; the score MFMAs of stage n+1 with
//     the softmax of stage n between them; hands P of stage n (bf16, 2 KB) to its consumer in LDS
//   consumer wave (same heads): O (32 heads x 256 f32) in 128 VGPRs; P.V of stage n-1 with P from
//     LDS; issues the stage copies
// One work-group barrier per stage orders the copies, P and the buffer reuse.  The softmax keeps
// the fixed per-unit reference of decode_pipe.hip (a second pass with the exact max when a score
// runs more than 2^kRefSlack above it).  The per-token scale multiplies the latent part of the
// score and P (the value rows), as decode.hip does for fp8: s = scale * (q_lat . e) + q_rope . k_r;
// P.V takes bf16(p * scale); the row sum takes p.
#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "plan_common.h"
#include "ld_internal.h"

namespace ld {
namespace {

typedef int int2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) int2v lds_int2v;

template <int G>
struct P8Cfg {
  static constexpr int DL = 256, DR = 64;
  static constexpr int HBG = 2;                         // 32-head blocks per group (64 heads)
  static constexpr int ROLE = G * HBG;                  // waves per role
  static constexpr int THREADS = 2 * ROLE * kWaveSize;  // producers, then consumers
  static constexpr int CROW = G * DL;                   // bytes of a token's codes (LDS and memory)
  static constexpr int CODES = kTile * CROW;
  static constexpr int RW = DR * 2;                     // rope row bytes
  static constexpr int MR = swz_mask(RW);
  static constexpr int ROPE_OFF = CODES;
  static constexpr int SC_OFF = ROPE_OFF + kTile * RW;
  static constexpr int BUF = SC_OFF + kTile * 4;
  static constexpr int NBUF = G == 2 ? 6 : 5;  // one GLA group: two work groups per CU
  // stage m is read by the producers in iterations m-1 (scores) and m (softmax: scales) and by the
  // consumers in iteration m+1 (P.V); the copies of stage n+AHEAD are issued in iteration n into
  // the buffer stage n-2 has left
  static constexpr int AHEAD = NBUF - 2;
  // 1 KB copies per wave and stage.  Consumer waves copy the first CODE_C * ROLE code blocks, the
  // first ROPE_C * ROLE rope blocks and the scales (every consumer the same 128 bytes); producer
  // waves copy the rest (CODE_P, ROPE_P per wave).
  static constexpr int CODE_BLOCKS = CODES / 1024;
  static constexpr int ROPE_BLOCKS = kTile * RW / 1024;
  static constexpr int CODE_P = 0;
  static constexpr int ROPE_P = 0;
  static constexpr int CODE_C = CODE_BLOCKS / ROLE - CODE_P;
  static constexpr int ROPE_C = ROPE_BLOCKS / ROLE - ROPE_P;
  static constexpr int CPW_C = CODE_C + ROPE_C + 1;
  static constexpr int CPW_P = CODE_P + ROPE_P;
  static constexpr int KL = DL / 16;                    // latent k-steps of S
  static constexpr int KR = DR / 16;                    // rope k-steps of S
  static constexpr int CB = DL / 32;                    // 32-column blocks of O
  static constexpr int PBLK = 2 * 64 * 16;              // P of one head block and stage (bytes)
  static_assert(CODE_BLOCKS % ROLE == 0 && ROPE_BLOCKS % ROLE == 0, "copy dealing");
  static_assert(CPW_C <= 8 && CPW_P <= 5, "copies per work slot");
  static_assert(KL == 16 && KR == 4 && CB == 8, "the work slots are laid out for 256 + 64 dims");
  static_assert(NBUF * BUF + 2 * ROLE * PBLK + 4 * kUnitPages + 4 * 32 * ROLE + 64 <= 160 * 1024, "LDS budget");
};

// Chunk key of a code row: the 16-byte chunk c of a group's 256 codes sits at c ^ ckey(t) in row t.
// Bits 1..3 of the key take eight distinct values on every 8 aligned rows, so a transposed read of
// 8 rows x two neighbouring chunks (32 lanes) touches 16 distinct chunk slots; on every 16 aligned
// rows the key is a bijection, so 16 lanes reading one chunk of 16 rows do too.
__device__ __forceinline__ int ckey(int t) { return ((t & 7) << 1) | ((t >> 3) & 1); }

__device__ __forceinline__ bf16x8_t cvt8(unsigned lo, unsigned hi) {
  return __builtin_bit_cast(bf16x8_t, e4m3x8_to_bf16x8(lo, hi));
}

template <int G>
__global__ __launch_bounds__(G * 256) void decode_pipe8_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  using C = P8Cfg<G>;
  using M = Mma<KV_BF16>;
  __shared__ __attribute__((aligned(256))) char lds[C::NBUF * C::BUF];
  __shared__ __attribute__((aligned(16))) char lds_p[2 * C::ROLE * C::PBLK];  // [stage parity][head block]
  __shared__ float lds_l[C::ROLE * 32];                                       // row sums for the consumers
  __shared__ int lds_pages[kUnitPages];
  __shared__ int s_unit[5];
  __shared__ int s_again;

  // unit of this work group: the XCD-blocked mapping of decode_kernel
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int y = x >> 3;
  const int sb = y % a.wg_per_unit;
  const int yy = y / a.wg_per_unit;
  int unit, b, t_begin, t_end, nsplit;
  if (a.fused_plan) {
    if (threadIdx.x < 64) fused_plan_unit(a, x, xcd, yy, sb, s_unit);
    __syncthreads();
    if (s_unit[0] < 0) return;
    unit = s_unit[0];
    b = s_unit[1];
    t_begin = s_unit[2];
    t_end = s_unit[3];
    nsplit = s_unit[4];
  } else {
    const int nunits = a.header[0];
    const int per = (nunits + 7) >> 3;
    if (yy >= per) return;
    unit = xcd * per + yy;
    if (unit >= nunits) return;
    const Unit u = a.units[unit];
    b = u.b;
    t_begin = u.t_begin;
    t_end = u.t_end;
    nsplit = a.seqs[4 * b];
  }
  // Work group sb of a unit serves query token qi = sb / wpt (which sees the first L_b - qlen + 1
  // + qi rows) and the cache groups [lset0, lset0 + G) of it: query sets qi * CG + lset0 + ..
  const int wpt = a.wg_per_unit / a.qlen;
  const int qi = sb / wpt;
  const int lset0 = (sb - qi * wpt) * G;
  const int CG = a.cache_groups;
  if (a.qlen > 1) {
    const int Lb = clampi(a.seq_lens[b], 0, a.max_pages * a.page_size);
    t_end = max(t_begin, min(t_end, Lb - a.qlen + 1 + qi));
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool producer = wave < C::ROLE;
  const int rw = producer ? wave : wave - C::ROLE;  // head block index within the role: group, block
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int gl = rw / C::HBG;
  const int hb = rw % C::HBG;
  const int gs = qi * CG + lset0 + gl;
  const int head_in_set = hb * 32 + col;
  const int head = gs * a.heads_per_set + head_in_set;
  const int32_t* __restrict__ bt_row = block_table + (size_t)b * a.max_pages;
  const int page_size = a.page_size;
  const int first_page = t_begin / page_size;
  const int unit_pages = t_end > t_begin ? (t_end - 1) / page_size - first_page + 1 : 0;
  for (int i = threadIdx.x; i < unit_pages && i < kUnitPages; i += C::THREADS)
    lds_pages[i] = clampi(bt_row[first_page + i], 0, a.num_pages - 1);
  __syncthreads();

  const int nstage = (t_end - t_begin + kTile - 1) / kTile;
  auto buf_of = [](int n) { return (unsigned)((n % C::NBUF) * C::BUF); };
  char* const pslot = lds_p + rw * C::PBLK + lane * 16;  // + parity * ROLE * PBLK + p2 * 1024

  const char* kbase = static_cast<const char*>(a.k);
  const int grow = CG * C::DL;  // bytes of a token's codes in the pool (every cache group)
  const char* rbase = static_cast<const char*>(a.rope);
  const char* sbase = reinterpret_cast<const char*>(a.kscale);
  const unsigned lds_u = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  struct StageSrc {
    size_t r0;  // pool row of the stage's first token
    int tlast;  // last row of the unit in this stage (rows past it repeat it)
  };
  auto stage_src = [&](int stage0) -> StageSrc {
    const int pi = stage0 / page_size - first_page;
    const int page = __builtin_amdgcn_readfirstlane(lds_pages[min(pi, kUnitPages - 1)]);
    return StageSrc{(size_t)page * page_size + (stage0 % page_size), t_end - 1 - stage0};
  };
  // Copy j of a wave's share of a stage (see P8Cfg): code blocks, then rope blocks, then (consumers)
  // the 128 bytes of scales (lanes 0..7).  A stage's rows lie in one page.  The source row of a lane
  // is min(token, tlast) (rows past a unit's end repeat its last row), and its LDS chunk is its
  // chunk XORed with the row's key, which splits into a part fixed by the copy (a scalar, passed
  // through an empty asm so that the per-lane offsets are made inside the loop, not held across it)
  // and a part fixed by the lane:
  //  - code rows of 256 bytes (one group): block q holds rows 4 q .. 4 q + 3, 16 lanes a row; lane ln
  //    has row r = ln / 16 and chunk ln % 16, and ckey(4 q + r) = (r << 1) ^ ((q & 1) << 3) ^ (q >> 1 & 1);
  //  - code rows of 512 bytes (two groups): block q holds rows 2 q, 2 q + 1, 32 lanes a row; lane ln
  //    has row r = ln / 32 and chunk ln % 32 (the key touches its low four bits), and
  //    ckey(2 q + r) = (r << 1) ^ ((q & 3) << 2) ^ (q >> 2 & 1);
  //  - rope rows of 128 bytes: block q holds rows 8 q .. 8 q + 7, 8 lanes a row; lane ln has row
  //    r = ln / 8, and swz_key(8 q + r) & 7 is r rotated left by one, bit 0 XORed with q's bit 0.
  constexpr int RPB = 1024 / C::CROW;  // code rows per 1 KB block
  static_assert(RPB == 4 || RPB == 2, "code rows of 256 or 512 bytes");
  const int crow_r = lane / (C::CROW / 16);
  const int crow_c = (lane % (C::CROW / 16)) ^ (crow_r << 1);
  auto copy_block = [&](const StageSrc& src, unsigned buf, int j) __attribute__((always_inline)) {
    const int ncode = producer ? C::CODE_P : C::CODE_C;
    const int nrope = producer ? C::ROPE_P : C::ROPE_C;
    if (j < ncode) {
      const int q = (producer ? C::ROLE * C::CODE_C : 0) + rw + C::ROLE * j;
      int kq = RPB == 4 ? (((q & 1) << 3) | ((q >> 1) & 1)) : (((q & 3) << 2) | ((q >> 2) & 1));
      asm volatile("" : "+s"(kq));
      const int row = min(RPB * q + crow_r, src.tlast);
      const unsigned voff = __umul24((unsigned)row, (unsigned)grow) + (unsigned)((crow_c ^ kq) << 4);
      dma16_asm_at(kbase + src.r0 * (size_t)grow + lset0 * C::DL, voff, lds_u + buf + q * 1024);
    } else if (j < ncode + nrope) {
      const int q = (producer ? C::ROLE * C::ROPE_C : 0) + rw + C::ROLE * (j - ncode);
      static_assert(C::RW == 128, "rope rows of 128 bytes");
      int qb = q & 1;
      asm volatile("" : "+s"(qb));
      const int r = lane >> 3;
      const int row = min(8 * q + r, src.tlast);
      const int c = (lane & 7) ^ (((r << 1) | (r >> 2)) & 7) ^ qb;
      const unsigned voff = (unsigned)((row << 7) + (c << 4));
      dma16_asm_at(rbase + src.r0 * (size_t)C::RW, voff, lds_u + buf + C::ROPE_OFF + q * 1024);
    } else if (lane < kTile * 4 / 16) {
      dma16_asm_at(sbase + src.r0 * 4, (unsigned)(lane * 16), lds_u + buf + C::SC_OFF);
    }
  };
  auto copy_stage = [&](const StageSrc& src, unsigned buf) __attribute__((always_inline)) {
    if (producer) {
#pragma unroll
      for (int j = 0; j < C::CPW_P; ++j) copy_block(src, buf, j);
    } else {
#pragma unroll
      for (int j = 0; j < C::CPW_C; ++j) copy_block(src, buf, j);
    }
  };
  // this wave's copies of stage m have landed, `later` stages' copies being issued after them
  auto wait_copies = [&](int later) __attribute__((always_inline)) {
    static_assert(C::AHEAD - 1 <= 3, "wait cases");
    if (producer) {
      if (later <= 0)
        wait_vmcnt<0>();
      else if (later == 1)
        wait_vmcnt<C::CPW_P>();
      else if (later == 2)
        wait_vmcnt<2 * C::CPW_P>();
      else
        wait_vmcnt<3 * C::CPW_P>();
    } else {
      if (later <= 0)
        wait_vmcnt<0>();
      else if (later == 1)
        wait_vmcnt<C::CPW_C>();
      else if (later == 2)
        wait_vmcnt<2 * C::CPW_C>();
      else
        wait_vmcnt<3 * C::CPW_C>();
    }
  };
  // the prologue of a pass: this wave's share of stages 0 .. AHEAD-1, then stage 0 landed
  auto prologue = [&]() __attribute__((always_inline)) {
    const int pre = min(C::AHEAD, nstage);
    for (int m = 0; m < pre; ++m) copy_stage(stage_src(t_begin + m * kTile), buf_of(m));
    wait_copies(pre - 1);
    lds_barrier();
  };

  if (producer) {
    // ================================ producer: scores and softmax ================================
    bf16x8_t qf[C::KL + C::KR];
    {
      // latent k-steps come in pairs: lanes of half h read code chunk j + 8 h of their token for
      // pair j, whose first eight codes are k-step 2 j and last eight k-step 2 j + 1
      const size_t qrow = (size_t)b * a.heads + head;
      const __bf16* qlp = static_cast<const __bf16*>(a.q_lat) + qrow * C::DL + h * 128;
      const __bf16* qrp = static_cast<const __bf16*>(a.q_rope) + qrow * C::DR + h * 8;
#pragma unroll
      for (int j = 0; j < C::KL / 2; ++j) {
        qf[2 * j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qlp + j * 16));
        qf[2 * j + 1] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qlp + j * 16 + 8));
      }
#pragma unroll
      for (int j = 0; j < C::KR; ++j)
        qf[C::KL + j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrp + j * 16));
    }
    // score operands: code pair j at kc0 ^ 16 j; rope k-step j at ROPE_OFF + (kr0 ^ 32 j)
    const int tr = M::row_token(col);
    const int kc0 = tr * C::CROW + gl * 256 + (((8 * h) ^ ckey(tr)) << 4);
    const int kr0 = lds_off(tr, C::RW, C::MR, h * 16);
    const float c2 = a.scale_log2;
    float l_run = 0.f;       // sum of 2^(score - ref) over the unit
    float ref = 0.f;         // fixed reference of this head (log2 domain)
    float mmax = -INFINITY;  // exact max of this head's scaled scores over the unit (log2 domain)
    bool over = false;       // a stage max exceeded ref + kRefSlack
    bool fixed = false;      // second pass: ref = mmax of the first

    // the 20 score MFMAs of one stage in five groups of four (latent pairs 2g, 2g + 1 for g < 4,
    // the rope k-steps for g = 4), `work(g)` after each group; code reads run two pairs ahead
    auto scores = [&](const char* cur, floatx16& SL, floatx16& SR, auto&& work) __attribute__((always_inline)) {
      int kc = kc0, kr = kr0;
      asm volatile("" : "+v"(kc), "+v"(kr));
      uint4 ring[3];
      ring[0] = *reinterpret_cast<const uint4*>(cur + kc);
      ring[1] = *reinterpret_cast<const uint4*>(cur + (kc ^ 16));
      uint4 rope[C::KR];
#pragma unroll
      for (int g = 0; g < 5; ++g) {
        if (g < 4) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * g + jj;
            if (j + 2 < C::KL / 2) ring[(j + 2) % 3] = *reinterpret_cast<const uint4*>(cur + (kc ^ (16 * (j + 2))));
            if (j == C::KL / 2 - 1) {
#pragma unroll
              for (int r = 0; r < C::KR; ++r)
                rope[r] = *reinterpret_cast<const uint4*>(cur + C::ROPE_OFF + (kr ^ (32 * r)));
            }
            const uint4 raw = ring[j % 3];
            SL = M::mma(cvt8(raw.x, raw.y), qf[2 * j], j == 0 ? floatx16{} : SL);
            SL = M::mma(cvt8(raw.z, raw.w), qf[2 * j + 1], SL);
          }
        } else {
#pragma unroll
          for (int r = 0; r < C::KR; ++r)
            SR = M::mma(__builtin_bit_cast(bf16x8_t, rope[r]), qf[C::KL + r], r == 0 ? floatx16{} : SR);
        }
        work(g);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // softmax of one stage in five pieces: g = -1 before the score MFMAs of the next stage (it
    // frees the stage's raw scores), g = 0..3 after their first four groups; pieces 2 and 3 store
    // P^T (p * scale, bf16: the B operand of the consumer's P.V MFMA, lane for lane) into LDS.  The
    // token scales are read into sc ahead of piece -1 and again ahead of piece 2.
    float sv[16], sc[16], mt = 0.f, psum = 0.f;
    auto read_scales = [&](const char* cur) __attribute__((always_inline)) {
      const float4* sp = reinterpret_cast<const float4*>(cur + C::SC_OFF);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // registers 4 q .. 4 q + 3 hold tokens 16 (q / 2) + 8 h + 4 (q % 2) ..
        const float4 v = sp[(16 * (q >> 1) + 8 * h + 4 * (q & 1)) / 4];
        sc[4 * q] = v.x, sc[4 * q + 1] = v.y, sc[4 * q + 2] = v.z, sc[4 * q + 3] = v.w;
      }
    };
    auto softmax_piece = [&](const floatx16& SL, const floatx16& SR, int g, int n, bool last_stage, const char* cur)
                             __attribute__((always_inline)) {
      const int stage0 = t_begin + n * kTile;
      if (g == -1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = __builtin_fmaf(sc[i], SL[i], SR[i]);
        if (last_stage) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sv[i] = (stage0 + M::token_of(i, h) < t_end) ? sv[i] : -INFINITY;
        }
        // maximum (NaN-propagating) is one v_maximum3_f32 per two values; a NaN score makes its
        // head's row NaN either way
        mt = sv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = __builtin_elementwise_maximum(mt, sv[i]);
      } else if (g == 0) {
        mt = fmaxf(mt, xor32(mt)) * c2;
        if (!fixed && n == 0) ref = mt;
        mmax = fmaxf(mmax, mt);
        over |= mt > ref + kRefSlack;
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -ref));
      } else if (g == 1) {
#pragma unroll
        for (int i = 8; i < 16; ++i) sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -ref));
        read_scales(cur);
      } else {
        // g = 2: tokens of k-step 0 (registers 0..7), g = 3: k-step 1 (registers 8..15)
        const int p2 = g - 2;
        if (last_stage) {
          // rows past the unit's end have p = 0; their scale slots may hold anything
#pragma unroll
          for (int j = 0; j < 8; ++j)
            sc[8 * p2 + j] = (stage0 + M::token_of(8 * p2 + j, h) < t_end) ? sc[8 * p2 + j] : 0.f;
        }
        bf16x8_t f;
        if (p2 == 0) psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          f[j] = (__bf16)(sv[8 * p2 + j] * sc[8 * p2 + j]);
          psum += sv[8 * p2 + j];
        }
        *reinterpret_cast<bf16x8_t*>(pslot + (n & 1) * (C::ROLE * C::PBLK) + p2 * 1024) = f;
        if (p2 == 1) l_run += psum + xor32(psum);
      }
    };

    for (int pass = 0; pass < 2; ++pass) {
      l_run = 0.f;
      over = false;
      if (pass == 1) {
        ref = mmax;
        fixed = true;
      }
      if (nstage > 0) {
        prologue();
        floatx16 SLA, SRA, SLB, SRB;
        read_scales(lds);
        scores(lds, SLA, SRA, [](int) {});
        // iteration n: scores of stage n+1 with the softmax of stage n between them; P of stage n
        // to LDS.  One more iteration (n = nstage) only meets the consumers' barrier.
        for (int n = 0; n <= nstage; ++n) {
          if (n + 1 < nstage) wait_copies(min(C::AHEAD - 2, nstage - 2 - n));
          lds_barrier();
          if (n == nstage) break;
          const char* cur = lds + buf_of(n);
          const bool last = n + 1 == nstage;
          const bool refill_now = n + C::AHEAD < nstage;
          const StageSrc src = stage_src(t_begin + (n + C::AHEAD) * kTile);
          const unsigned refill = buf_of(n + C::AHEAD);
          softmax_piece(SLA, SRA, -1, n, last, cur);
          if (!last) {
            scores(lds + buf_of(n + 1), SLB, SRB, [&](int g) __attribute__((always_inline)) {
              if (g < 4) softmax_piece(SLA, SRA, g, n, false, cur);
              // this wave's copies of stage n + AHEAD, spread over the five score groups
#pragma unroll
              for (int j = 0; j < C::CPW_P; ++j)
                if (refill_now && g == (5 * j) / C::CPW_P) copy_block(src, refill, j);
            });
            read_scales(lds + buf_of(n + 1));
            SLA = SLB;
            SRA = SRB;
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) softmax_piece(SLA, SRA, g, n, true, cur);
          }
        }
      }
      // run the unit again with the exact max if any head of the work group overflowed its reference
      if (threadIdx.x == 0) s_again = 0;
      __syncthreads();
      if (__any(over) && lane == 0) s_again = 1;
      __syncthreads();
      if (!s_again || pass == 1) break;
      __syncthreads();
    }
    // the row sums for the consumers; the lse
    if (h == 0) lds_l[rw * 32 + col] = l_run;
    const float lse_v = (ref + log2f(l_run)) * kLn2;
    if (h == 0) {
      if (nsplit == 1)
        a.lse[(size_t)b * a.rows + head] = lse_v;
      else
        a.part_lse[(((size_t)unit * a.groups + gs) * C::HBG + hb) * 32 + col] = lse_v;
    }
    __syncthreads();
    return;
  }

  // ================================ consumer: P.V and the copies ================================
  // value operand of column block c and token k-step p2: (vt0 + p2 * 16 rows) ^ 32 c
  int vt0;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tok = 8 * (g16 >> 1) + (i16 >> 1);
    vt0 = tok * C::CROW + gl * 256 + ((((g16 & 1) ^ ckey(tok)) & 15) << 4) + (i16 & 1) * 8;
  }
  floatx16 acc[C::CB];

  // O^T += V^T . P^T over the eight column blocks and two token k-steps of stage m, in four groups
  // of four MFMAs with `work(g)` after group g (the copies, one per group: a copy holds up the wave
  // that issues it, so they are spread rather than issued in a burst); the transposed code reads
  // run four MFMAs ahead
  auto pv = [&](int m, auto&& work) __attribute__((always_inline)) {
    const char* cur = lds + buf_of(m);
    const char* pp = pslot + (m & 1) * (C::ROLE * C::PBLK);
    const bf16x8_t pf0 = *reinterpret_cast<const bf16x8_t*>(pp);
    const bf16x8_t pf1 = *reinterpret_cast<const bf16x8_t*>(pp + 1024);
    int v0 = vt0;
    asm volatile("" : "+v"(v0));
    auto vread = [&](int i) -> int2v {
      const int p2 = i / C::CB, c = i % C::CB;
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_int2v*)(cur + ((v0 + p2 * 16 * C::CROW) ^ (32 * c))));
    };
    constexpr int N = 2 * C::CB;
    int2v ring[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ring[i] = vread(i);
#pragma unroll
    for (int g = 0; g < N / 4; ++g) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int i = 4 * g + jj;
        const int2v raw = ring[i & 3];
        if (i + 4 < N) ring[i & 3] = vread(i + 4);
        acc[i % C::CB] = M::mma(cvt8((unsigned)raw[0], (unsigned)raw[1]), i < C::CB ? pf0 : pf1, acc[i % C::CB]);
      }
      work(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int k = 0; k < C::CB; ++k) acc[k] = floatx16{};
    if (nstage > 0) {
      prologue();
      // iteration n: (stage n+1 must land before the producers score it) P.V of stage n-1, and the
      // copies of stage n + AHEAD into the buffer stage n-2 has left
      for (int n = 0; n <= nstage; ++n) {
        if (n + 1 < nstage) wait_copies(min(C::AHEAD - 2, nstage - 2 - n));
        lds_barrier();
        const bool refill_now = n + C::AHEAD < nstage;
        const StageSrc src = stage_src(t_begin + (n + C::AHEAD) * kTile);
        const unsigned refill = buf_of(n + C::AHEAD);
        if (n >= 1) {
          pv(n - 1, [&](int g) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < C::CPW_C; ++j)
              if (refill_now && g == (4 * j) / C::CPW_C) copy_block(src, refill, j);
          });
        } else if (refill_now) {
          copy_stage(src, refill);
        }
      }
    }
    // the producers decide whether the unit runs again
    __syncthreads();
    __syncthreads();
    if (!s_again || pass == 1) break;
    __syncthreads();
  }

  // ---- epilogue: the layouts of decode.hip with one wave per head block
  __syncthreads();  // the producers' row sums
  const float l_run = lds_l[rw * 32 + col];
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  if (nsplit == 1) {
    const size_t orow = (size_t)b * a.rows + head;
#pragma unroll
    for (int k = 0; k < C::CB; ++k) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = k * 32 + 8 * g4 + 4 * h;
        const float o0 = acc[k][4 * g4 + 0] * inv_l, o1 = acc[k][4 * g4 + 1] * inv_l;
        const float o2 = acc[k][4 * g4 + 2] * inv_l, o3 = acc[k][4 * g4 + 3] * inv_l;
        if (a.out_bf16) {
          __bf16* dst = static_cast<__bf16*>(a.out) + orow * C::DL + c;
          *reinterpret_cast<bf16x4_t*>(dst) = bf16x4_t{(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
        } else {
          float* dst = static_cast<float*>(a.out) + orow * C::DL + c;
          *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  } else {
    const size_t blk = ((size_t)unit * a.groups + gs) * C::HBG + hb;
    if (a.part_bf16) {
      __bf16* dst = static_cast<__bf16*>(a.part_out) + blk * (32 * C::DL);
#pragma unroll
      for (int k = 0; k < C::CB; ++k)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x8_t v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)(acc[k][8 * j + e] * inv_l);
          *reinterpret_cast<bf16x8_t*>(dst + ((k * 2 + j) * 64 + lane) * 8) = v;
        }
    } else {
      float* dst = static_cast<float*>(a.part_out) + blk * (32 * C::DL);
#pragma unroll
      for (int k = 0; k < C::CB; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(dst + ((k * 4 + j) * 64 + lane) * 4) =
              make_float4(acc[k][4 * j] * inv_l, acc[k][4 * j + 1] * inv_l, acc[k][4 * j + 2] * inv_l,
                          acc[k][4 * j + 3] * inv_l);
    }
  }
}

template <int G>
int wgs_per_cu8() {
  static int cache[kMaxDevices] = {};
  return occupancy_cached(cache, reinterpret_cast<const void*>(decode_pipe8_kernel<G>), G * 256);
}

}  // namespace

// Shapes of this kernel: an fp8 cache of 256-dim latent groups plus a 64-dim bf16 RoPE key, a bf16
// query, 64 heads per group, and one or two groups per work group.
bool decode_pipe8_serves(const ld_problem& p, int nsets, int hblocks) {
  return p.kv_dtype == LD_FP8_E4M3 && p.q_dtype == LD_BF16 &&
         (p.variant == LD_VARIANT_GLA || p.variant == LD_VARIANT_MLA) && p.d_latent == 256 && p.d_rope == 64 &&
         hblocks == 2 && p.num_q_heads == 64 * p.num_groups && (nsets == 1 || nsets == 2) &&
         p.num_groups % nsets == 0;
}

int launch_decode_pipe8(const ld_problem& p, const DecodeArgs& a, void* stream) {
  if (!decode_pipe8_serves(p, a.nsets, a.hblocks)) return -1;
  const int units8 = (a.max_units + 7) / 8 * 8;
  const dim3 grid(units8 * a.wg_per_unit);
  if (a.nsets == 2)
    hipLaunchKernelGGL(decode_pipe8_kernel<2>, grid, dim3(512), 0, static_cast<hipStream_t>(stream), a, a.block_table);
  else
    hipLaunchKernelGGL(decode_pipe8_kernel<1>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a, a.block_table);
  return (int)hipGetLastError();
}

int decode_pipe8_wgs_per_cu(int nsets) { return nsets == 2 ? wgs_per_cu8<2>() : wgs_per_cu8<1>(); }

}  // namespace ld
