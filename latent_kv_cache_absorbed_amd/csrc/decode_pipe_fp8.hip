// Software-pipelined decode kernel for latent caches stored as fp8 E4M3 codes with a per-token
// scale: GLA with 256-dim latent groups and 64 heads per group ("Mamba核心作者新作…" (jsbsmhs.com),
// the GLA section and the FP8 serving test), every group of the cache in one work group (GLA-2:
// two groups, 128 heads; one group, 64 heads: a tensor-parallel share), gfx950.  See
// include/latent_decode.h for the operation and its sources.
//
// The structure is decode_pipe.hip's: one wave per SIMD and per 32-head block, over every score and
// value dim of its group,
//   Q (32 heads x (256 + 64) bf16)   80 VGPRs, loaded once per unit
//   O (32 heads x 256 f32)          128 AGPRs, accumulated by the P.V MFMAs
//   S latent and rope parts          32 VGPRs per stage, two stages live
// the scores of stage n+1 interleaved with the softmax of stage n, then the P.V of stage n, and the
// fixed per-unit softmax reference (a second pass with the exact max when a score runs more than
// 2^kRefSlack above it).
//
// The stage is copied as stored: 32 rows of codes (G x 256 bytes), 32 rope keys (bf16) and 32
// scales, 20.6 KB for GLA-2 against 36.9 KB for a bf16 stage of the same rows, into six stage
// buffers (five stages in flight).  The codes are converted to bf16 when an MFMA operand is read:
//   score operand (8 dims of one token per lane): one 16-byte read gives two k-steps' operands
//   value operand (8 tokens of one column per lane): ds_read_b64_tr_b8, which hands lane i of each
//     16 lanes byte i of the 8 rows that lane pairs (2e, 2e+1) point at
// and v_cvt_scalef32_pk_bf16_fp8 (scale 1) makes each pair of codes two bf16, exactly.  The
// per-token scale multiplies the latent part of the score and P (the value rows), as decode.hip
// does for fp8: s = scale * (q_lat . e) + q_rope . k_r; P.V takes bf16(p * scale); the row sum
// takes p.
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
  static constexpr int WAVES = G * HBG;
  static constexpr int THREADS = WAVES * kWaveSize;
  static constexpr int CROW = G * DL;                   // bytes of a token's codes (LDS and memory)
  static constexpr int CODES = kTile * CROW;
  static constexpr int RW = DR * 2;                     // rope row bytes
  static constexpr int MR = swz_mask(RW);
  static constexpr int ROPE_OFF = CODES;
  static constexpr int SC_OFF = ROPE_OFF + kTile * RW;
  static constexpr int BUF = SC_OFF + kTile * 4;
  static constexpr int NBUF = 6;
  static constexpr int AHEAD = NBUF - 1;                // stages copied ahead of the one computed
  static constexpr int CODE_CP = CODES / 1024 / WAVES;  // 1 KB copies per wave and stage
  static constexpr int ROPE_CP = kTile * RW / 1024 / WAVES;
  static constexpr int CPW = CODE_CP + ROPE_CP + 1;     // + the scales (every wave copies them)
  static constexpr int KL = DL / 16;                    // latent k-steps of S
  static constexpr int KR = DR / 16;                    // rope k-steps of S
  static constexpr int CB = DL / 32;                    // 32-column blocks of O
  static_assert(CODES % (1024 * WAVES) == 0 && (kTile * RW) % (1024 * WAVES) == 0, "copy dealing");
  static_assert(CPW <= 9, "one copy per work slot of an iteration");
  static_assert(KL == 16 && KR == 4 && CB == 8, "the work slots are laid out for 256 + 64 dims");
  static_assert(NBUF * BUF + 4 * kUnitPages + 64 <= 160 * 1024, "LDS budget");
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
__global__ __launch_bounds__(G * 128) void decode_pipe8_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  using C = P8Cfg<G>;
  using M = Mma<KV_BF16>;
  __shared__ __attribute__((aligned(256))) char lds[C::NBUF * C::BUF];
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
  // query token qi of the unit's work groups (token qi sees the first L_b - qlen + 1 + qi rows);
  // the work group serves every cache group of that token: query sets qi * G .. qi * G + G - 1
  const int qi = sb;
  if (a.qlen > 1) {
    const int Lb = clampi(a.seq_lens[b], 0, a.max_pages * a.page_size);
    t_end = max(t_begin, min(t_end, Lb - a.qlen + 1 + qi));
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int gl = wave / C::HBG;  // this wave's group (latent slice)
  const int hb = wave % C::HBG;  // and 32-head block in it
  const int gs = qi * G + gl;
  const int head_in_set = hb * 32 + col;
  const int head = gs * a.heads_per_set + head_in_set;
  const int32_t* __restrict__ bt_row = block_table + (size_t)b * a.max_pages;
  const int page_size = a.page_size;
  const int first_page = t_begin / page_size;
  const int unit_pages = t_end > t_begin ? (t_end - 1) / page_size - first_page + 1 : 0;
  for (int i = threadIdx.x; i < unit_pages && i < kUnitPages; i += C::THREADS)
    lds_pages[i] = clampi(bt_row[first_page + i], 0, a.num_pages - 1);
  __syncthreads();

  // ---- stage copies: wave w copies 1 KB blocks w, w + WAVES, .. of the code region, then of the
  // rope region, then the 128 bytes of scales (lanes 0..7; every wave copies the same bytes, so that
  // every wave issues CPW copies a stage).  A stage's rows lie in one page.
  const char* kbase = static_cast<const char*>(a.k);
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
  auto copy_block = [&](const StageSrc& src, unsigned buf, int j) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // re-derived per copy, so the offsets hold no registers across the loop
    if (j < C::CODE_CP) {
      const int q = wave + C::WAVES * j;
      const int t = (q * 1024 + ln * 16) / C::CROW;
      const int slot = ((q * 1024 + ln * 16) % C::CROW) >> 4;
      const int c = (slot & 15) ^ ckey(t);
      const int tu = min((q * 1024) / C::CROW, src.tlast);
      unsigned voff = (unsigned)((min(t, src.tlast) - tu) * C::CROW + (slot & ~15) * 16 + c * 16);
      asm volatile("" : "+v"(voff));
      dma16_asm_at(kbase + (src.r0 + tu) * (size_t)C::CROW, voff, lds_u + buf + q * 1024);
    } else if (j < C::CODE_CP + C::ROPE_CP) {
      const int q = wave + C::WAVES * (j - C::CODE_CP);
      const int t = q * (1024 / C::RW) + ln / (C::RW / 16);
      const int c = (ln % (C::RW / 16)) ^ (swz_key(t) & C::MR);
      const int tu = min(q * (1024 / C::RW), src.tlast);
      unsigned voff = (unsigned)((min(t, src.tlast) - tu) * C::RW + c * 16);
      asm volatile("" : "+v"(voff));
      dma16_asm_at(rbase + (src.r0 + tu) * (size_t)C::RW, voff, lds_u + buf + C::ROPE_OFF + q * 1024);
    } else if (ln < kTile * 4 / 16) {
      dma16_asm_at(sbase + src.r0 * 4, (unsigned)(ln * 16), lds_u + buf + C::SC_OFF);
    }
  };
  // copy j of an iteration goes after work slot slot_of(j): slots 0..4 follow the five groups of
  // score MFMAs, slots 5..8 the four groups of P.V MFMAs (a copy holds up the wave that issues it,
  // so they are spread rather than issued in a burst)
  auto slot_of = [](int j) { return j < 3 ? 2 * j : 2 + j; };

  // ---- this lane's query fragments (B operand of S^T = K . Q^T).  Latent k-steps come in pairs:
  // lanes of half h read code chunk j + 8 h of their token for pair j, whose first eight codes are
  // k-step 2 j and last eight k-step 2 j + 1; the query is laid out to match.
  bf16x8_t qf[C::KL + C::KR];
  {
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

  // ---- per-lane LDS offsets within a stage buffer.  Score: code pair j at kc0 ^ 16 j; rope k-step
  // j at ROPE_OFF + (kr0 ^ 32 j).  Value operand of column block c and token k-step p2:
  // (vt0 + p2 * 16 rows) ^ 32 c.
  const int tr = M::row_token(col);
  const int kc0 = tr * C::CROW + gl * 256 + (((8 * h) ^ ckey(tr)) << 4);
  const int kr0 = lds_off(tr, C::RW, C::MR, h * 16);
  int vt0;
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int tok = 8 * (g16 >> 1) + (i16 >> 1);
    vt0 = tok * C::CROW + gl * 256 + ((((g16 & 1) ^ ckey(tok)) & 15) << 4) + (i16 & 1) * 8;
  }

  const int nstage = (t_end - t_begin + kTile - 1) / kTile;
  const float c2 = a.scale_log2;

  floatx16 acc[C::CB];
  float l_run = 0.f;       // sum of 2^(score - ref) over the unit
  float ref = 0.f;         // fixed reference of this head (log2 domain)
  float mmax = -INFINITY;  // exact max of this head's scaled scores over the unit (log2 domain)
  bool over = false;       // a stage max exceeded ref + kRefSlack
  bool fixed = false;      // second pass: ref = mmax of the first

  // The 20 score MFMAs of one stage in five groups of four (latent pairs 2g, 2g + 1 for g < 4, the
  // rope k-steps for g = 4), `work(g)` after each group; code reads run two pairs ahead.
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
          const bf16x8_t a0 = cvt8(raw.x, raw.y);
          const bf16x8_t a1 = cvt8(raw.z, raw.w);
          SL = M::mma(a0, qf[2 * j], j == 0 ? floatx16{} : SL);
          SL = M::mma(a1, qf[2 * j + 1], SL);
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

  // softmax of one stage in five pieces: g = -1 before the score MFMAs of the next stage (it frees
  // the stage's raw scores), g = 0..3 after their first four groups.  Leaves pf (P^T fragments of
  // p * scale, bf16) and updates l_run / ref / mmax / over.  The token scales are read into sc
  // ahead of piece -1 and again ahead of piece 2 (so that they hold no registers in between).
  bf16x8_t pf[2];
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
  auto softmax_piece = [&](const floatx16& SL, const floatx16& SR, int g, bool first, bool last_stage, int stage0,
                           const char* cur) __attribute__((always_inline)) {
    if (g == -1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = __builtin_fmaf(sc[i], SL[i], SR[i]);
      if (last_stage) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = (stage0 + M::token_of(i, h) < t_end) ? sv[i] : -INFINITY;
      }
      mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])),
                           fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]))));
    } else if (g == 0) {
      mt = fmaxf(mt, xor32(mt)) * c2;
      if (!fixed && first) ref = mt;
      mmax = fmaxf(mmax, mt);
      over |= mt > ref + kRefSlack;
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -ref));
    } else if (g == 1) {
#pragma unroll
      for (int i = 8; i < 16; ++i) sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -ref));
      read_scales(cur);
    } else if (g == 2) {
      if (last_stage) {
        // rows past the unit's end have p = 0; their scale slots may hold anything, so it is dropped
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = (stage0 + M::token_of(i, h) < t_end) ? sc[i] : 0.f;
      }
      bf16x8_t f;
      psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f[j] = (__bf16)(sv[j] * sc[j]);
        psum += sv[j];
      }
      pf[0] = f;
    } else if (g == 3) {
      bf16x8_t f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f[j] = (__bf16)(sv[8 + j] * sc[8 + j]);
        psum += sv[8 + j];
      }
      pf[1] = f;
      l_run += psum + xor32(psum);
    }
  };

  // O^T += V^T . P^T over the eight column blocks and two token k-steps, in groups of four MFMAs
  // (`work(g)` after group g); the transposed code reads run four MFMAs ahead
  auto pv = [&](const char* cur, auto&& work) __attribute__((always_inline)) {
    int v0 = vt0;
    asm volatile("" : "+v"(v0));
    auto vread = [&](int i) -> int2v {
      const int p2 = i / C::CB, c = i % C::CB;
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_int2v*)(cur + ((v0 + p2 * 16 * C::CROW) ^ (32 * c))));
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
        mfma_pv_valu_a(acc[i % C::CB], cvt8((unsigned)raw[0], (unsigned)raw[1]), pf[i / C::CB]);
      }
      work(5 + g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // this wave's copies of stage n have landed, `later` stages' copies being issued after them
  auto wait_copies = [&](int later) __attribute__((always_inline)) {
    static_assert(C::AHEAD - 1 <= 4, "wait cases");
    if (later <= 0)
      wait_vmcnt<0>();
    else if (later == 1)
      wait_vmcnt<C::CPW>();
    else if (later == 2)
      wait_vmcnt<2 * C::CPW>();
    else if (later == 3)
      wait_vmcnt<3 * C::CPW>();
    else
      wait_vmcnt<4 * C::CPW>();
  };
  auto buf_of = [](int n) { return (unsigned)((n % C::NBUF) * C::BUF); };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int k = 0; k < C::CB; ++k) acc[k] = floatx16{};
    l_run = 0.f;
    over = false;
    if (pass == 1) {
      ref = mmax;
      fixed = true;
    }
    if (nstage > 0) {
      // prologue: stages 0 .. AHEAD-1 in flight, scores of stage 0
      const int pre = min(C::AHEAD, nstage);
      for (int m = 0; m < pre; ++m) {
        const StageSrc src = stage_src(t_begin + m * kTile);
#pragma unroll
        for (int j = 0; j < C::CPW; ++j) copy_block(src, buf_of(m), j);
      }
      wait_copies(pre - 1);
      lds_barrier();
      floatx16 SLA, SRA, SLB, SRB;
      read_scales(lds);
      scores(lds, SLA, SRA, [](int) {});
      // iteration n: scores of stage n+1 with the softmax of stage n between them, then P.V of n;
      // the copies of stage n + AHEAD go into the buffer stage n - 1 has left
      auto iter = [&](int n, floatx16& SL, floatx16& SR, floatx16& SLn, floatx16& SRn) __attribute__((always_inline)) {
        const int stage0 = t_begin + n * kTile;
        const bool refill_now = n + C::AHEAD < nstage;
        const StageSrc src = stage_src(t_begin + (n + C::AHEAD) * kTile);
        const unsigned refill = buf_of(n + C::AHEAD);
        const char* cur = lds + buf_of(n);
        const bool last = n + 1 == nstage;
        softmax_piece(SL, SR, -1, n == 0, last, stage0, cur);
        if (!last) {
          wait_copies(min(C::AHEAD - 2, nstage - 2 - n));
          lds_barrier();
          scores(lds + buf_of(n + 1), SLn, SRn, [&](int g) __attribute__((always_inline)) {
            softmax_piece(SL, SR, g, n == 0, false, stage0, cur);
#pragma unroll
            for (int j = 0; j < C::CPW; ++j)
              if (refill_now && slot_of(j) == g) copy_block(src, refill, j);
          });
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) softmax_piece(SL, SR, g, n == 0, true, stage0, cur);
        }
        pv(cur, [&](int s) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < C::CPW; ++j)
            if (refill_now && slot_of(j) == s) copy_block(src, refill, j);
          // the next stage's scales, for its piece -1 (its copies have landed: waited above)
          if (s == 7 && !last) read_scales(lds + buf_of(n + 1));
        });
      };
      // one iteration per trip, the next stage's scores moved into place after it: unrolling by two
      // with the roles of the two score sets swapped makes the register allocator keep a third set
      // and move the query into AGPRs
      for (int n = 0; n < nstage; ++n) {
        iter(n, SLA, SRA, SLB, SRB);
        SLA = SLB;
        SRA = SRB;
      }
    }
    mfma_pv_drain();
    // run the unit again with the exact max if any head of the work group overflowed its reference
    if (threadIdx.x == 0) s_again = 0;
    __syncthreads();
    if (__any(over) && lane == 0) s_again = 1;
    __syncthreads();
    if (!s_again || pass == 1) break;
    __syncthreads();
  }

  // ---- epilogue: the layouts of decode.hip with one wave per head block
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_v = (ref + log2f(l_run)) * kLn2;
  if (nsplit == 1) {
    const size_t orow = (size_t)b * a.rows + head;
    if (h == 0) a.lse[orow] = lse_v;
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
    if (h == 0) a.part_lse[blk * 32 + col] = lse_v;
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
  return occupancy_cached(cache, reinterpret_cast<const void*>(decode_pipe8_kernel<G>), G * 128);
}

}  // namespace

// Shapes of this kernel: an fp8 cache of 256-dim latent groups plus a 64-dim bf16 RoPE key, a bf16
// query, 64 heads per group, and every group of the cache (one or two) in one work group.
bool decode_pipe8_serves(const ld_problem& p, int nsets, int hblocks) {
  return p.kv_dtype == LD_FP8_E4M3 && p.q_dtype == LD_BF16 &&
         (p.variant == LD_VARIANT_GLA || p.variant == LD_VARIANT_MLA) && p.d_latent == 256 && p.d_rope == 64 &&
         hblocks == 2 && p.num_q_heads == 64 * p.num_groups && nsets == p.num_groups &&
         (p.num_groups == 1 || p.num_groups == 2);
}

int launch_decode_pipe8(const ld_problem& p, const DecodeArgs& a, void* stream) {
  if (!decode_pipe8_serves(p, a.nsets, a.hblocks)) return -1;
  const int units8 = (a.max_units + 7) / 8 * 8;
  const dim3 grid(units8 * a.wg_per_unit);
  if (p.num_groups == 2)
    hipLaunchKernelGGL(decode_pipe8_kernel<2>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a, a.block_table);
  else
    hipLaunchKernelGGL(decode_pipe8_kernel<1>, grid, dim3(128), 0, static_cast<hipStream_t>(stream), a, a.block_table);
  return (int)hipGetLastError();
}

int decode_pipe8_wgs_per_cu(const ld_problem& p) { return p.num_groups == 2 ? wgs_per_cu8<2>() : wgs_per_cu8<1>(); }

}  // namespace ld
