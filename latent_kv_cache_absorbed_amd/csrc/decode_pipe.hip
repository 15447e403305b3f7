// Software-pipelined decode kernel for the latent shapes whose query set over one latent slice fits
// one work group of one wave per 32-head block, gfx950: absorbed MLA (128 heads over one 576-dim
// shared row) and MLRA (128 heads over one 128-dim branch plus the shared 64-dim rope key, one work
// group per branch).  See include/latent_decode.h for the operation and its sources.
//
// Each wave is one block of 32 heads over all score and value dims.  For MLA (one wave per SIMD):
//   Q (32 heads x 576 bf16)  144 VGPRs, loaded once per unit
//   O (32 heads x 512 f32)   256 AGPRs, accumulated by the P.V MFMAs
//   S (32 tokens x 32 heads)  16 VGPRs per stage, two stages live
// (an MLRA branch: Q 48 VGPRs, O 64 AGPRs, two work groups per CU).
// No wave shares scores with another, so the only work-group barrier is the one that recycles the
// stage buffers.  Each wave runs its stages as a software pipeline: while the score MFMAs of stage
// n+1 run, the wave computes the softmax of stage n between them, then issues the P.V MFMAs of stage
// n.  The MFMA pipe of the SIMD so stays busy with one wave, and the softmax costs no MFMA time.
//
// Softmax reference.  O lives in AGPRs, which VALU instructions cannot scale in place, so the kernel
// never rescales O: every head takes the max of its unit's first stage as a fixed reference r (log2
// domain) and accumulates p = 2^(s - r).  Probabilities above 1 are fine up to 2^kRefSlack; a stage
// whose max exceeds r + kRefSlack flags the unit, and the work group then runs the unit once more
// with r = the unit's exact max (known from the first pass), where no p exceeds 1.  The normalised
// result does not depend on r (it cancels between numerator and denominator).
//
// Stage buffers, DMA, swizzle, MFMA layouts and the split-partial format are those of decode.hip
// (decode_common.h), so the plan and the combine are shared.
#include <hip/hip_runtime.h>

#include "decode_common.h"
#include "plan_common.h"
#include "ld_internal.h"

namespace ld {
namespace {

template <int DL, int DR, int HB, int G>
struct PCfg {
  using M = Mma<KV_BF16>;
  static constexpr int WAVES = HB;
  static constexpr int GROW = G * DL * 2 + DR * 2;   // cached row bytes: G latent slices, then the rope key
  static constexpr int ROPE_COL = G * DL * 2;        // byte offset of the rope key in a cached row
  static constexpr int THREADS = WAVES * kWaveSize;
  static constexpr int KL = DL / 16;                 // latent k-steps of S
  static constexpr int KR = DR / 16;                 // rope k-steps of S
  static constexpr int KS = KL + KR;
  static constexpr int CB = DL / 32;                 // 32-column blocks of O
  static constexpr int LW = DL * 2;                  // latent row bytes in LDS
  static constexpr int RW = DR * 2;                  // rope row bytes in LDS
  static constexpr int SETCH = DL * 2 / 16;
  static constexpr int MLS = cmin(SETCH - 1, swz_mask(LW));
  static constexpr int MR = swz_mask(RW);
  static constexpr int ROPE_OFF = kTile * LW;
  static constexpr int BUF = ROPE_OFF + kTile * RW;
  static constexpr int NBUF = 4;
  static constexpr int DMA_BLOCKS = kTile * (LW + RW) / 1024;
  static constexpr int DMA_PER_WAVE = DMA_BLOCKS / WAVES;
  static constexpr int LPW = kTile * LW / 1024 / WAVES;   // latent copies per wave and stage
  static constexpr int NGS = KS / 4;                     // groups of four score MFMAs per stage
  static constexpr int NKL = (MLS + 1) / 2;          // latent k-steps per swizzle group
  static constexpr int NVT = (MLS >> 2) + 1;          // V column blocks per swizzle group
  static_assert(DMA_BLOCKS % WAVES == 0, "every wave issues the same number of copies");
  static_assert(KS % 4 == 0 && CB % 4 == 0, "k-steps and column blocks come in groups of four");
  static_assert((kTile * LW / 1024) % WAVES == 0 && kTile * RW == 1024 * WAVES, "copy dealing: one rope block per wave");
  static_assert(NGS == 9 || NGS == 3, "the softmax is laid out over nine or three score groups");
  // Where the copies of stage n + 3 go in iteration n (a copy instruction holds up the wave that
  // issues it, so they are paced rather than issued in a burst).  576-dim rows: nine copies, one per
  // two groups of MFMAs (five among the nine score groups, four among the eight P.V groups).
  // 192-dim rows: three copies, one after each of the three score groups.
  static constexpr __device__ bool copy_after_score(int g) { return NGS == 9 ? (g & 1) == 0 : true; }
  static constexpr __device__ int score_copy(int g) { return NGS == 9 ? g / 2 : g; }
  static constexpr __device__ bool copy_after_pv(int g) { return NGS == 9 ? (g & 1) != 0 : false; }
  static constexpr __device__ int pv_copy(int g) { return 5 + g / 2; }
  static_assert(2 * KR <= MR + 1, "rope row must lie in one swizzle group");
  static_assert(pow2(LW) && pow2(RW) && (kTile * RW) % 1024 == 0, "row sizes");
  static_assert(NBUF * BUF + 4 * kUnitPages + 64 <= 160 * 1024, "LDS budget");
};

template <int DL, int DR, int HB, int G, int MINB>
__global__ __launch_bounds__(HB * 64, MINB) void decode_pipe_kernel(DecodeArgs a, const int32_t* __restrict__ block_table) {
  using C = PCfg<DL, DR, HB, G>;
  using M = typename C::M;
  __shared__ __attribute__((aligned(128))) char lds_b0[C::BUF];
  __shared__ __attribute__((aligned(128))) char lds_b1[C::BUF];
  __shared__ __attribute__((aligned(128))) char lds_b2[C::BUF];
  __shared__ __attribute__((aligned(128))) char lds_b3[C::BUF];
  __shared__ int lds_pages[kUnitPages];
  __shared__ int s_unit[5];
  __shared__ int s_again;

  // unit of this work group: the same XCD-blocked mapping as decode_kernel
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
  // query token qi and latent slice `branch` of the work group (several query tokens: token qi sees
  // the first L_b - qlen + 1 + qi rows); query set gs = qi * G + branch (MLA: one slice, G = 1)
  const int qi = sb / G;
  const int branch = sb - qi * G;
  const int gs = qi * G + branch;
  if (a.qlen > 1) {
    const int Lb = clampi(a.seq_lens[b], 0, a.max_pages * a.page_size);
    t_end = max(t_begin, min(t_end, Lb - a.qlen + 1 + qi));
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int hb = wave;
  const int head_in_set = hb * 32 + col;
  const bool valid = head_in_set < a.heads_per_set;
  const int head = qi * a.heads_per_set + (valid ? head_in_set : 0);
  const int32_t* __restrict__ bt_row = block_table + (size_t)b * a.max_pages;
  const int page_size = a.page_size;
  const int first_page = t_begin / page_size;
  const int unit_pages = t_end > t_begin ? (t_end - 1) / page_size - first_page + 1 : 0;
  for (int i = threadIdx.x; i < unit_pages && i < kUnitPages; i += C::THREADS)
    lds_pages[i] = clampi(bt_row[first_page + i], 0, a.num_pages - 1);
  __syncthreads();

  const int grow_bytes = C::GROW;
  const size_t page_bytes = (size_t)page_size * C::GROW;
  const int lat_col = branch * (DL * 2);  // byte offset of the work group's latent slice in a cached row
  const char* kbase = static_cast<const char*>(a.k);
  // Stage copies.  Wave w copies 1 KB blocks w, w + 4, .. of the latent region and block w of the
  // rope region (the dealing of dma_region): copy j < LPW is latent block w + 4 j (LPW = 8 for a
  // 512-dim slice, 2 for a 128-dim one), copy LPW the rope block.  The stage's rows come from one
  // page: its id is read from LDS once per stage.
  struct StageSrc {
    const char* rows;  // the stage's first cached row
    int tlast;         // last valid row of the stage (rows past it repeat it)
  };
  auto stage_src = [&](int stage0) -> StageSrc {
    const int pi = stage0 / page_size - first_page;
    const int page = __builtin_amdgcn_readfirstlane(lds_pages[min(pi, kUnitPages - 1)]);
    const size_t r0 = (size_t)page * page_size + (stage0 % page_size);
    return StageSrc{kbase + r0 * (size_t)grow_bytes, t_end - 1 - stage0};
  };
  // Stage copies in few instructions.  The source row of a copy lane is min(token, tlast) (rows
  // past a unit's end repeat its last row) and its LDS chunk is the lane's chunk XORed with
  // swz_key(token); for the row sizes below the key splits into a part fixed by the copy (a scalar)
  // and a part fixed by the lane.  The scalar part passes through an empty asm, so the per-lane
  // offsets depend on a value made inside the loop and are not hoisted into registers held across it.
  //  - 1 KB latent rows (MLA): copy j holds stage row q = wave + 4 j; lane ln lands chunk
  //    ln ^ swz_key(q), and swz_key(q) = kw ^ kj: bits 1 and 2 are q's two low bits (the wave), bit 3
  //    is the wave's bit 0 XOR j's bit 1, bit 0 is bit 0 of j ^ (j >> 1).
  //  - 256-byte latent rows (an MLRA branch): copy j holds rows 4 q .. 4 q + 3 (q = wave + 4 j), 16
  //    lanes a row; lane ln has row r = ln / 16 and lands chunk (ln % 16) ^ swz_key(4 q + r), where
  //    swz_key(4 q + r) = kq(q) ^ kr(r) (kq: bit 0 = bit 0 of q ^ (q >> 1), bit 3 = q's bit 1;
  //    kr: bits 1 and 3 = r's bit 0, bit 2 = r's bit 1).
  //  - 128-byte rope rows: the wave's block holds rows 8 wave .. 8 wave + 7, 8 lanes a row; lane ln
  //    has row r = ln / 8 and lands chunk (ln % 8) ^ (swz_key(8 wave + r) & 7), whose three bits are
  //    r rotated left by one, bit 0 XORed with the wave's bit 0.
  constexpr bool kFastLat1K = C::LW == 1024 && C::WAVES == 4;
  constexpr bool kFastLat256 = C::LW == 256 && C::WAVES == 4;
  constexpr bool kFastRope = C::RW == 128 && C::WAVES == 4;
  const int kw = ((wave & 1) << 1) | (((wave >> 1) & 1) << 2) | ((wave & 1) << 3);
  const int r16 = lane >> 4;
  const int c16 = (lane & 15) ^ (((r16 & 1) << 1) | (((r16 >> 1) & 1) << 2) | ((r16 & 1) << 3));
  auto copy_block = [&](const StageSrc& src, char* buf, int j) __attribute__((always_inline)) {
    const unsigned lbuf = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)buf;
    if (j < C::LPW) {
      const int q = wave + 4 * j;
      if constexpr (kFastLat1K) {
        int key = kw ^ (((j ^ (j >> 1)) & 1) | (((j >> 1) & 1) << 3));
        asm volatile("" : "+s"(key));
        const int row = min(q, src.tlast);
        const unsigned voff = ((unsigned)(lane ^ key) << 4) + (unsigned)(row * C::GROW + lat_col);
        dma16_asm_at(src.rows, voff, lbuf + (unsigned)(q * 1024));
        return;
      }
      if constexpr (kFastLat256) {
        int kq = ((q ^ (q >> 1)) & 1) | (((q >> 1) & 1) << 3);
        asm volatile("" : "+s"(kq));
        const int row = min(4 * q + r16, src.tlast);
        const unsigned voff = __umul24((unsigned)row, (unsigned)C::GROW) + (unsigned)(lat_col + ((c16 ^ kq) << 4));
        dma16_asm_at(src.rows, voff, lbuf + (unsigned)(q * 1024));
        return;
      }
    } else if constexpr (kFastRope) {
      int wb = wave & 1;
      asm volatile("" : "+s"(wb));
      const int r = lane >> 3;
      const int row = min(8 * wave + r, src.tlast);
      const int c = (lane & 7) ^ (((r << 1) | (r >> 2)) & 7) ^ wb;
      const unsigned voff = __umul24((unsigned)row, (unsigned)C::GROW) + (unsigned)(C::ROPE_COL + (c << 4));
      dma16_asm_at(src.rows, voff, lbuf + (unsigned)(C::ROPE_OFF + wave * 1024));
      return;
    }
    // the general form (other row sizes): the per-lane offsets are derived from the
    // lane index afresh (the empty asm hides that they are loop invariant), so they do not hold
    // registers across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (j < C::LPW) {
      const int q = wave + C::WAVES * j;
      constexpr int CPR = C::LW / 16;
      const int t = (q * 1024) / C::LW + ln / CPR;
      const int cp = ln % CPR;
      const int c = (cp & ~C::MLS) | ((cp & C::MLS) ^ (swz_key(t) & C::MLS));
      const int tf = (q * 1024) / C::LW;
      const int tu = min(tf, src.tlast);
      unsigned voff = (unsigned)((min(t, src.tlast) - tu) * grow_bytes + lat_col + (c << 4));
      asm volatile("" : "+v"(voff));
      dma16_asm(src.rows + (size_t)tu * grow_bytes, voff, buf + q * 1024);
    } else {
      const int q = wave;
      constexpr int CPR = C::RW / 16;
      const int t = (q * 1024) / C::RW + ln / CPR;
      const int cp = ln % CPR;
      const int c = (cp & ~C::MR) | ((cp & C::MR) ^ (swz_key(t) & C::MR));
      const int tf = (q * 1024) / C::RW;
      const int tu = min(tf, src.tlast);
      unsigned voff = (unsigned)((min(t, src.tlast) - tu) * grow_bytes + C::ROPE_COL + (c << 4));
      asm volatile("" : "+v"(voff));
      dma16_asm(src.rows + (size_t)tu * grow_bytes, voff, buf + C::ROPE_OFF + q * 1024);
    }
  };
  auto issue_stage = [&](int stage0, char* buf) {
    const StageSrc src = stage_src(stage0);
#pragma unroll
    for (int j = 0; j < C::DMA_PER_WAVE; ++j) copy_block(src, buf, j);
  };

  // this lane's query fragments (B operand of S^T = K . Q^T): all latent and rope k-steps
  bf16x8_t qf[C::KS];
  {
    const size_t qrow = ((size_t)b * a.heads + head) * G + branch;
    const __bf16* qlp = static_cast<const __bf16*>(a.q_lat) + qrow * DL + h * 8;
    const __bf16* qrp = static_cast<const __bf16*>(a.q_rope) + qrow * DR + h * 8;
#pragma unroll
    for (int k = 0; k < C::KL; ++k) {
      uint4 v = *reinterpret_cast<const uint4*>(qlp + k * 16);
      if (!valid) v = make_uint4(0u, 0u, 0u, 0u);
      qf[k] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int j = 0; j < C::KR; ++j) {
      uint4 v = *reinterpret_cast<const uint4*>(qrp + j * 16);
      if (!valid) v = make_uint4(0u, 0u, 0u, 0u);
      qf[C::KL + j] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // per-lane LDS offsets (see decode.hip): S operand of k-step k is klat0 ^ 32 (k % NKL) (+ group
  // offset); rope k-step j is krope0 ^ 32 j; V^T operand of column block c is vtr0[rb] ^ 64 (c % NVT)
  const int tr = M::row_token(col);
  const int klat0 = lds_off(tr, C::LW, C::MLS, h * 16);
  const int krope0 = lds_off(tr, C::RW, C::MR, h * 16);
  int vtr0[2];
  {
    const int g16 = lane >> 4;
    const int L16 = lane & 15;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int tt = 8 * (g16 >> 1) + 4 * rb + (L16 >> 2);
      vtr0[rb] = lds_off(tt, C::LW, C::MLS, 2 * (g16 & 1) * 16 + (L16 & 3) * 8);
    }
  }
  auto s_operand = [&](const char* cur, int k, int kl, int kr) -> bf16x8_t {
    if (k < C::KL) {
      const int o = (kl ^ (32 * (k & (C::NKL - 1)))) + 32 * (k & ~(C::NKL - 1));
      return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(cur + o));
    }
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(cur + C::ROPE_OFF + (kr ^ (32 * (k - C::KL)))));
  };

  const int nstage = (t_end - t_begin + kTile - 1) / kTile;
  const float c2 = a.scale_log2;

  floatx16 acc[C::CB];
  float l_run = 0.f;     // sum of 2^(score - ref) over the unit
  float ref = 0.f;       // fixed reference of this head (log2 domain)
  float mmax = -INFINITY;  // exact max of this head's scaled scores over the unit (log2 domain)
  bool over = false;     // a stage max exceeded ref + kRefSlack
  bool fixed = false;    // second pass: ref = mmax of the first

  // The score MFMAs of one stage (36 for 576-dim rows, 12 for 192-dim ones), with the softmax work
  // `work(g)` of the previous stage placed after each group g of four; operands are read four k-steps
  // ahead through a ring of five registers (two ahead measured 2% slower: the LDS latency under the
  // stage copies exceeds two MFMAs).
  constexpr int kScoreAhead = 4, kScoreRing = 5;
  auto scores = [&](const char* cur, floatx16& S, auto&& work) __attribute__((always_inline)) {
    int kl = klat0, kr = krope0;
    asm volatile("" : "+v"(kl), "+v"(kr));
    bf16x8_t ring[kScoreRing];
#pragma unroll
    for (int k = 0; k < kScoreAhead; ++k) ring[k] = s_operand(cur, k, kl, kr);
#pragma unroll
    for (int g = 0; g < C::NGS; ++g) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 4 * g + j;
        if (k + kScoreAhead < C::KS) ring[(k + kScoreAhead) % kScoreRing] = s_operand(cur, k + kScoreAhead, kl, kr);
        S = M::mma(ring[k % kScoreRing], qf[k], k == 0 ? floatx16{} : S);
      }
      work(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // softmax of one stage's scores, in nine pieces (g = 0 .. 8: max, reference, four exp2 pieces, two
  // bf16 packs, row sum); the state it leaves: pf (P^T fragments, bf16), and l_run / ref / mmax /
  // over updated
  bf16x8_t pf[2];
  float sv[16], mt = 0.f;
  auto softmax_piece = [&](const floatx16& S, int g, bool first, bool last_stage, int stage0)
                           __attribute__((always_inline)) {
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = S[i];
      if (last_stage) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = (stage0 + M::token_of(i, h) < t_end) ? sv[i] : -INFINITY;
      }
      // maximum (NaN-propagating) is one v_maximum3_f32 per two values; fmaxf would first quieten
      // every MFMA result with an extra v_max.  A NaN score makes its head's row NaN either way.
      mt = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = __builtin_elementwise_maximum(mt, sv[i]);
    } else if (g == 1) {
      mt = fmaxf(mt, xor32(mt)) * c2;
      if (!fixed && first) ref = mt;
      mmax = fmaxf(mmax, mt);
      over |= mt > ref + kRefSlack;
    } else if (g >= 2 && g < 6) {
#pragma unroll
      for (int i = 4 * (g - 2); i < 4 * (g - 1); ++i) sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -ref));
    } else if (g == 6) {
      bf16x8_t f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (__bf16)sv[j];
      pf[0] = f;
    } else if (g == 7) {
      bf16x8_t f;
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = (__bf16)sv[8 + j];
      pf[1] = f;
    } else if (g == 8) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
      float psum = 0.f;
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pf[p2][2 * j], pf[p2][2 * j + 1]}, one2, psum, false);
      l_run += psum + xor32(psum);
    }
  };
  // the pieces that follow score group g: one each over nine groups; over three groups pieces 0-1,
  // 2-5 and 6-8
  auto softmax_group = [&](const floatx16& S, int g, bool first, bool last_stage, int stage0)
                           __attribute__((always_inline)) {
    if constexpr (C::NGS == 9) {
      softmax_piece(S, g, first, last_stage, stage0);
    } else {
      const int lo = g == 0 ? 0 : (g == 1 ? 2 : 6), hi = g == 0 ? 2 : (g == 1 ? 6 : 9);
#pragma unroll
      for (int pc = lo; pc < hi; ++pc) softmax_piece(S, pc, first, last_stage, stage0);
    }
  };

  // O^T += V^T . P^T over all column blocks, in groups of four MFMAs (`work(g)` after group g); the
  // V operands are read two MFMAs ahead
  auto pv = [&](const char* cur, auto&& work) __attribute__((always_inline)) {
    int v0 = vtr0[0], v1 = vtr0[1];
    asm volatile("" : "+v"(v0), "+v"(v1));
    auto vop = [&](int i) -> bf16x8_t {
      const int p2 = i / C::CB, c = i % C::CB;
      const int cstat = 16 * p2 * C::LW + 64 * (c & ~(C::NVT - 1));
      const int cx = 64 * (c & (C::NVT - 1));
      const bf16x4_t lo = lds_read_tr(cur + (v0 ^ cx) + cstat);
      const bf16x4_t hi = lds_read_tr(cur + (v1 ^ cx) + cstat);
      return bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    constexpr int N = 2 * C::CB;
    bf16x8_t ring[4];
    ring[0] = vop(0);
    ring[1] = vop(1);
#pragma unroll
    for (int g = 0; g < N / 4; ++g) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        if (i + 2 < N) ring[(i + 2) & 3] = vop(i + 2);
        mfma_pv(acc[i % C::CB], ring[i & 3], pf[i / C::CB]);
      }
      work(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // this wave's copies of stage n have landed (those of the later stage already issued may not)
  auto wait_stage = [&](int n) __attribute__((always_inline)) {
    if (n + 1 < nstage)
      wait_vmcnt<C::DMA_PER_WAVE>();
    else
      wait_vmcnt<0>();
  };

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
      // prologue: stages 0..2 in flight, scores of stage 0
      issue_stage(t_begin, lds_b0);
      if (nstage > 1) issue_stage(t_begin + kTile, lds_b1);
      if (nstage > 2) issue_stage(t_begin + 2 * kTile, lds_b2);
      if (nstage >= 3)
        wait_vmcnt<2 * C::DMA_PER_WAVE>();
      else if (nstage == 2)
        wait_vmcnt<C::DMA_PER_WAVE>();
      else
        wait_vmcnt<0>();
      lds_barrier();
      floatx16 SA, SB;
      scores(lds_b0, SA, [](int) {});
      // iteration n: scores of stage n+1 with the softmax of stage n between them, then P.V of n
      // the stage refilled in iteration n is n + 3: its page (index into lds_pages) and its first
      // token's offset in that page, advanced one stage per iteration (a page holds whole stages)
      int rf_pi = (t_begin + 3 * kTile) / page_size - first_page;
      int rf_off = (t_begin + 3 * kTile) % page_size;
      auto iter = [&](int n, floatx16& S, floatx16& Snext, char* cur, char* nxt, char* refill)
                      __attribute__((always_inline)) {
        const int stage0 = t_begin + n * kTile;
        const bool refill_now = n + 3 < nstage;
        const int rf_page = __builtin_amdgcn_readfirstlane(lds_pages[min(rf_pi, kUnitPages - 1)]);
        // (page ids are clamped to [0, num_pages) and a page's bytes fit in 32 bits: unsigned 32 x 32
        // -> 64-bit products, no sign extension)
        const StageSrc src{kbase + (uint64_t)(uint32_t)rf_page * (uint32_t)page_bytes +
                               (uint32_t)rf_off * (uint32_t)grow_bytes,
                           t_end - 1 - (stage0 + 3 * kTile)};
        rf_off += kTile;
        if (rf_off >= page_size) {
          rf_off = 0;
          ++rf_pi;
        }
        if (n + 1 < nstage) {
          wait_stage(n + 1);
          lds_barrier();
          // the copies of stage n + 3 are spread over the iteration (C::copy_after_score / pv)
          scores(nxt, Snext, [&](int g) {
            softmax_group(S, g, n == 0, false, stage0);
            if (refill_now && C::copy_after_score(g)) copy_block(src, refill, C::score_copy(g));
          });
        } else {
#pragma unroll
          for (int g = 0; g < C::NGS; ++g) softmax_group(S, g, n == 0, true, stage0);
        }
        pv(cur, [&](int g) __attribute__((always_inline)) {
          if (refill_now && C::copy_after_pv(g)) copy_block(src, refill, C::pv_copy(g));
        });
      };
      for (int n0 = 0; n0 < nstage; n0 += 4) {
        iter(n0, SA, SB, lds_b0, lds_b1, lds_b3);
        if (n0 + 1 < nstage) iter(n0 + 1, SB, SA, lds_b1, lds_b2, lds_b0);
        if (n0 + 2 < nstage) iter(n0 + 2, SA, SB, lds_b2, lds_b3, lds_b1);
        if (n0 + 3 < nstage) iter(n0 + 3, SB, SA, lds_b3, lds_b0, lds_b2);
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

  // ---- epilogue (the layouts of decode.hip with one wave per head block)
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_v = (ref + log2f(l_run)) * kLn2;
  if (nsplit == 1) {
    if (!valid) return;
    const size_t orow = (size_t)b * a.rows + (size_t)(qi * a.heads_per_set + head_in_set) * G + branch;
    if (h == 0) a.lse[orow] = lse_v;
#pragma unroll
    for (int k = 0; k < C::CB; ++k) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = k * 32 + 8 * g4 + 4 * h;
        const float o0 = acc[k][4 * g4 + 0] * inv_l, o1 = acc[k][4 * g4 + 1] * inv_l;
        const float o2 = acc[k][4 * g4 + 2] * inv_l, o3 = acc[k][4 * g4 + 3] * inv_l;
        if (a.out_bf16) {
          __bf16* dst = static_cast<__bf16*>(a.out) + orow * DL + c;
          *reinterpret_cast<bf16x4_t*>(dst) = bf16x4_t{(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
        } else {
          float* dst = static_cast<float*>(a.out) + orow * DL + c;
          *reinterpret_cast<float4*>(dst) = make_float4(o0, o1, o2, o3);
        }
      }
    }
  } else {
    const size_t blk = ((size_t)unit * a.groups + gs) * HB + hb;
    if (h == 0) a.part_lse[blk * 32 + col] = lse_v;
    if (a.part_bf16) {
      __bf16* dst = static_cast<__bf16*>(a.part_out) + blk * (32 * DL);
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
      float* dst = static_cast<float*>(a.part_out) + blk * (32 * DL);
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

}  // namespace

// The pipelined kernel serves bf16 latent caches whose query set is 128 heads over one latent slice
// and the rope key: absorbed MLA (one 512-dim slice) and MLRA (one work group per 128-dim branch, four
// branches or one branch of a tensor-parallel share).  Launchers return hipError_t, or -1 when the
// shape is not the kernel's.
namespace {

template <int DL, int G, int MINB>
int run_pipe(const DecodeArgs& a, void* stream) {
  const int units8 = (a.max_units + 7) / 8 * 8;
  hipLaunchKernelGGL((decode_pipe_kernel<DL, 64, 4, G, MINB>), dim3(units8 * a.wg_per_unit), dim3(4 * kWaveSize), 0,
                     static_cast<hipStream_t>(stream), a, a.block_table);
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode_pipe(const ld_problem& p, const DecodeArgs& a, void* stream) {
  if (!decode_pipe_serves(p, a.nsets, a.hblocks)) return -1;
  if (p.variant == LD_VARIANT_MLA) return run_pipe<512, 1, 1>(a, stream);
  return p.num_groups == 4 ? run_pipe<128, 4, 2>(a, stream) : run_pipe<128, 1, 2>(a, stream);
}

bool decode_pipe_serves(const ld_problem& p, int nsets, int hblocks) {
  if (p.kv_dtype != LD_BF16 || p.q_dtype != LD_BF16 || p.d_rope != 64 || nsets != 1 || hblocks != 4) return false;
  if (p.variant == LD_VARIANT_MLA) return p.d_latent == 512;
  return p.variant == LD_VARIANT_MLRA && p.d_latent == 128 && (p.num_groups == 4 || p.num_groups == 1);
}

int decode_pipe_wgs_per_cu(const ld_problem& p) {
  static int cache[3][kMaxDevices] = {};
  if (p.variant == LD_VARIANT_MLA)
    return occupancy_cached(cache[0], reinterpret_cast<const void*>(decode_pipe_kernel<512, 64, 4, 1, 1>),
                            4 * kWaveSize);
  if (p.num_groups == 4)
    return occupancy_cached(cache[1], reinterpret_cast<const void*>(decode_pipe_kernel<128, 64, 4, 4, 2>),
                            4 * kWaveSize);
  return occupancy_cached(cache[2], reinterpret_cast<const void*>(decode_pipe_kernel<128, 64, 4, 1, 2>),
                          4 * kWaveSize);
}

}  // namespace ld
