// Decode-attention kernels for gfx950 (CDNA4): one query token per sequence against a paged,
// shrunk KV cache.  See include/latent_decode.h for the operation and its sources.
//
// Work decomposition.  A work unit is (sequence b, token chunk [t_begin, t_end)) from the
// split-KV planner.  A "set" is a group of query heads that score against the same cached
// rows: all H heads for MLA, one latent group for GLA, one branch for MLRA, one kv head for
// GQA/GTA, all heads for MQA.  A work group handles NSETS sets of one unit, HB blocks of 32
// heads per set and SPLIT waves per head block.  Per 32-token stage the work group copies the
// rows it needs into LDS once (asynchronous global->LDS DMA into one of NBUF stage buffers, so
// later stages stream in while one is computed), and every wave reads them from there:
//
//   S^T[token, head] = K_stage . Q^T           (v_mfma_f32_32x32x16_bf16; Q stays in VGPRs)
//   online softmax over the token axis         (each lane owns one head: 16 scores here and
//                                               16 in the lane 32 apart)
//   O^T[col, head]  += V_stage^T . P^T          (same MFMA; P never leaves registers; the V^T
//                                               operand comes from ds_read_b64_tr_b16)
//
// With SPLIT = 2 the two waves of a head block share its work: each scores over half of the
// latent dims and half of the rope dims, the pair adds its two partial scores through LDS
// (floating-point addition commutes, so both waves hold bit-identical scores and run the same
// softmax), and each wave then accumulates half of the V columns.  A wave so holds half the
// query and accumulator registers (for MLA 72 + 128 instead of 144 + 256), two waves fit on a
// SIMD, and each hides the other's LDS latency.
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

#include "decode_common.h"
#include "plan_common.h"
#include "ld_internal.h"

namespace ld {
namespace {

// ------------------------------------------------------------------------------------------
// compile-time shape of one kernel instance
// ------------------------------------------------------------------------------------------
template <int KV, int DL, int DR, int KIND, int NSETS, int HB, int SPLIT>
struct Cfg {
  using M = Mma<KV>;
  using CT = typename M::CT;
  static constexpr int ES = sizeof(CT);                       // LDS element bytes (fp8 staged as bf16)
  static constexpr int GES = (KV == KV_FP8) ? 1 : ES;         // global latent element bytes
  static constexpr int WAVES = NSETS * HB * SPLIT;
  static constexpr int THREADS = WAVES * kWaveSize;
  static constexpr int KL = DL / M::KSTEP;                    // latent (K) k-steps of S
  static constexpr int KR = DR / M::KSTEP;                    // rope k-steps of S
  static constexpr int KLW = KL / SPLIT, KRW = KR / SPLIT;    // k-steps per wave
  static constexpr int CB = DL / 32;                          // 32-column blocks of O
  static constexpr int CBW = CB / SPLIT;                      // column blocks per wave
  static constexpr int LW = NSETS * DL * ES;                  // latent / K row bytes in LDS
  static constexpr int RW = DR * ES;                          // rope row bytes in LDS
  static constexpr int VW = (KIND == KIND_SHARED) ? NSETS * DL * ES : 0;
  // swizzle masks; a set's slice of a row starts on a swizzle-group boundary
  static constexpr int SETCH = DL * ES / 16;                  // chunks per set slice
  static constexpr int MLS = cmin(SETCH - 1, swz_mask(LW));
  static constexpr int MR = swz_mask(RW > 0 ? RW : 32);
  static constexpr int MV = (KIND == KIND_SHARED) ? cmin(SETCH - 1, swz_mask(VW > 0 ? VW : 32)) : MLS;
  static constexpr int LAT_OFF = 0;
  static constexpr int ROPE_OFF = kTile * LW;
  static constexpr int V_OFF = ROPE_OFF + kTile * RW;
  static constexpr int SC_OFF = V_OFF + kTile * VW;
  static constexpr int BUF = SC_OFF + ((KV == KV_FP8) ? kTile * 4 : 0);
  static constexpr int BUF_AL = (BUF + 127) / 128 * 128;
  static constexpr int EXCH = (SPLIT == 2) ? WAVES * 16 * 64 * 4 : 16;   // partial-score exchange
  // stage buffers: as many as fit (up to 4); the fp8 path stages through registers and keeps two
  static constexpr int NB_FIT = (160 * 1024 - EXCH - 4 * kUnitPages) / BUF_AL;
  static constexpr int NBUF = (KV == KV_FP8) ? 2 : cmin(NB_FIT, 4);
  static constexpr int LDS_TOTAL =
      2 * BUF_AL + (NBUF > 2 ? BUF_AL : 128) + (NBUF > 3 ? BUF_AL : 128) + EXCH + 4 * kUnitPages;
  static constexpr int VRB = (KIND == KIND_SHARED) ? VW : LW;   // row bytes of the V source region
  static constexpr int V_REG = (KIND == KIND_SHARED) ? V_OFF : LAT_OFF;
  static constexpr int FP8_ITEMS = kTile * NSETS * DL / 16;      // 16-code pieces of an fp8 stage
  static constexpr int FP8_PER_THREAD = (KV == KV_FP8) ? (FP8_ITEMS + THREADS - 1) / THREADS : 1;
  // 1 KB DMA blocks per stage (all regions) and the fewest any wave issues per stage
  static constexpr int DMA_BLOCKS = (KV == KV_FP8) ? kTile * RW / 1024 : kTile * (LW + RW + VW) / 1024;
  static constexpr bool PP = (WAVES == 8) && (KV != KV_FP8);     // see the stage loop
  static constexpr int DMA_WAVES = PP ? WAVES / 2 : WAVES;         // waves that issue copies
  static constexpr int DMA_MIN_PER_WAVE = DMA_BLOCKS / DMA_WAVES;
  static_assert(DL % 32 == 0 && DL % M::KSTEP == 0 && DR % M::KSTEP == 0, "unsupported dims");
  static_assert(KL % SPLIT == 0 && KR % SPLIT == 0 && CB % SPLIT == 0, "dims must split evenly");
  static_assert(SPLIT == 1 || M::EPL == 8, "split waves need the bf16 operand path");
  // a wave's latent k-steps and column blocks must start on swizzle-group boundaries
  static_assert(SPLIT == 1 || ((2 * KLW) % (MLS + 1) == 0 && (4 * CBW) % (MV + 1) == 0), "split alignment");
  static_assert(SETCH % (MLS + 1) == 0, "set alignment");
  static_assert(pow2(LW) && LW >= 32 && (DR == 0 || (pow2(RW) && RW >= 32)), "row sizes must be powers of two");
  static_assert((kTile * LW) % 1024 == 0 && (kTile * RW) % 1024 == 0, "regions must be whole DMA blocks");
  static_assert(NBUF >= 2 && LDS_TOTAL <= 160 * 1024, "LDS budget");
};

// ------------------------------------------------------------------------------------------
// the decode kernel
// ------------------------------------------------------------------------------------------
// ------------------------------------------------------------------------------------------
template <int KV, int DL, int DR, int KIND, int NSETS, int HB, int SPLIT>
__global__ __launch_bounds__(NSETS* HB* SPLIT * 64) void decode_kernel(DecodeArgs a,
                                                                       const int32_t* __restrict__ block_table) {
  using C = Cfg<KV, DL, DR, KIND, NSETS, HB, SPLIT>;
  using M = typename C::M;
  using CT = typename C::CT;
  using Frag = typename M::Frag;
  constexpr int ES = C::ES;
  constexpr int WAVES = C::WAVES;
  // Stage buffers are separate LDS objects (and the stage loop is unrolled over them) so that
  // the compiler's alias scopes tell the buffers apart: a read of stage n then waits only for
  // the copies into stage n's buffer, not for every copy in flight.
  __shared__ __attribute__((aligned(128))) char lds_b0[C::BUF_AL];
  __shared__ __attribute__((aligned(128))) char lds_b1[C::BUF_AL];
  __shared__ __attribute__((aligned(128))) char lds_b2[C::NBUF > 2 ? C::BUF_AL : 128];
  __shared__ __attribute__((aligned(128))) char lds_b3[C::NBUF > 3 ? C::BUF_AL : 128];
  __shared__ __attribute__((aligned(16))) float lds_exch[C::EXCH / 4];
  __shared__ int lds_pages[kUnitPages];

  // XCD-aware mapping: work groups are dealt to the 8 XCDs round-robin, so blockIdx mod 8 names
  // the XCD.  All work groups of one unit land on one XCD, and XCD k takes the consecutive units
  // [k*per, (k+1)*per): the splits of one sequence share an L2, which fetches its query once.
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int y = x >> 3;
  const int sb = y % a.wg_per_unit;
  const int yy = y / a.wg_per_unit;
  int unit, b, t_begin, t_end, nsplit;
  if (a.fused_plan) {
    __shared__ int s_unit[5];
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

  // Work group sb of a unit serves query token qi = sb / wpt and the cache sets (latent slices /
  // kv heads) [lset0, lset0 + NSETS); its query rows form the sets qi * cache_groups + lset0 + s.
  // Token qi (of qlen) sees the first L_b - qlen + 1 + qi cache rows.
  const int wpt = a.wg_per_unit / a.qlen;  // work groups per query token
  const int qi = sb / wpt;
  const int lset0 = (sb - qi * wpt) * NSETS;
  const int set0 = qi * a.cache_groups + lset0;
  const int G = a.groups;
  if (a.qlen > 1) {
    const int Lb = clampi(a.seq_lens[b], 0, a.max_pages * a.page_size);
    t_end = max(t_begin, min(t_end, Lb - a.qlen + 1 + qi));
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, kept in an SGPR
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int s = wave / (HB * SPLIT);  // wave-uniform: set, head block, half
  const int hb = (wave / SPLIT) % HB;
  const int half = wave % SPLIT;
  const int gs = set0 + s;
  const int head_in_set = hb * 32 + col;
  const bool valid = head_in_set < a.heads_per_set;
  // query row of this lane: set gs * heads_per_set + head; MLRA: (token, head, branch), branch innermost
  const int CGr = a.cache_groups;
  const int head = (a.mlra ? qi : gs) * a.heads_per_set + (valid ? head_in_set : 0);
  const int row = a.mlra ? head * CGr + (gs - qi * CGr) : head;
  const int32_t* __restrict__ bt_row = block_table + (size_t)b * a.max_pages;
  const int page_size = a.page_size;
  // The unit's block-table entries (at most kUnitPages) are staged in LDS up front, so that issuing
  // a stage's copies waits for an LDS read rather than for a dependent scalar load from memory.
  const int first_page = t_begin / page_size;
  const int unit_pages = t_end > t_begin ? (t_end - 1) / page_size - first_page + 1 : 0;
  for (int i = threadIdx.x; i < unit_pages && i < kUnitPages; i += C::THREADS)
    lds_pages[i] = clampi(bt_row[first_page + i], 0, a.num_pages - 1);
  __syncthreads();

  // global row geometry (bytes): latent variants store [G latents | rope] per token (fp8: codes
  // only, the rope key lives in its own pool); GQA/MQA/GTA store [G kv heads][DL] per token
  const int CG = a.cache_groups;
  const int grow_bytes = (KIND == KIND_LATENT) ? (CG * DL * C::GES + (KV == KV_FP8 ? 0 : DR * ES)) : CG * DL * ES;
  const char* kbase = static_cast<const char*>(a.k);

  // ---- issue the copies of one stage into buffer `buf`
  uint4 pre[C::FP8_PER_THREAD];
  float pre_sc = 0.f;
  auto issue_stage = [&](int stage0, char* buf) {
    // every token of a stage lies in one page (stages are page aligned and page_size % 32 == 0)
    const int pi = stage0 / page_size - first_page;
    // a unit spans at most kUnitPages pages (planner rule); the clamp only keeps the read in bounds
    const int page = __builtin_amdgcn_readfirstlane(lds_pages[min(pi, kUnitPages - 1)]);
    const size_t r0 = (size_t)page * page_size + (stage0 % page_size);
    const int tlast = t_end - 1 - stage0;  // rows past the unit's end repeat its last row
    const char* krows = kbase + r0 * (size_t)grow_bytes;
    if constexpr (KV != KV_FP8) {
      dma_region<C::LW, C::MLS, C::DMA_WAVES, 0>(buf + C::LAT_OFF, wave, lane, krows, grow_bytes, tlast, [&](int cb) {
        const int s2 = cb / (DL * ES);
        return (lset0 + s2) * DL * ES + (cb - s2 * DL * ES);
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
                                                   (size_t)(lset0 + s2) * DL + w);
        }
      }
      if (threadIdx.x < kTile) pre_sc = a.kscale[r0 + min((int)threadIdx.x, tlast)];
    }
    if constexpr (KIND == KIND_LATENT && DR > 0) {
      if constexpr (KV == KV_FP8) {
        const char* rrows = static_cast<const char*>(a.rope) + r0 * (size_t)(DR * 2);
        dma_region<C::RW, C::MR, C::DMA_WAVES, 0>(buf + C::ROPE_OFF, wave, lane, rrows, DR * 2, tlast,
                                                  [&](int cb) { return cb; });
      } else {
        dma_region<C::RW, C::MR, C::DMA_WAVES, kTile * C::LW / 1024>(buf + C::ROPE_OFF, wave, lane, krows, grow_bytes,
                                                                     tlast, [&](int cb) { return CG * DL * ES + cb; });
      }
    }
    if constexpr (KIND == KIND_SHARED) {
      const char* vrows = static_cast<const char*>(a.v) + r0 * (size_t)grow_bytes;
      dma_region<C::VW, C::MV, C::DMA_WAVES, kTile *(C::LW + C::RW) / 1024>(
          buf + C::V_OFF, wave, lane, vrows, grow_bytes, tlast, [&](int cb) {
            const int s2 = cb / (DL * ES);
            return (lset0 + s2) * DL * ES + (cb - s2 * DL * ES);
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
          *reinterpret_cast<uint4*>(rowp + lds_off(t, C::LW, C::MLS, k16 * 32)) = e4m3x8_to_bf16x8(pre[r].x, pre[r].y);
          *reinterpret_cast<uint4*>(rowp + lds_off(t, C::LW, C::MLS, k16 * 32 + 16)) =
              e4m3x8_to_bf16x8(pre[r].z, pre[r].w);
        }
      }
      if (threadIdx.x < kTile) reinterpret_cast<float*>(buf + C::SC_OFF)[threadIdx.x] = pre_sc;
    }
    (void)buf;
  };

  // ---- this lane's query fragments (B operand of S^T = K . Q^T) for the wave's k-steps:
  // latent k-steps [half*KLW, +KLW) and rope k-steps [half*KRW, +KRW).  The loads are issued
  // without branches (lanes past the set's heads read head 0 and are zeroed).
  Frag ql[C::KLW];
  Frag qr[C::KRW > 0 ? C::KRW : 1];
  {
    const size_t qrow = a.mlra ? ((size_t)b * a.heads + head) * CGr + (gs - qi * CGr) : (size_t)b * a.heads + head;
    const CT* qlp = static_cast<const CT*>(a.q_lat) + qrow * DL + half * C::KLW * M::KSTEP + h * M::EPL;
    const CT* qrp = static_cast<const CT*>(a.q_rope) + qrow * DR + half * C::KRW * M::KSTEP + h * M::EPL;
    if constexpr (M::EPL == 8) {
#pragma unroll
      for (int k = 0; k < C::KLW; ++k) {
        uint4 v = *reinterpret_cast<const uint4*>(qlp + k * M::KSTEP);
        if (!valid) v = make_uint4(0u, 0u, 0u, 0u);
        ql[k] = __builtin_bit_cast(Frag, v);
      }
#pragma unroll
      for (int j = 0; j < C::KRW; ++j) {
        uint4 v = *reinterpret_cast<const uint4*>(qrp + j * M::KSTEP);
        if (!valid) v = make_uint4(0u, 0u, 0u, 0u);
        qr[j] = __builtin_bit_cast(Frag, v);
      }
    } else {
#pragma unroll
      for (int k = 0; k < C::KLW; ++k) {
        const float v = qlp[k * M::KSTEP];
        ql[k] = valid ? v : 0.f;
      }
#pragma unroll
      for (int j = 0; j < C::KRW; ++j) {
        const float v = qrp[j * M::KSTEP];
        qr[j] = valid ? v : 0.f;
      }
    }
  }

  floatx16 acc[C::CBW];
#pragma unroll
  for (int k = 0; k < C::CBW; ++k) acc[k] = floatx16{};
  float m_run = -INFINITY;  // running (possibly stale, see kRescaleSlack) max of this head's log2 scores
  float l_run = 0.f;        // running sum of 2^(score - m_run)

  const int tr = M::row_token(col);  // stage token this lane's S row stands for

  // Per-lane LDS byte offsets (bf16 path).  Each is the offset of this lane's first operand;
  // the others follow by XOR with a constant, because the swizzle XORs the low chunk bits and
  // the operands of consecutive k-steps (column blocks) differ only in those bits.
  //   S operand, latent: chunk 2k + h of the wave's slice of row tr  -> klat0 ^ 32 (k % NKL)
  //   S operand, rope:   chunk 2(half*KRW + j) + h of row tr          -> krope0 ^ 32 j
  //   V^T operand: lane group g = lane/16 serves columns 16*(g%2) + (lane%16) of a 32-column
  //   block and tokens 8*(g/2) + 4*rb + [0, 4) of a 16-token k-step; its source lane
  //   L = lane%16 loads columns 4*(L%4) .. +3 of token 8*(g/2) + 4*rb + L/4  -> vtr0[rb] ^ 64 (c % NVT)
  constexpr int NKL = (C::MLS + 1) / 2 > 0 ? (C::MLS + 1) / 2 : 1;
  constexpr int NVT = (C::MV >> 2) + 1;
  static_assert(M::EPL != 8 || DR == 0 || 2 * C::KR <= C::MR + 1, "rope row must lie in one swizzle group");
  const int lat_base = s * DL * ES + half * C::KLW * M::KSTEP * ES;  // wave's first latent byte in a row
  const int v_base = s * DL * ES + half * C::CBW * 32 * ES;          // wave's first V column byte in a row
  int klat0 = 0, krope0 = 0, vtr0[2] = {0, 0};
  if constexpr (M::EPL == 8) {
    klat0 = lat_base + lds_off(tr, C::LW, C::MLS, h * 16);
    if constexpr (DR > 0) krope0 = lds_off(tr, C::RW, C::MR, (2 * half * C::KRW + h) * 16);
    const int g16 = lane >> 4;
    const int L16 = lane & 15;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int tt = 8 * (g16 >> 1) + 4 * rb + (L16 >> 2);
      vtr0[rb] = v_base + lds_off(tt, C::VRB, C::MV, 2 * (g16 & 1) * 16 + (L16 & 3) * 8);
    }
  }

  // ---- prologue: the first NBUF-1 stages
  constexpr int NB = C::NBUF;
  const int nstage = (t_end - t_begin + kTile - 1) / kTile;
  char* const bufs[4] = {lds_b0, lds_b1, lds_b2, lds_b3};
  // with the half-stage offset (see the stage loop) only the early half of the waves copies
  const bool late = C::PP && wave >= WAVES / 2;  // wave-uniform
  if (!late) {
#pragma unroll
    for (int n = 0; n < NB - 1; ++n)
      if (n < nstage) issue_stage(t_begin + n * kTile, bufs[n]);
  }
  finish_stage(bufs[0]);

  // The work on a stage has two parts.  part_s: this wave's (partial) scores, into sp; with
  // SPLIT = 2 they are posted for the partner wave.  part_pv: (the partner's half added) the online
  // softmax and O += P.V.  A barrier separates the two parts of a stage.
  float sp[16];
  auto part_s = [&](char* const cur) __attribute__((always_inline)) {
    // ---- S^T over this wave's k-steps: rows = stage tokens (permuted), columns = 32 heads
    floatx16 sl = floatx16{};
    floatx16 sr = floatx16{};
    if constexpr (M::EPL == 8) {
      // the offsets are re-derived inside every stage (the empty asm hides that they are loop
      // invariant), so the compiler does not keep one register per operand address
      int kl = klat0, kr = krope0;
      asm volatile("" : "+v"(kl), "+v"(kr));
#pragma unroll
      for (int k = 0; k < C::KLW; ++k) {
        const int o = (kl ^ (32 * (k & (NKL - 1)))) + 32 * (k & ~(NKL - 1));
        const Frag af = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(cur + C::LAT_OFF + o));
        sl = M::mma(af, ql[k], sl);
        if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the operand reads in flight
      }
#pragma unroll
      for (int j = 0; j < C::KRW; ++j) {
        const Frag af = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(cur + C::ROPE_OFF + (kr ^ (32 * j))));
        if constexpr (KV == KV_FP8)
          sr = M::mma(af, qr[j], sr);
        else
          sl = M::mma(af, qr[j], sl);
      }
    } else {
#pragma unroll
      for (int k = 0; k < C::KLW; ++k) {
        const float af = *reinterpret_cast<const float*>(cur + C::LAT_OFF +
                                                         lds_off(tr, C::LW, C::MLS, (s * DL + k * M::KSTEP + h) * ES));
        sl = M::mma(af, ql[k], sl);
        if ((k & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < C::KRW; ++j) {
        const float af = *reinterpret_cast<const float*>(cur + C::ROPE_OFF +
                                                         lds_off(tr, C::RW, C::MR, (j * M::KSTEP + h) * ES));
        sl = M::mma(af, qr[j], sl);
      }
    }

    float tok_scale[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      tok_scale[i] = (KV == KV_FP8) ? reinterpret_cast<const float*>(cur + C::SC_OFF)[M::token_of(i, h)] : 1.f;
    // fp8: the per-token scale multiplies the latent part of the score only
#pragma unroll
    for (int i = 0; i < 16; ++i) sp[i] = (KV == KV_FP8) ? tok_scale[i] * sl[i] + sr[i] : sl[i];

    if constexpr (SPLIT == 2) {
      // post this wave's partial scores (lane-contiguous 16-byte pieces) for the partner
      floatx4* mine = reinterpret_cast<floatx4*>(lds_exch + (wave >> 1) * (2 * 16 * 64) + half * 16 * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) mine[j * 64 + lane] = floatx4{sp[4 * j], sp[4 * j + 1], sp[4 * j + 2], sp[4 * j + 3]};
    }
  };
  auto part_pv = [&](const int n, char* const cur) __attribute__((always_inline)) {
    const int stage0 = t_begin + n * kTile;
    if constexpr (SPLIT == 2) {
      // add the partner's partial scores (posted before the barrier that precedes this part)
      const floatx4* other =
          reinterpret_cast<const floatx4*>(lds_exch + (wave >> 1) * (2 * 16 * 64) + (1 - half) * 16 * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 o = other[j * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[4 * j + e] += o[e];
      }
    }
    float tok_scale[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      tok_scale[i] = (KV == KV_FP8) ? reinterpret_cast<const float*>(cur + C::SC_OFF)[M::token_of(i, h)] : 1.f;

    // ---- online softmax (log2 domain) over this lane's 16 tokens and its partner lane's 16.
    // Rows past the unit's end exist only in its last stage.  The scale is positive, so the max
    // is taken over the raw scores and each exponent is one fma.
    if (stage0 + kTile > t_end) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sp[i] = (stage0 + M::token_of(i, h) < t_end) ? sp[i] : -INFINITY;
    }
    float mt = sp[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sp[i]);
    mt = fmaxf(mt, xor32(mt)) * a.scale_log2;
    // raise the running max only when this stage's max exceeds it by more than the slack
    const bool raise = mt > m_run + kRescaleSlack;
    const float m_new = raise ? mt : m_run;
    const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 on the first stage
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float sv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[i], a.scale_log2, -m_use));
    if (n > 0 && __any(alpha != 1.f)) {  // rare; O is still zero on the first stage
#pragma unroll
      for (int k = 0; k < C::CBW; ++k) acc[k] *= alpha;
    }

    // ---- P^T fragments (B operand of the PV MFMA) and the stage's row sum.  bf16: the sum is
    // taken over the rounded P the PV product uses; fp8 folds the token scale into P (it scales
    // V) and sums the unscaled probabilities.
    Frag pf[M::PSTEPS];
    float psum = 0.f;
    if constexpr (M::EPL == 8) {
#pragma unroll
      for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
        bf16x8_t f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = (__bf16)(sv[8 * p2 + j] * tok_scale[8 * p2 + j]);
        pf[p2] = f;
      }
      if constexpr (KV == KV_FP8) {
#pragma unroll
        for (int i = 0; i < 16; ++i) psum += sv[i];
      } else {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int p2 = 0; p2 < M::PSTEPS; ++p2)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pf[p2][2 * j], pf[p2][2 * j + 1]}, one2, psum, false);
      }
    } else {
#pragma unroll
      for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
        pf[p2] = sv[p2];
        psum += sv[p2];
      }
    }
    psum += xor32(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;

    // ---- O^T += V^T . P^T over this wave's column blocks
    if constexpr (M::EPL == 8) {
      int v0 = vtr0[0], v1 = vtr0[1];
      asm volatile("" : "+v"(v0), "+v"(v1));
      const char* vs = cur + C::V_REG;
#pragma unroll
      for (int k = 0; k < C::CBW; ++k) {
#pragma unroll
        for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
          const int cstat = 16 * p2 * C::VRB + 64 * (k & ~(NVT - 1));
          const int cx = 64 * (k & (NVT - 1));
          const bf16x4_t lo = lds_read_tr(vs + (v0 ^ cx) + cstat);
          const bf16x4_t hi = lds_read_tr(vs + (v1 ^ cx) + cstat);
          acc[k] = M::mma(bf16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, pf[p2], acc[k]);
        }
        if (k & 1) __builtin_amdgcn_sched_barrier(0);  // bound the operand reads in flight
      }
    } else {
      const char* vsrc = cur + C::V_REG;
#pragma unroll
      for (int k = 0; k < C::CBW; ++k) {
#pragma unroll
        for (int p2 = 0; p2 < M::PSTEPS; ++p2) {
          const int tt = 2 * p2 + h;
          const Frag af =
              *reinterpret_cast<const float*>(vsrc + lds_off(tt, C::VRB, C::MV, (s * DL + k * 32 + col) * ES));
          acc[k] = M::mma(af, pf[p2], acc[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // With eight waves (two per SIMD) the two halves of the work group run half a stage apart, so
  // that on every SIMD one wave's score MFMAs overlap the other wave's softmax and P.V.  Every
  // wave runs the same program (barrier, part_s(n), barrier, part_pv(n) per stage); the late half
  // passes one extra barrier first, the early half one extra barrier last, so with barriers
  // counted across the work group the early half computes part_s(n) after barrier 2n and
  // part_pv(n) after 2n+1, the late half one barrier later.  Only the early half issues the
  // copies: it waits for its copies of stage n before barrier 2n (the first read of stage n comes
  // after it), and refills stage n-1's buffer after barrier 2n+1 (its last read, the late half's
  // part_pv(n-1), comes before it).  Without the offset (fewer waves, or the fp8 cache, which is
  // staged through registers) every wave copies and the refill follows the first barrier.
  constexpr bool PP = C::PP;
  auto wait_stage = [&](const int n) __attribute__((always_inline)) {
    // this wave's copies of stage n have landed; those of the (up to NB-2) later stages already
    // issued may stay in flight
    if constexpr (KV == KV_FP8) {
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      const int later = min(nstage - 1 - n, NB - 2);
      if (later >= 2 && NB >= 4)
        wait_vmcnt<2 * C::DMA_MIN_PER_WAVE>();
      else if (later >= 1 && NB >= 3)
        wait_vmcnt<C::DMA_MIN_PER_WAVE>();
      else
        wait_vmcnt<0>();
    }
  };
  auto iter = [&](const int n, char* const cur, char* const refill, char* const nxt) __attribute__((always_inline)) {
    if (!late) wait_stage(n);
    lds_barrier();
    if (!PP && n + NB - 1 < nstage) issue_stage(t_begin + (n + NB - 1) * kTile, refill);
    part_s(cur);
    if constexpr (PP || SPLIT == 2) lds_barrier();
    if (PP && !late && n + NB - 1 < nstage) issue_stage(t_begin + (n + NB - 1) * kTile, refill);
    part_pv(n, cur);
    if (n + 1 < nstage) finish_stage(nxt);
  };

  if (late) lds_barrier();
  // unrolled over the stage buffers, so that every LDS access names its buffer statically
  for (int n0 = 0; n0 < nstage; n0 += NB) {
    iter(n0, bufs[0], bufs[NB - 1], bufs[1 % NB]);
    if (n0 + 1 < nstage) iter(n0 + 1, bufs[1 % NB], bufs[0], bufs[2 % NB]);
    if constexpr (NB > 2)
      if (n0 + 2 < nstage) iter(n0 + 2, bufs[2 % NB], bufs[1], bufs[3 % NB]);
    if constexpr (NB > 3)
      if (n0 + 3 < nstage) iter(n0 + 3, bufs[3 % NB], bufs[2], bufs[4 % NB]);
  }
  if (PP && !late) lds_barrier();

  // ---- epilogue: normalise; final output for unsplit sequences, partials otherwise.  A unit
  // with no tokens (an empty sequence) has l = 0 and gives out = 0, lse = -inf.
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_v = (m_run + log2f(l_run)) * kLn2;
  if (nsplit == 1) {
    if (!valid) return;
    const size_t orow = (size_t)b * a.rows + row;
    if (h == 0 && half == 0) a.lse[orow] = lse_v;
#pragma unroll
    for (int k = 0; k < C::CBW; ++k) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int c = (half * C::CBW + k) * 32 + 8 * g4 + 4 * h;
        const float o0 = acc[k][4 * g4 + 0] * inv_l, o1 = acc[k][4 * g4 + 1] * inv_l;
        const float o2 = acc[k][4 * g4 + 2] * inv_l, o3 = acc[k][4 * g4 + 3] * inv_l;
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
    // Partials in fragment order: slot block (unit, set, head block) holds 32 heads x DL values
    // as [column block][piece][lane][value], a piece being 8 (bf16) or 4 (f32) consecutive
    // accumulator registers, so every store instruction writes 1 KB contiguous.  All lanes
    // store (those past the set's heads hold finite values the combine ignores).
    const size_t blk = ((size_t)unit * G + gs) * HB + hb;
    if (h == 0 && half == 0) a.part_lse[blk * 32 + col] = lse_v;
    if (a.part_bf16) {
      __bf16* dst = static_cast<__bf16*>(a.part_out) + blk * (32 * DL);
#pragma unroll
      for (int k = 0; k < C::CBW; ++k)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x8_t v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (__bf16)(acc[k][8 * j + e] * inv_l);
          *reinterpret_cast<bf16x8_t*>(dst + (((half * C::CBW + k) * 2 + j) * 64 + lane) * 8) = v;
        }
    } else {
      float* dst = static_cast<float*>(a.part_out) + blk * (32 * DL);
#pragma unroll
      for (int k = 0; k < C::CBW; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(dst + (((half * C::CBW + k) * 4 + j) * 64 + lane) * 4) =
              make_float4(acc[k][4 * j] * inv_l, acc[k][4 * j + 1] * inv_l, acc[k][4 * j + 2] * inv_l,
                          acc[k][4 * j + 3] * inv_l);
    }
  }
}

template <int KV, int DL, int DR, int KIND, int NSETS, int HB, int SPLIT>
int run(const DecodeArgs& a, void* stream) {
  if (a.nsets != NSETS || a.hblocks != HB) return -1;
  auto fn = decode_kernel<KV, DL, DR, KIND, NSETS, HB, SPLIT>;
  const int units8 = (a.max_units + 7) / 8 * 8;
  const dim3 grid(units8 * a.wg_per_unit);
  hipLaunchKernelGGL(fn, grid, dim3(NSETS * HB * SPLIT * kWaveSize), 0, static_cast<hipStream_t>(stream), a,
                     a.block_table);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// the instantiated shapes: (kv dtype, d_latent, d_rope, kind, sets per work group, 32-head
// blocks per set, waves per head block)
// ------------------------------------------------------------------------------------------
#define LD_SHAPES(X)                                                                          \
  /* MLA: 128 / 64 heads */                                                                   \
  X(KV_BF16, 512, 64, KIND_LATENT, 1, 4, 2) X(KV_BF16, 512, 64, KIND_LATENT, 1, 2, 2)          \
  X(KV_FP8, 512, 64, KIND_LATENT, 1, 4, 2)                                                    \
  /* GLA-2 (2 groups x 64 heads), GLA-4 (4 groups x 32 heads), one group of 128 heads */      \
  X(KV_BF16, 256, 64, KIND_LATENT, 2, 2, 2) X(KV_BF16, 256, 64, KIND_LATENT, 4, 1, 1)          \
  X(KV_BF16, 256, 64, KIND_LATENT, 1, 4, 2) X(KV_FP8, 256, 64, KIND_LATENT, 2, 2, 2)           \
  X(KV_FP8, 256, 64, KIND_LATENT, 4, 1, 1) X(KV_FP8, 256, 64, KIND_LATENT, 1, 4, 2)            \
  /* one GLA group of 64 heads (a tensor-parallel share) */                                   \
  X(KV_BF16, 256, 64, KIND_LATENT, 1, 2, 2) X(KV_FP8, 256, 64, KIND_LATENT, 1, 2, 2)            \
  /* MLRA, two branches or one of 128 heads per work group (bf16 with 4 or 1 branches: pipe) */\
  X(KV_BF16, 128, 64, KIND_LATENT, 2, 4, 1) X(KV_BF16, 128, 64, KIND_LATENT, 1, 4, 1)          \
  X(KV_FP8, 128, 64, KIND_LATENT, 2, 4, 1) X(KV_FP8, 128, 64, KIND_LATENT, 1, 4, 1)            \
  /* small latent shapes: up to 32 heads per set */                                           \
  X(KV_F32, 64, 16, KIND_LATENT, 1, 1, 1) X(KV_F32, 64, 16, KIND_LATENT, 2, 1, 1)              \
  X(KV_F32, 64, 16, KIND_LATENT, 4, 1, 1) X(KV_BF16, 64, 16, KIND_LATENT, 1, 1, 1)             \
  X(KV_BF16, 64, 16, KIND_LATENT, 2, 1, 1) X(KV_BF16, 64, 16, KIND_LATENT, 4, 1, 1)            \
  X(KV_FP8, 64, 16, KIND_LATENT, 1, 1, 1) X(KV_FP8, 64, 16, KIND_LATENT, 2, 1, 1)              \
  X(KV_FP8, 64, 16, KIND_LATENT, 4, 1, 1)                                                      \
  /* GQA: 4 kv heads (K and V) per work group; GTA: 8; MQA: one kv head of 64 or 32 heads */  \
  X(KV_BF16, 128, 0, KIND_SHARED, 4, 1, 1) X(KV_BF16, 128, 0, KIND_SHARED, 2, 1, 1)            \
  X(KV_BF16, 128, 0, KIND_SHARED, 1, 2, 1) X(KV_BF16, 128, 0, KIND_SHARED, 1, 1, 1)            \
  /* MQA with large head dims (MFA-style single kv head): 256 and 512 */                      \
  X(KV_BF16, 256, 0, KIND_SHARED, 1, 2, 1) X(KV_BF16, 256, 0, KIND_SHARED, 1, 1, 1)            \
  X(KV_BF16, 512, 0, KIND_SHARED, 1, 2, 2) X(KV_BF16, 512, 0, KIND_SHARED, 1, 1, 2)            \
  X(KV_BF16, 128, 0, KIND_TIED, 8, 1, 1) X(KV_BF16, 128, 0, KIND_TIED, 4, 1, 1)                \
  X(KV_BF16, 128, 0, KIND_TIED, 1, 2, 1) X(KV_BF16, 128, 0, KIND_TIED, 1, 1, 1)                \
  X(KV_F32, 64, 0, KIND_SHARED, 4, 1, 1) X(KV_F32, 64, 0, KIND_SHARED, 1, 1, 1)                \
  X(KV_F32, 64, 0, KIND_TIED, 4, 1, 1) X(KV_F32, 64, 0, KIND_TIED, 1, 1, 1)

int kv_code(const ld_problem& p) { return p.kv_dtype == LD_FP8_E4M3 ? KV_FP8 : p.kv_dtype == LD_BF16 ? KV_BF16 : KV_F32; }
int kind_code(const ld_problem& p) {
  if (p.variant <= LD_VARIANT_MLRA) return KIND_LATENT;
  return p.variant == LD_VARIANT_GTA ? KIND_TIED : KIND_SHARED;
}

}  // namespace

bool decode_instantiated(const ld_problem& p, int nsets, int hblocks) {
  const int kv = kv_code(p), kind = kind_code(p), dl = p.d_latent, dr = p.d_rope;
#define LD_MATCH(KV_, DL_, DR_, KIND_, NS_, HB_, SP_) \
  if (kv == KV_ && dl == DL_ && dr == DR_ && kind == KIND_ && nsets == NS_ && hblocks == HB_) return true;
  LD_SHAPES(LD_MATCH)
#undef LD_MATCH
  return false;
}

int launch_decode(const ld_problem& p, const DecodeArgs& a, void* stream) {
  if (decode_pipe_serves(p, a.nsets, a.hblocks)) return launch_decode_pipe(p, a, stream);
  if (decode_pipe8_serves(p, a.nsets, a.hblocks)) return launch_decode_pipe8(p, a, stream);
  const int kv = kv_code(p), kind = kind_code(p), dl = p.d_latent, dr = p.d_rope;
#define LD_RUN(KV_, DL_, DR_, KIND_, NS_, HB_, SP_)                                               \
  if (kv == KV_ && dl == DL_ && dr == DR_ && kind == KIND_ && a.nsets == NS_ && a.hblocks == HB_) \
    return run<KV_, DL_, DR_, KIND_, NS_, HB_, SP_>(a, stream);
  LD_SHAPES(LD_RUN)
#undef LD_RUN
  return -1;
}

// Work groups of a shape's decode kernel that can be resident on one CU at once (registers, LDS,
// waves), as the runtime reports it for the current device; 1 when it cannot be queried (no
// device).  Cached per shape and device.
template <int KV, int DL, int DR, int KIND, int NSETS, int HB, int SPLIT>
int wgs_per_cu_of() {
  static int cache[kMaxDevices] = {};  // 0: not queried yet
  return occupancy_cached(cache, reinterpret_cast<const void*>(decode_kernel<KV, DL, DR, KIND, NSETS, HB, SPLIT>),
                          NSETS * HB * SPLIT * kWaveSize);
}

int decode_wgs_per_cu(const ld_problem& p, int nsets, int hblocks) {
  if (decode_pipe_serves(p, nsets, hblocks)) return decode_pipe_wgs_per_cu(p);
  if (decode_pipe8_serves(p, nsets, hblocks)) return decode_pipe8_wgs_per_cu(nsets);
  const int kv = kv_code(p), kind = kind_code(p), dl = p.d_latent, dr = p.d_rope;
#define LD_OCC(KV_, DL_, DR_, KIND_, NS_, HB_, SP_) \
  if (kv == KV_ && dl == DL_ && dr == DR_ && kind == KIND_ && nsets == NS_ && hblocks == HB_) \
    return wgs_per_cu_of<KV_, DL_, DR_, KIND_, NS_, HB_, SP_>();
  LD_SHAPES(LD_OCC)
#undef LD_OCC
  return 1;
}

int occupancy_cached(int* cache, const void* kernel, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (v > 0) return v;
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0);
  v = (e == hipSuccess && n > 0) ? n : 1;
  __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);  // every thread computes the same value
  return v;
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

}  // namespace ld
