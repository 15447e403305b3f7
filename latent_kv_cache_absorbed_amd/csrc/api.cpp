// Host side of the C ABI: problem checks, workspace layout, the host copy of the split-KV
// planner, and the launch sequence plan -> decode -> combine.  See include/latent_decode.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "ld_internal.h"

namespace ld {
namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }
bool latent(const ld_problem& p) { return p.variant <= LD_VARIANT_MLRA; }

struct Shape {
  int heads_per_set = 0, hblocks = 0, nsets = 0, wg_per_unit = 0;
};

// Sets per work group: the largest of 8, 4, 2, 1 that divides G and has a kernel built for it
// (covering all of a set's heads in blocks of 32).
Shape launch_shape(const ld_problem& p) {
  Shape s;
  const int H = p.num_q_heads, G = p.num_groups;
  s.heads_per_set = p.variant == LD_VARIANT_MLRA ? H : H / G;
  s.hblocks = (s.heads_per_set + 31) / 32;
  // fp8 GLA groups of 64 heads: one group per work group (two work groups of four waves share a CU,
  // and their barriers do not hold each other up)
  if (decode_pipe8_serves(p, 1, s.hblocks) && decode_instantiated(p, 1, s.hblocks)) {
    s.nsets = 1;
    s.wg_per_unit = G * p.q_len;
    return s;
  }
  // bf16 MLRA: one branch of 128 heads per work group (the pipelined kernel)
  if (p.variant == LD_VARIANT_MLRA && decode_pipe_serves(p, 1, s.hblocks) && decode_instantiated(p, 1, s.hblocks)) {
    s.nsets = 1;
    s.wg_per_unit = G * p.q_len;
    return s;
  }
  for (int n = 8; n >= 1; n >>= 1) {
    if (G % n) continue;
    if (!decode_instantiated(p, n, s.hblocks)) continue;
    s.nsets = n;
    s.wg_per_unit = G / n * p.q_len;  // (several query tokens: a group of work groups per token)
    break;
  }
  return s;
}

// Forced splits: the most splits one sequence can get, the requested count or, when a split would
// span more than kUnitPages pages, ceil(max_pages_per_seq / kUnitPages).
int32_t forced_split_bound(const ld_problem& p) {
  const int32_t longest = (p.max_pages_per_seq + kUnitPages - 1) / kUnitPages;
  return p.num_splits > longest ? p.num_splits : longest;
}

WsLayout ws_layout(const ld_problem& p, int num_cus) {
  WsLayout w;
  w.max_units = max_units_for(p, num_cus);
  w.rows = rows_per_seq(p);
  w.d_v = p.d_latent;
  size_t off = 0;
  w.header = off;
  off += 256;
  w.units = off;
  off = round256(off + (size_t)w.max_units * sizeof(Unit));
  w.seqs = off;
  off = round256(off + (size_t)p.batch * 4 * sizeof(int32_t));
  const size_t slots = (size_t)w.max_units * query_sets(p) * launch_shape(p).hblocks * 32;
  w.part_lse = off;
  off = round256(off + slots * sizeof(float));
  w.part_out = off;
  off = round256(off + slots * w.d_v * (p.out_dtype == LD_BF16 ? 2 : 4));
  // combine tasks: a sequence with n > 1 splits is merged in ceil(n / kCombineChunk) chunks (an empty
  // one in one task), so there are at most max_units / kCombineChunk + B of them.  Forced splits: a
  // sequence gets the requested count, or more when a split would span more than kUnitPages pages,
  // so the bound takes the larger of the two.
  const int32_t n_forced = forced_split_bound(p);
  w.max_tasks = p.num_splits > 0 ? p.batch * ((n_forced + kCombineChunk - 1) / kCombineChunk)
                                 : (w.max_units + kCombineChunk - 1) / kCombineChunk + p.batch;
  const size_t vals = p.out_dtype == LD_BF16 ? 8 : 4;   // values per piece
  const size_t pieces = (size_t)query_sets(p) * launch_shape(p).hblocks * (w.d_v / 32) * (16 / vals) * 64;
  w.xblocks = (int32_t)(pieces / 256);
  w.tasks = off;
  off = round256(off + (size_t)w.max_tasks * 4 * sizeof(int32_t));
  // a sequence merged in more than one chunk has more than kCombineChunk units
  w.max_multi = p.num_splits > 0 ? (n_forced > kCombineChunk ? p.batch : 0)
                                 : std::min<int32_t>(p.batch, w.max_units / (kCombineChunk + 1));
  w.multi = off;
  off = round256(off + (size_t)(w.max_multi > 0 ? w.max_multi : 1) * sizeof(int32_t));
  w.l2_out = off;
  off = round256(off + (size_t)w.max_tasks * pieces * vals * sizeof(float));
  w.l2_lse = off;
  off = round256(off + (size_t)w.max_tasks * pieces * sizeof(float));
  w.ccount = off;
  off = round256(off + (size_t)w.max_tasks * w.xblocks * sizeof(int32_t));
  w.total = off;
  return w;
}

}  // namespace

int32_t rows_per_seq(const ld_problem& p) {
  return p.q_len * (p.variant == LD_VARIANT_MLRA ? p.num_q_heads * p.num_groups : p.num_q_heads);
}

// Sets of query rows (their partial blocks and combine pieces): the groups of every query token
int32_t query_sets(const ld_problem& p) { return p.q_len * p.num_groups; }

// Units the automatic planner aims for: one wave of work groups over the chip, i.e. as many work
// groups per CU as can be resident at once (at most 4; several for the small work groups of the
// shared-KV and one-share shapes, one for the 8-wave latent shapes).  The finer split applies only
// while units keep kMinChunkPages pages (see plan_common.h).
int32_t base_units_for(const ld_problem& p, int32_t num_cus) {
  const Shape s = launch_shape(p);
  const int wpu = s.wg_per_unit > 0 ? s.wg_per_unit : 1;
  const int t = num_cus / wpu;
  return t < 1 ? 1 : t;
}

int32_t target_units_for(const ld_problem& p, int32_t num_cus) {
  const Shape s = launch_shape(p);
  int occ = s.nsets > 0 ? decode_wgs_per_cu(p, s.nsets, s.hblocks) : 1;
  occ = occ < 1 ? 1 : (occ > 4 ? 4 : occ);
  return base_units_for(p, num_cus) * occ;
}

// A unit spans at most kUnitPages pages, so a sequence has at most ceil(max_pages / kUnitPages)
// units of the longest length; auto: at most target + B units of the computed chunk on top.
int32_t max_units_for(const ld_problem& p, int32_t num_cus) {
  const long long longest = (p.max_pages_per_seq + kUnitPages - 1) / kUnitPages;
  long long m;
  if (p.num_splits > 0)
    m = (long long)p.batch * forced_split_bound(p);
  else
    m = target_units_for(p, num_cus) + (long long)p.batch * longest;
  return (int32_t)(m > (1 << 30) ? (1 << 30) : m);
}

}  // namespace ld

using namespace ld;

extern "C" {

int32_t ld_abi_version(void) { return LD_ABI_VERSION; }

const char* ld_status_string(int32_t s) {
  switch (s) {
    case LD_OK: return "ok";
    case LD_ERR_NULL_POINTER: return "a required pointer is NULL";
    case LD_ERR_BAD_SHAPE: return "bad or inconsistent problem shape";
    case LD_ERR_BAD_DTYPE: return "unsupported dtype combination";
    case LD_ERR_MISALIGNED: return "a pointer is not aligned as required";
    case LD_ERR_UNSUPPORTED: return "shape not supported by the built kernels";
    case LD_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LD_ERR_BAD_METADATA: return "block table or sequence lengths out of range";
    case LD_ERR_HIP: return "HIP launch failed";
    case LD_ERR_BAD_STRUCT: return "ld_problem struct_size mismatch";
    default: return "unknown status";
  }
}

int32_t ld_check_problem(const ld_problem* p) {
  if (!p) return LD_ERR_NULL_POINTER;
  if (p->struct_size != sizeof(ld_problem)) return LD_ERR_BAD_STRUCT;
  if (p->variant < LD_VARIANT_MLA || p->variant > LD_VARIANT_GTA) return LD_ERR_BAD_SHAPE;
  if (p->batch < 0 || p->num_q_heads < 1 || p->num_groups < 1 || p->d_latent < 1 || p->d_rope < 0)
    return LD_ERR_BAD_SHAPE;
  if (p->page_size < 1 || p->page_size > (1 << 20) || p->num_pages < 1 || p->max_pages_per_seq < 1)
    return LD_ERR_BAD_SHAPE;
  if ((long long)p->max_pages_per_seq * p->page_size > 0x7fffffffLL) return LD_ERR_BAD_SHAPE;
  if (p->num_splits < 0) return LD_ERR_BAD_SHAPE;
  if (p->q_len < 1 || p->q_len > 16) return LD_ERR_BAD_SHAPE;
  if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f)) return LD_ERR_BAD_SHAPE;
  const int H = p->num_q_heads, G = p->num_groups;
  switch (p->variant) {
    case LD_VARIANT_MLA:
    case LD_VARIANT_MQA:
      if (G != 1) return LD_ERR_BAD_SHAPE;
      break;
    case LD_VARIANT_GLA:
    case LD_VARIANT_GQA:
    case LD_VARIANT_GTA:
      if (H % G) return LD_ERR_BAD_SHAPE;
      break;
    default:
      break;
  }
  if (latent(*p)) {
    if (p->d_rope < 1) return LD_ERR_BAD_SHAPE;
  } else if (p->d_rope != 0) {
    return LD_ERR_BAD_SHAPE;
  }
  // dtypes: f32 query with f32 cache; bf16 query with bf16 or (latent) fp8 cache
  if (p->out_dtype != LD_F32 && p->out_dtype != LD_BF16) return LD_ERR_BAD_DTYPE;
  if (p->kv_dtype == LD_F32) {
    if (p->q_dtype != LD_F32) return LD_ERR_BAD_DTYPE;
  } else if (p->kv_dtype == LD_BF16) {
    if (p->q_dtype != LD_BF16) return LD_ERR_BAD_DTYPE;
  } else if (p->kv_dtype == LD_FP8_E4M3) {
    if (p->q_dtype != LD_BF16 || !latent(*p)) return LD_ERR_BAD_DTYPE;
  } else {
    return LD_ERR_BAD_DTYPE;
  }
  // stages of 32 tokens must not straddle pages
  if (p->page_size % kTile) return LD_ERR_UNSUPPORTED;
  if (launch_shape(*p).nsets == 0) return LD_ERR_UNSUPPORTED;
  return LD_OK;
}

int32_t ld_workspace_size(const ld_problem* p, size_t* bytes) {
  if (!bytes) return LD_ERR_NULL_POINTER;
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  *bytes = ws_layout(*p, device_cu_count()).total;
  return LD_OK;
}

int32_t ld_plan_host(const ld_problem* p, const int32_t* seq_lens_host, int32_t num_cus, int32_t* chunk_out,
                     int32_t* num_units, int32_t* splits_out, int32_t* first_unit_out) {
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  if ((p->batch > 0 && (!seq_lens_host || !splits_out || !first_unit_out)) || !chunk_out || !num_units)
    return LD_ERR_NULL_POINTER;
  if (num_cus < 1) return LD_ERR_BAD_SHAPE;
  const long long cap = (long long)p->max_pages_per_seq * p->page_size;
  const int page = p->page_size;
  auto clampL = [&](int32_t L) -> long long { return L < 0 ? 0 : (L > cap ? cap : L); };
  long long chunk = 0;
  if (p->num_splits == 0) {
    // the smallest multiple of the page that gives at most `target` units (bisection on pages)
    long long mx = 0;
    for (int b = 0; b < p->batch; ++b) mx = std::max(mx, clampL(seq_lens_host[b]));
    auto chunk_for = [&](long long target) {
      long long lo = 1, hi = std::max(1LL, (mx + page - 1) / page);
      while (lo < hi) {
        const long long mid = (lo + hi) / 2, c = mid * page;
        long long cnt = 0;
        for (int b = 0; b < p->batch; ++b) cnt += (clampL(seq_lens_host[b]) + c - 1) / c;
        if (cnt <= target)
          hi = mid;
        else
          lo = mid + 1;
      }
      return std::min(lo, (long long)kUnitPages) * page;
    };
    // the finer target (several resident work groups per CU) down to kMinChunkPages pages, never
    // coarser than one unit per CU
    const long long base = base_units_for(*p, num_cus), target = target_units_for(*p, num_cus);
    const long long c1 = chunk_for(base);
    chunk = target == base ? c1 : std::max(chunk_for(target), std::min(c1, (long long)kMinChunkPages * page));
  }
  long long units = 0;
  for (int b = 0; b < p->batch; ++b) {
    const long long L = clampL(seq_lens_host[b]);
    long long ck = chunk;
    if (p->num_splits > 0) {
      const long long per = (L + p->num_splits - 1) / p->num_splits;
      ck = (per + page - 1) / page * page;
      if (ck < page) ck = page;
      if (ck > (long long)kUnitPages * page) ck = (long long)kUnitPages * page;
    }
    const long long n = (L + ck - 1) / ck;
    splits_out[b] = (int32_t)n;
    first_unit_out[b] = (int32_t)units;
    units += n;
  }
  *chunk_out = (int32_t)chunk;
  *num_units = (int32_t)units;
  return LD_OK;
}

int32_t ld_validate_metadata(const ld_problem* p, const int32_t* block_table_host, const int32_t* seq_lens_host) {
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  if (p->batch == 0) return LD_OK;
  if (!block_table_host || !seq_lens_host) return LD_ERR_NULL_POINTER;
  const long long cap = (long long)p->max_pages_per_seq * p->page_size;
  for (int b = 0; b < p->batch; ++b) {
    const int32_t L = seq_lens_host[b];
    if (L < 0 || L > cap) return LD_ERR_BAD_METADATA;
    const int used = (int)((L + p->page_size - 1) / p->page_size);
    for (int i = 0; i < used; ++i) {
      const int32_t pg = block_table_host[(size_t)b * p->max_pages_per_seq + i];
      if (pg < 0 || pg >= p->num_pages) return LD_ERR_BAD_METADATA;
    }
  }
  return LD_OK;
}

}  // extern "C"

namespace {

int32_t check_pointers(const ld_problem* p, const void* q_latent, const void* q_rope, const ld_kv_cache* cache,
                       const int32_t* block_table, const int32_t* seq_lens, const void* out, const float* lse) {
  const bool lat = latent(*p);
  const bool fp8 = p->kv_dtype == LD_FP8_E4M3;
  if (!q_latent || !cache || !cache->k || !block_table || !seq_lens || !out || !lse) return LD_ERR_NULL_POINTER;
  if (lat && !q_rope) return LD_ERR_NULL_POINTER;
  if (fp8 && (!cache->rope || !cache->scale)) return LD_ERR_NULL_POINTER;
  if ((p->variant == LD_VARIANT_GQA || p->variant == LD_VARIANT_MQA) && !cache->v) return LD_ERR_NULL_POINTER;
  if (!aligned(q_latent, 16) || (lat && !aligned(q_rope, 16)) || !aligned(cache->k, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return LD_ERR_MISALIGNED;
  if (cache->v && !aligned(cache->v, 16)) return LD_ERR_MISALIGNED;
  if (fp8 && (!aligned(cache->rope, 16) || !aligned(cache->scale, 16))) return LD_ERR_MISALIGNED;
  return LD_OK;
}

int32_t check_workspace(const ld_problem* p, const void* workspace, size_t workspace_bytes, WsLayout* w) {
  if (!workspace) return LD_ERR_NULL_POINTER;
  if (!aligned(workspace, 256)) return LD_ERR_MISALIGNED;
  *w = ws_layout(*p, device_cu_count());
  if (workspace_bytes < w->total) return LD_ERR_WORKSPACE_TOO_SMALL;
  return LD_OK;
}

DecodeArgs decode_args(const ld_problem* p, const WsLayout& w, void* workspace) {
  const Shape s = launch_shape(*p);
  char* ws = static_cast<char*>(workspace);
  DecodeArgs a{};
  a.header = reinterpret_cast<const int32_t*>(ws + w.header);
  a.units = reinterpret_cast<const Unit*>(ws + w.units);
  a.seqs = reinterpret_cast<const int32_t*>(ws + w.seqs);
  a.part_lse = reinterpret_cast<float*>(ws + w.part_lse);
  a.part_out = ws + w.part_out;
  a.tasks = reinterpret_cast<const int32_t*>(ws + w.tasks);
  a.multi = reinterpret_cast<const int32_t*>(ws + w.multi);
  a.l2_out = reinterpret_cast<float*>(ws + w.l2_out);
  a.l2_lse = reinterpret_cast<float*>(ws + w.l2_lse);
  a.ccount = reinterpret_cast<int32_t*>(ws + w.ccount);
  a.max_tasks = w.max_tasks;
  a.max_multi = w.max_multi;
  a.xblocks = w.xblocks;
  a.batch = p->batch;
  a.heads = p->num_q_heads * p->q_len;
  a.groups = query_sets(*p);
  a.qlen = p->q_len;
  a.cache_groups = p->num_groups;
  a.heads_per_set = s.heads_per_set;
  a.rows = w.rows;
  a.max_pages = p->max_pages_per_seq;
  a.num_pages = p->num_pages;
  a.page_size = p->page_size;
  a.nsets = s.nsets;
  a.hblocks = s.hblocks;
  a.wg_per_unit = s.wg_per_unit;
  a.max_units = w.max_units;
  a.out_bf16 = p->out_dtype == LD_BF16;
  a.part_bf16 = a.out_bf16;
  a.mlra = p->variant == LD_VARIANT_MLRA;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  return a;
}

PlanArgs plan_args(const ld_problem* p, const WsLayout& w, void* workspace, const int32_t* seq_lens) {
  char* ws = static_cast<char*>(workspace);
  PlanArgs pa;
  pa.seq_lens = seq_lens;
  pa.header = reinterpret_cast<int32_t*>(ws + w.header);
  pa.units = reinterpret_cast<Unit*>(ws + w.units);
  pa.seqs = reinterpret_cast<int32_t*>(ws + w.seqs);
  pa.tasks = reinterpret_cast<int32_t*>(ws + w.tasks);
  pa.multi = reinterpret_cast<int32_t*>(ws + w.multi);
  pa.ccount = reinterpret_cast<int32_t*>(ws + w.ccount);
  pa.ccount_n = w.max_tasks * w.xblocks;
  pa.max_tasks = w.max_tasks;
  pa.max_multi = w.max_multi;
  pa.batch = p->batch;
  pa.capacity = p->max_pages_per_seq * p->page_size;
  pa.page_size = p->page_size;
  pa.target_units = target_units_for(*p, device_cu_count());
  pa.base_units = base_units_for(*p, device_cu_count());
  pa.forced_splits = p->num_splits;
  pa.max_units = w.max_units;
  return pa;
}

// The decode launch shared by ld_decode_planned (plan read from the workspace) and
// ld_latent_decode (plan derived in the kernel, fused = true).
int32_t decode_launch(const ld_problem* p, const WsLayout& w, const void* q_latent, const void* q_rope,
                      const ld_kv_cache* cache, const int32_t* block_table, const int32_t* seq_lens, void* out,
                      float* lse, void* workspace, bool fused, void* stream) {
  DecodeArgs a = decode_args(p, w, workspace);
  a.q_lat = q_latent;
  a.q_rope = q_rope;
  a.k = cache->k;
  a.rope = cache->rope;
  a.v = cache->v;
  a.kscale = cache->scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.fused_plan = fused ? 1 : 0;
  if (fused) a.plan = plan_args(p, w, workspace, seq_lens);
  const int r = launch_decode(*p, a, stream);
  if (r == -1) return LD_ERR_UNSUPPORTED;
  return r == hipSuccess ? LD_OK : LD_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t ld_plan(const ld_problem* p, const int32_t* seq_lens, void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  if (p->batch == 0) return LD_OK;
  if (!seq_lens) return LD_ERR_NULL_POINTER;
  if (!aligned(seq_lens, 4)) return LD_ERR_MISALIGNED;
  WsLayout w;
  const int32_t sw = check_workspace(p, workspace, workspace_bytes, &w);
  if (sw != LD_OK) return sw;
  return launch_plan(plan_args(p, w, workspace, seq_lens), stream) == hipSuccess ? LD_OK : LD_ERR_HIP;
}

int32_t ld_decode_planned(const ld_problem* p, const void* q_latent, const void* q_rope, const ld_kv_cache* cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  if (p->batch == 0) return LD_OK;
  const int32_t sp = check_pointers(p, q_latent, q_rope, cache, block_table, seq_lens, out, lse);
  if (sp != LD_OK) return sp;
  WsLayout w;
  const int32_t sw = check_workspace(p, workspace, workspace_bytes, &w);
  if (sw != LD_OK) return sw;
  return decode_launch(p, w, q_latent, q_rope, cache, block_table, seq_lens, out, lse, workspace, false, stream);
}

int32_t ld_combine_planned(const ld_problem* p, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  if (p->batch == 0) return LD_OK;
  if (!out || !lse) return LD_ERR_NULL_POINTER;
  if (!aligned(out, 16) || !aligned(lse, 4)) return LD_ERR_MISALIGNED;
  WsLayout w;
  const int32_t sw = check_workspace(p, workspace, workspace_bytes, &w);
  if (sw != LD_OK) return sw;
  DecodeArgs a = decode_args(p, w, workspace);
  a.out = out;
  a.lse = lse;
  return launch_combine_ws(a, p->d_latent, stream) == hipSuccess ? LD_OK : LD_ERR_HIP;
}

int32_t ld_plan_decode(const ld_problem* p, const void* q_latent, const void* q_rope, const ld_kv_cache* cache,
                       const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const int32_t st = ld_check_problem(p);
  if (st != LD_OK) return st;
  if (p->batch == 0) return LD_OK;
  const int32_t sp = check_pointers(p, q_latent, q_rope, cache, block_table, seq_lens, out, lse);
  if (sp != LD_OK) return sp;
  WsLayout w;
  const int32_t sw = check_workspace(p, workspace, workspace_bytes, &w);
  if (sw != LD_OK) return sw;
  // one launch fewer than ld_plan + ld_decode_planned: the decode kernel plans for itself and
  // leaves the plan arrays in the workspace for the combine
  return decode_launch(p, w, q_latent, q_rope, cache, block_table, seq_lens, out, lse, workspace, true, stream);
}

int32_t ld_latent_decode(const ld_problem* p, const void* q_latent, const void* q_rope, const ld_kv_cache* cache,
                         const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int32_t r = ld_plan_decode(p, q_latent, q_rope, cache, block_table, seq_lens, out, lse, workspace,
                                   workspace_bytes, stream);
  if (r != LD_OK || p->batch == 0) return r;
  return ld_combine_planned(p, out, lse, workspace, workspace_bytes, stream);
}

int32_t ld_cache_append(const ld_problem* p, const void* c_new, const void* kr_new, const int32_t* block_table,
                        const int32_t* seq_lens, const ld_kv_cache* cache, float rope_base, void* stream) {
  if (!p || !cache) return LD_ERR_NULL_POINTER;
  if (p->struct_size != sizeof(ld_problem)) return LD_ERR_BAD_STRUCT;
  if (!latent(*p)) return LD_ERR_UNSUPPORTED;
  if (p->batch < 0 || p->num_groups < 1 || p->d_latent < 1 || p->d_rope < 0 || (p->d_rope & 1))
    return LD_ERR_BAD_SHAPE;
  if (p->variant == LD_VARIANT_MLA && p->num_groups != 1) return LD_ERR_BAD_SHAPE;
  if (p->page_size < 1 || p->page_size > (1 << 20) || p->num_pages < 1 || p->max_pages_per_seq < 1)
    return LD_ERR_BAD_SHAPE;
  if ((long long)p->max_pages_per_seq * p->page_size > 0x7fffffffLL) return LD_ERR_BAD_SHAPE;
  if ((long long)p->num_groups * p->d_latent > (1 << 24)) return LD_ERR_BAD_SHAPE;
  if (!std::isfinite(rope_base) || !(rope_base > 0.f)) return LD_ERR_BAD_SHAPE;
  if (p->q_dtype != LD_F32 && p->q_dtype != LD_BF16) return LD_ERR_BAD_DTYPE;
  if (p->kv_dtype != LD_F32 && p->kv_dtype != LD_BF16 && p->kv_dtype != LD_FP8_E4M3) return LD_ERR_BAD_DTYPE;
  if (p->batch == 0) return LD_OK;
  const bool fp8 = p->kv_dtype == LD_FP8_E4M3;
  if (!c_new || (p->d_rope > 0 && !kr_new) || !block_table || !seq_lens || !cache->k) return LD_ERR_NULL_POINTER;
  if (fp8 && (!cache->scale || (p->d_rope > 0 && !cache->rope))) return LD_ERR_NULL_POINTER;
  if (!aligned(c_new, 16) || (kr_new && !aligned(kr_new, 16)) || !aligned(cache->k, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4))
    return LD_ERR_MISALIGNED;
  if (fp8 && (!aligned(cache->scale, 4) || (cache->rope && !aligned(cache->rope, 16)))) return LD_ERR_MISALIGNED;
  AppendArgs a{};
  a.c_new = c_new;
  a.kr_new = kr_new;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.k = const_cast<void*>(cache->k);
  a.rope = const_cast<void*>(cache->rope);
  a.scale = const_cast<float*>(cache->scale);
  a.batch = p->batch;
  a.d_lat = p->num_groups * p->d_latent;
  a.d_rope = p->d_rope;
  a.page_size = p->page_size;
  a.num_pages = p->num_pages;
  a.max_pages = p->max_pages_per_seq;
  a.in_bf16 = p->q_dtype == LD_BF16;
  a.rope_base = rope_base;
  return launch_append(a, p->kv_dtype, stream) == 0 ? LD_OK : LD_ERR_HIP;
}

int32_t ld_head_projection(int32_t m, int32_t heads, int32_t n, int32_t k, const void* a, const void* w, void* c,
                           int32_t out_dtype, void* stream) {
  if (m < 0 || heads < 1 || n < 32 || n % 32 || k < 16 || k % 16) return LD_ERR_BAD_SHAPE;
  if ((long long)m * heads * (k > n ? k : n) > (1LL << 40) || (long long)heads * n * k > (1LL << 40))
    return LD_ERR_BAD_SHAPE;
  if (out_dtype != LD_F32 && out_dtype != LD_BF16) return LD_ERR_BAD_DTYPE;
  if (m == 0) return LD_OK;
  if (!a || !w || !c) return LD_ERR_NULL_POINTER;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(c, 16)) return LD_ERR_MISALIGNED;
  ProjArgs pa;
  pa.a = a;
  pa.w = w;
  pa.c = c;
  pa.m = m;
  pa.heads = heads;
  pa.n = n;
  pa.k = k;
  return launch_head_projection(pa, out_dtype == LD_BF16, stream) == 0 ? LD_OK : LD_ERR_HIP;
}

int32_t ld_split_kv_combine(int32_t num_rows, int32_t d_v, int32_t max_splits, const float* partial_out,
                            const float* partial_lse, const int32_t* row_num_splits, int32_t out_dtype, void* out,
                            float* lse, void* stream) {
  if (num_rows < 0 || d_v < 4 || (d_v % 4) != 0 || max_splits < 1) return LD_ERR_BAD_SHAPE;
  if (out_dtype != LD_F32 && out_dtype != LD_BF16) return LD_ERR_BAD_DTYPE;
  if (num_rows == 0) return LD_OK;
  if (!partial_out || !partial_lse || !row_num_splits || !out || !lse) return LD_ERR_NULL_POINTER;
  if (!aligned(partial_out, 16) || !aligned(out, out_dtype == LD_F32 ? 16 : 8) || !aligned(partial_lse, 4) ||
      !aligned(row_num_splits, 4) || !aligned(lse, 4))
    return LD_ERR_MISALIGNED;
  if (launch_combine_rows(num_rows, d_v, max_splits, partial_out, partial_lse, row_num_splits,
                          out_dtype == LD_BF16, out, lse, stream) != hipSuccess)
    return LD_ERR_HIP;
  return LD_OK;
}

}  // extern "C"
