// Internal definitions shared by the host API and the gfx950 kernels of the
// decode-attention library.  Not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "latent_decode.h"

namespace ld {

// How a work group reads K and V.
enum Kind : int {
  KIND_LATENT = 0,  // MLA / GLA / MLRA: K = [latent slice | rope], V = the latent slice of the same row
  KIND_SHARED = 1,  // GQA / MQA: K and V rows from two pools
  KIND_TIED = 2,    // GTA: V is the K row itself
};

constexpr int kTile = 32;            // tokens per MFMA tile (one 32-row block)
constexpr int kWaveSize = 64;
constexpr int kPlanThreads = 256;
constexpr int kCombineChunk = 16;     // splits merged by one combine task
constexpr int kUnitPages = 512;       // pages a work unit spans at most (its block-table entries fit in LDS)
// The planner splits finer than one unit per CU (to fill several resident work groups per CU) only
// while units keep at least this many pages.
constexpr int kMinChunkPages = 16;
// Batches of at most this many sequences are combined by one launch of wide work groups (each
// sequence then has many splits); larger batches by per-task work groups and a chunk merge.
constexpr int kSeqCombineMaxBatch = 8;

// Work unit record written by the planner: one (sequence, token chunk).
struct alignas(16) Unit {
  int32_t b;
  int32_t t_begin;
  int32_t t_end;
  int32_t split;
};

// Workspace layout (byte offsets from the workspace base, each 256-aligned).
struct WsLayout {
  int32_t max_units = 0;
  int32_t max_tasks = 0;   // bound on combine tasks
  int32_t max_multi = 0;   // bound on sequences with more than one combine task
  int32_t xblocks = 0;     // work groups per combine task (256 piece positions each)
  int32_t rows = 0;        // R: output rows per sequence
  int32_t d_v = 0;
  size_t header = 0;       // int32[64]: [0] num_units, [1] chunk
  size_t units = 0;        // Unit[max_units]
  size_t seqs = 0;         // int32[4*B]: (num_splits, first_unit, first_task, num_tasks) per sequence
  size_t tasks = 0;        // int32[4*max_tasks]: (sequence, chunk, first_unit, num_splits) combine tasks
  size_t multi = 0;        // int32[max_multi]: sequences merged in more than one chunk
  size_t l2_out = 0;       // f32[max_tasks][pieces][values]: chunk results of multi-chunk sequences
  size_t l2_lse = 0;       // f32[max_tasks][pieces]: their lse, per piece lane
  size_t ccount = 0;       // int32[max_tasks][xblocks]: arrivals of a sequence's chunk tasks (first task's row)
  // Split partials, one slot per (unit, set, 32-head block, head): slots = max_units * G * hblocks * 32.
  // part_out holds each slot block's 32 x d_v values in MFMA-fragment order (see decode.hip),
  // bf16 when the output is bf16, else f32.
  size_t part_lse = 0;     // f32[slots]
  size_t part_out = 0;     // [slots][d_v]
  size_t total = 0;
};

// Planner inputs and the plan arrays it writes (ld_plan, or the decode kernel's fused prologue).
struct PlanArgs {
  const int32_t* seq_lens;
  int32_t* header;
  Unit* units;
  int32_t* seqs;
  int32_t* tasks;
  int32_t* multi;
  int32_t* ccount;        // int32[ccount_n]: combine arrival counters, zeroed by the planner
  int32_t ccount_n;
  int32_t max_tasks;
  int32_t max_multi;
  int32_t batch;
  int32_t capacity;       // max_pages_per_seq * page_size
  int32_t page_size;
  int32_t target_units;   // units the planner aims for (auto mode): resident work groups over the chip
  int32_t base_units;     // one work group per CU; the finer target applies down to kMinChunkPages
  int32_t forced_splits;  // 0 = auto
  int32_t max_units;
};

// Everything the decode kernels need, passed by value.
struct DecodeArgs {
  const void* q_lat;
  const void* q_rope;
  const void* k;
  const void* rope;      // fp8 cache: bf16 rope pool
  const void* v;
  const float* kscale;   // fp8 cache: per-token scale
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  const int32_t* header;
  const Unit* units;
  const int32_t* seqs;
  float* part_lse;
  void* part_out;
  const int32_t* tasks;
  const int32_t* multi;
  float* l2_out;
  float* l2_lse;
  int32_t* ccount;             // [max_tasks][xblocks]: chunk tasks of a sequence that have finished
  int32_t max_tasks, max_multi, xblocks;
  int32_t batch, heads, groups, heads_per_set, rows, max_pages, num_pages, page_size;
  int32_t nsets, hblocks;       // sets per work group, 32-head blocks per set
  int32_t wg_per_unit;          // work groups per unit (= groups / nsets)
  int32_t max_units;
  int32_t out_bf16;
  int32_t part_bf16;            // partials stored as bf16 (else f32)
  int32_t mlra;
  // Several query tokens per sequence (qlen > 1): a unit has wg_per_unit / qlen work groups per
  // token; the query sets are token x cache set (groups = qlen * cache_groups, heads = qlen * H),
  // token i seeing the first L_b - qlen + 1 + i rows.
  int32_t qlen, cache_groups;
  float scale_log2;             // softmax_scale * log2(e)
  // Fused plan (ld_latent_decode): every work group derives its unit from seq_lens with the
  // planner rule instead of reading the plan arrays, and the work groups write those arrays for
  // the combine (plan.* pointers).
  int32_t fused_plan;
  PlanArgs plan;
};


// Host planner rule shared (as a specification, not as code) with the device
// planner: see plan_chunk() in api.cpp and plan_kernel in plan_combine.hip.
int32_t target_units_for(const ld_problem& p, int32_t num_cus);
int32_t base_units_for(const ld_problem& p, int32_t num_cus);
int32_t max_units_for(const ld_problem& p, int32_t num_cus);
int32_t rows_per_seq(const ld_problem& p);
int32_t query_sets(const ld_problem& p);

// Launchers (plan_combine.hip, decode.hip).  They return hipError_t as int.
int launch_plan(const PlanArgs& a, void* stream);
int launch_combine_ws(const DecodeArgs& a, int32_t d_v, void* stream);
int launch_combine_rows(int32_t num_rows, int32_t d_v, int32_t max_splits, const float* part_out,
                        const float* part_lse, const int32_t* nsplits, int32_t out_bf16, void* out, float* lse,
                        void* stream);
// Returns hipError_t, or -1 when no kernel is built for the shape.
int launch_decode(const ld_problem& p, const DecodeArgs& a, void* stream);

// one decode step's token appended to the paged latent cache (append.hip)
struct AppendArgs {
  const void* c_new;            // [B, d_lat] latent rows (all groups), bf16 or f32
  const void* kr_new;           // [B, d_rope] un-rotated RoPE keys, same dtype
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* k;                      // cache rows (f32/bf16: [.., d_lat + d_rope]; fp8: codes [.., d_lat])
  void* rope;                   // fp8 cache: bf16 rope pool
  float* scale;                 // fp8 cache: per-token scale
  int32_t batch, d_lat, d_rope, page_size, num_pages, max_pages;
  int32_t in_bf16;
  float rope_base;
};
int launch_append(const AppendArgs& a, int kv_dtype, void* stream);

// per-head projection C[m, h, n] = sum_k W[h, n, k] A[m, h, k] (projection.hip)
struct ProjArgs {
  const void* a;   // bf16 [m, heads, k]
  const void* w;   // bf16 [heads, n, k]
  void* c;         // [m, heads, n], f32 or bf16
  int32_t m, heads, n, k;
};
int launch_head_projection(const ProjArgs& a, int out_bf16, void* stream);
// The software-pipelined kernel (decode_pipe.hip) for bf16 latent caches with 128 heads per work group
// over one latent slice and the rope key (absorbed MLA; MLRA with four branches or one): whether it
// serves the shape, its launcher (hipError_t, or -1 when it does not serve the shape) and how many of
// its work groups fit on one CU.
bool decode_pipe_serves(const ld_problem& p, int nsets, int hblocks);
int launch_decode_pipe(const ld_problem& p, const DecodeArgs& a, void* stream);
int decode_pipe_wgs_per_cu(const ld_problem& p);
// The kernel for fp8 latent caches (decode_pipe_fp8.hip): 256-dim latent groups with a 64-dim RoPE
// key, 64 heads per group, one or two groups per work group.
bool decode_pipe8_serves(const ld_problem& p, int nsets, int hblocks);
int launch_decode_pipe8(const ld_problem& p, const DecodeArgs& a, void* stream);
int decode_pipe8_wgs_per_cu(int nsets);
// Whether a decode kernel is built for p's dtype/dims/kind with `nsets` sets per work group and
// `hblocks` 32-head blocks per set.
bool decode_instantiated(const ld_problem& p, int nsets, int hblocks);
int decode_wgs_per_cu(const ld_problem& p, int nsets, int hblocks);
int device_cu_count();
// Devices whose occupancy figures are cached (per kernel and device): device ids 0 .. kMaxDevices-1.
constexpr int kMaxDevices = 64;
// Resident work groups per CU of `kernel` with `threads` threads on the current device, from the
// runtime's occupancy query, remembered in cache[device]; 1 when it cannot be queried.
int occupancy_cached(int* cache, const void* kernel, int threads);

}  // namespace ld
