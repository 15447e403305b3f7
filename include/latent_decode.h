/*
 * latent_decode.h -- C ABI of the MI355X (gfx950) decode-attention library.
 *
 * One decode step (one query token per sequence, at position L_b - 1) of
 * attention over a paged KV cache that has been shrunk by low-rank latent
 * compression or by sharing.
 *
 * What is computed.  For every query row r of sequence b with query q_r and
 * cache rows k_j, v_j (j = 0 .. L_b - 1):
 *     s_j = softmax_scale * (q_r . k_j)
 *     out_r = sum_j softmax_j(s) v_j,        lse_r = ln sum_j exp(s_j)
 * This is the attention formula of the MLA explainer on mlqm.cn (news 371735),
 * section 2.3; its section 2.2 gives the split of q and k into a semantic part
 * and a decoupled RoPE part, and only the semantic value enters the output.
 * The MLRA article (aitntnews, "超越MLA！新架构MLRA百万token，解码最高2.8倍速 |
 * ICLR'26"), in its MLA paragraph, states that folding W_UK into the query
 * turns MLA decode into one 576-dim MQA whose cached row is shared by all
 * heads; this library consumes that absorbed form and returns the output in
 * latent space.  Variants (ld_variant):
 *   MLA   row = [c (d_latent) | k_rope (d_rope)]; every head: k = row, v = c.
 *   GLA   row = [c_0 | .. | c_{G-1} | k_rope]; head h of group g = h / (H/G)
 *         scores against [c_g | k_rope] and averages c_g  (GTA/GLA article,
 *         jsbsmhs.com, section on Grouped Latent Attention).
 *   MLRA  row = [c_0 | .. | c_{G-1} | k_rope]; every head attends every branch
 *         separately, one softmax per branch; the branch outputs are returned
 *         per branch for the caller's up-projection and sum (MLRA article,
 *         "Block Decomposition" and "Moving the Sum Outside").
 *   GQA   per-kv-head K and V rows of d_latent dims; head h uses kv head
 *         h / (H/G).  MQA is GQA with G = 1 (MLRA article's list of methods).
 *   GTA   GQA whose V is the same tied state as K (GTA/GLA article, section on
 *         Grouped-Tied Attention).
 *
 * Several query tokens (q_len = Q > 1): every query row r becomes Q
 * rows (i, r), i = 0 .. Q-1, token i seeing the first L_b - Q + 1 + i cache rows
 * (none when that is not positive: out = 0, lse = -inf); the layouts below then
 * have Q*H rows per sequence where they have H, row i*H + h.
 *
 * Layouts (row-major, innermost dimension last):
 *   q_latent  MLA/GLA [B, H, d_latent]; MLRA [B, H, G, d_latent]; GQA/MQA/GTA [B, H, d_latent]
 *   q_rope    MLA/GLA [B, H, d_rope];   MLRA [B, H, G, d_rope];   NULL for GQA/MQA/GTA
 *             (already rotated: the library never applies RoPE)
 *   cache->k  latent variants, f32/bf16:  [num_pages, page_size, G*d_latent + d_rope]
 *             latent variants, fp8:      E4M3 codes [num_pages, page_size, G*d_latent]
 *             GQA/MQA/GTA:               [num_pages, page_size, G, d_latent]
 *   cache->rope   fp8 latent variants only: bf16 [num_pages, page_size, d_rope]
 *   cache->scale  fp8 latent variants only: f32 [num_pages, page_size]; the latent
 *                 value of a token is code_value * scale (OCP E4M3, bias 7, max 448)
 *   cache->v  GQA/MQA: [num_pages, page_size, G, d_latent]; GTA and latent variants: NULL
 *   block_table  int32 [B, max_pages_per_seq]: logical page i of sequence b is
 *                physical page block_table[b*max_pages_per_seq + i]
 *   seq_lens     int32 [B]: rows in the cache for sequence b, the current token included
 *   out       [B, R, d_latent] in out_dtype, with R = H*G for MLRA (row h*G + branch)
 *             and R = H otherwise
 *   lse       f32 [B, R]: natural-log sum of exp of the scaled scores
 *
 * Ownership and synchronisation: the caller allocates and owns every buffer,
 * the workspace included; pointers are device pointers unless a name says
 * _host.  The library never allocates or frees memory, never keeps a pointer
 * after returning and never synchronises: all work is queued on `stream`
 * (a hipStream_t; NULL means the default stream) and completes in stream
 * order.  Every entry point is thread-safe.
 *
 * Errors: every host-checkable problem (a NULL or non-16-byte-aligned pointer,
 * an unsupported shape or dtype, a too small workspace) is reported before
 * anything is queued, and a failed call queues nothing.  A launch failure is
 * LD_ERR_HIP.  The contents of block_table and seq_lens live on the device
 * and are not checked on the hot path; ld_validate_metadata checks host
 * copies.  On the device, lengths are clamped to [0, max_pages_per_seq *
 * page_size] and page ids to [0, num_pages) so that bad metadata cannot read
 * outside the cache (the numbers are then meaningless, but nothing faults).
 * A sequence with seq_len = 0 gets out = 0 and lse = -inf.
 */
#ifndef LATENT_DECODE_H
#define LATENT_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LD_ABI_VERSION 2

typedef enum ld_status {
  LD_OK = 0,
  LD_ERR_NULL_POINTER = 1,
  LD_ERR_BAD_SHAPE = 2,
  LD_ERR_BAD_DTYPE = 3,
  LD_ERR_MISALIGNED = 4,
  LD_ERR_UNSUPPORTED = 5,
  LD_ERR_WORKSPACE_TOO_SMALL = 6,
  LD_ERR_BAD_METADATA = 7,
  LD_ERR_HIP = 8,
  LD_ERR_BAD_STRUCT = 9
} ld_status;

typedef enum ld_variant {
  LD_VARIANT_MLA = 0,
  LD_VARIANT_GLA = 1,
  LD_VARIANT_MLRA = 2,
  LD_VARIANT_GQA = 3,
  LD_VARIANT_MQA = 4,
  LD_VARIANT_GTA = 5
} ld_variant;

typedef enum ld_dtype { LD_F32 = 0, LD_BF16 = 1, LD_FP8_E4M3 = 2 } ld_dtype;

/* Shape of one decode problem.  Enumerations are stored as int32_t so the
 * struct has one fixed layout for every caller. */
typedef struct ld_problem {
  uint32_t struct_size;      /* sizeof(ld_problem): guards against ABI drift */
  int32_t variant;           /* ld_variant */
  int32_t batch;             /* B >= 0 */
  int32_t num_q_heads;       /* H */
  int32_t num_groups;        /* G: GLA groups | MLRA branches | kv heads (GQA/GTA) | 1 (MLA, MQA) */
  int32_t d_latent;          /* per-group latent (MLA 512, GLA 256, MLRA 128) or head dim (GQA/MQA/GTA) */
  int32_t d_rope;            /* RoPE key dims of the latent variants (64); 0 for GQA/MQA/GTA */
  int32_t page_size;         /* tokens per page: 64 */
  int32_t num_pages;         /* physical pages in the cache pool */
  int32_t max_pages_per_seq; /* columns of block_table */
  int32_t q_dtype;           /* ld_dtype of q_latent and q_rope: F32 or BF16 */
  int32_t kv_dtype;          /* ld_dtype of the cache: F32, BF16 or FP8_E4M3 (latent variants) */
  int32_t out_dtype;         /* ld_dtype of out: F32 or BF16 */
  float softmax_scale;       /* multiplies q.k; positive and finite (else LD_ERR_BAD_SHAPE);
                                lse is reported in this scaled domain */
  int32_t num_splits;        /* 0: the planner splits long sequences over CUs; n >= 1: at most n splits,
                                except that no split spans more than 512 pages */
  int32_t q_len;             /* Q >= 1 query tokens per sequence (several for speculative / multi-token
                                decode; Q <= 16): query token i sits at position
                                L_b - Q + i and attends the cache rows 0 .. L_b - Q + i (causal) */
} ld_problem;

/* Device pointers of the paged cache (see the layouts above). */
typedef struct ld_kv_cache {
  const void* k;
  const void* rope;
  const void* v;
  const float* scale;
} ld_kv_cache;

/* ABI version of the loaded library (LD_ABI_VERSION). */
int32_t ld_abi_version(void);

/* Static text for a status code (never NULL). */
const char* ld_status_string(int32_t status);

/* Host-only shape/dtype check of a problem: the checks ld_latent_decode makes
 * before queuing anything (no pointers are examined).  LD_OK or the error. */
int32_t ld_check_problem(const ld_problem* p);

/* Bytes of device workspace ld_latent_decode needs for this problem (split-KV
 * partial outputs and the work list).  Depends on the shape and on the current
 * device (its compute-unit count and how many decode work groups fit on one),
 * never on the contents of seq_lens: query it with the device current that
 * will run the calls.  Returns LD_OK and writes *bytes, or a shape error. */
int32_t ld_workspace_size(const ld_problem* p, size_t* bytes);

/* One decode step: plan the split-KV work list from seq_lens, run the decode
 * kernel over every (sequence, token chunk), and merge the chunks of split
 * sequences with the log-sum-exp rule.  Asynchronous on `stream`; two launches:
 * the decode kernel derives the plan itself (the planner rule of ld_plan) and
 * leaves the plan in the workspace, then the combine.  The results are the
 * same bits as ld_plan + ld_decode_planned + ld_combine_planned.
 * workspace: device buffer of at least ld_workspace_size bytes, 256-byte
 * aligned, owned by the caller and not used concurrently by another call. */
int32_t ld_latent_decode(const ld_problem* p, const void* q_latent, const void* q_rope,
                         const ld_kv_cache* cache, const int32_t* block_table, const int32_t* seq_lens,
                         void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* The first of ld_latent_decode's two launches: the decode kernel with the planner rule applied in
 * its own prologue, which leaves the plan arrays in the workspace.  Followed by ld_combine_planned
 * (same problem, output buffers and workspace, same stream), it is ld_latent_decode, launch for
 * launch and bit for bit; the split lets a caller put work or a timing event between the decode
 * and the merge of its split partials (the flash-decoding combine).  Argument checks, ownership and
 * errors as ld_latent_decode. */
int32_t ld_plan_decode(const ld_problem* p, const void* q_latent, const void* q_rope, const ld_kv_cache* cache,
                       const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Size of the fixed device array that ld_latent_decode_noalloc uses as its workspace (64 MiB). */
#define LD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): ld_latent_decode with the workspace taken from a fixed
 * device array of the library, LD_NOALLOC_SCRATCH_BYTES bytes, instead of a caller buffer.  Same
 * problem, arguments, layouts, results (the same bits) and errors as ld_latent_decode.
 *   - It allocates nothing: no hipMalloc/hipFree, no library allocation.  The array is part of the
 *     library's device code; each GPU the library runs on holds its own copy until the process
 *     ends.  Its device address is looked up on the first call on each device.
 *   - A problem whose ld_workspace_size exceeds LD_NOALLOC_SCRATCH_BYTES is rejected with
 *     LD_ERR_WORKSPACE_TOO_SMALL before anything is queued (every one-token workload of the
 *     benchmark fits; several query tokens at batch 64 and 128 heads do not).
 *   - Every call on one GPU shares that GPU's array and leaves its contents behind (the decode
 *     kernel re-initialises what must start at zero).  Calls that overlap on one GPU -- on two
 *     streams, or from two threads without ordering -- race on the array: order them on one
 *     stream, or use ld_latent_decode with a workspace of one's own per stream. */
int32_t ld_latent_decode_noalloc(const ld_problem* p, const void* q_latent, const void* q_rope,
                                 const ld_kv_cache* cache, const int32_t* block_table, const int32_t* seq_lens,
                                 void* out, float* lse, void* stream);

/* Stage-wise form of ld_latent_decode: ld_plan, then ld_decode_planned, then
 * ld_combine_planned, queued on one stream in that order with the same problem
 * shape and workspace.  The plan depends only on seq_lens and the shape, so a
 * caller that runs several layers over the same sequences in one decode step
 * can plan once and run decode + combine per layer.  Each stage has the
 * argument checks, ownership and error behaviour of ld_latent_decode. */
int32_t ld_plan(const ld_problem* p, const int32_t* seq_lens, void* workspace, size_t workspace_bytes, void* stream);
int32_t ld_decode_planned(const ld_problem* p, const void* q_latent, const void* q_rope, const ld_kv_cache* cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);
int32_t ld_combine_planned(const ld_problem* p, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Merge per-split partial results with the log-sum-exp rule (flash-decoding
 * combine).  For row r with n = row_num_splits[r] (0 <= n <= max_splits):
 *   lse_r = ln sum_{s<n} exp(partial_lse[r][s])
 *   out_r = sum_{s<n} exp(partial_lse[r][s] - lse_r) * partial_out[r][s][:]
 * Each partial_out[r][s] is that split's normalised output; a split whose lse
 * is -inf has zero weight; n = 0 or all splits empty gives out = 0, lse = -inf;
 * a NaN lse among a row's splits makes that row's out and lse NaN (as the rule
 * computes it; the decode's own merge treats its split partials the same way).
 * partial_out f32 [num_rows, max_splits, d_v]; partial_lse f32 [num_rows, max_splits];
 * row_num_splits int32 [num_rows]; out [num_rows, d_v] in out_dtype; lse f32 [num_rows].
 * d_v must be a multiple of 4. */
int32_t ld_split_kv_combine(int32_t num_rows, int32_t d_v, int32_t max_splits, const float* partial_out,
                            const float* partial_lse, const int32_t* row_num_splits, int32_t out_dtype, void* out,
                            float* lse, void* stream);

/* Append the decode step's new token of every sequence to the paged latent cache (latent variants:
 * MLA, GLA, MLRA).  This is the step that precedes the attention: the cached row of a token is its
 * latent c^KV followed by its decoupled RoPE key k^R, already rotated (MLA explainer, mlqm.cn news
 * 371735, sections 2.2 and 2.4; MLRA article, MLA paragraph: only the latent and the RoPE key are
 * cached); the fp8 cache follows the FP8 serving of the GTA/GLA article (jsbsmhs.com).
 *   For sequence b with L = seq_lens[b] >= 1 (the length counting the new token) the token goes to
 *   logical position pos = L - 1: physical page block_table[b*max_pages_per_seq + pos / page_size],
 *   slot pos % page_size.  A sequence with L <= 0, with L > max_pages_per_seq * page_size, or whose
 *   block-table entry for that page lies outside [0, num_pages) is skipped: nothing of the cache is
 *   written for it (unlike the decode, which only reads and clamps, a write must not land in a slot
 *   the metadata does not name).
 *   c_new   [B, G*d_latent]: the token's latent row (all groups), in q_dtype (F32 or BF16)
 *   kr_new  [B, d_rope]: its RoPE key before rotation, in q_dtype; d_rope must be even
 *   RoPE:   pair (2i, 2i+1) turns by pos * rope_base^(-2i/d_rope) (angle, cosine, sine and rotation
 *           in fp64, then rounded to the cache dtype); rope_base > 0 and finite
 *   kv_dtype F32/BF16: cache->k row = [latent | rotated key], converted with round to nearest even
 *   kv_dtype FP8_E4M3: one scale per token, scale = amax|latent| / 448 in fp32 (1 for a zero row);
 *           cache->k gets the E4M3 code nearest to latent / scale (fp32 division, clamped to +-448,
 *           ties to the even code), cache->scale the scale, cache->rope the rotated key in bf16.
 * The problem's num_q_heads, out_dtype, softmax_scale and num_splits are not used.  The cache
 * pointers are written through (the memory must be writable).  GQA/MQA/GTA give LD_ERR_UNSUPPORTED.
 * Asynchronous on `stream`; a failed call queues nothing. */
int32_t ld_cache_append(const ld_problem* p, const void* c_new, const void* kr_new, const int32_t* block_table,
                        const int32_t* seq_lens, const ld_kv_cache* cache, float rope_base, void* stream);

/* Per-head projection around the absorbed decode step, bf16 operands, fp32 accumulation:
 *   c[i, h, j] = sum_{t < k} w[h, j, t] * a[i, h, t]       (i < m, h < heads, j < n)
 * It is the query absorption, which folds the key up-projection into the query so attention runs in
 * latent space (a = q^C [B, H, d_nope], w[h] = W_UK[h]^T stored [d_latent, d_nope]), and the output
 * up-projection that maps the latent result back (a = o_lat [B, H, d_latent], w[h] = W_UV[h]
 * [d_v, d_latent]); for MLRA, a holds a head's branch outputs side by side [B, H, G*d_latent] and
 * w[h] the branch up-projections side by side, which sums the branches after projecting them (MLRA
 * article: the MLA paragraph, and "Moving the Sum Outside"; the "MLA vs MQA" page lists a custom
 * latent-projection kernel).
 *   a bf16 [m, heads, k]; w bf16 [heads, n, k] (row j of w[h] holds the k weights of output j);
 *   c [m, heads, n] in out_dtype (F32 or BF16, rounded to nearest even).  n a multiple of 32, k a
 *   multiple of 16, pointers 16-byte aligned.  m = 0 does nothing.  Asynchronous on `stream`.  The first
 *   call on a device with 256 < k <= 512 (k % 64 == 0, n % 64 == 0) also raises, once, the dynamic LDS
 *   limit of the kernel that serves it (a host-side attribute; its failure is reported as LD_ERR_HIP). */
int32_t ld_head_projection(int32_t m, int32_t heads, int32_t n, int32_t k, const void* a, const void* w, void* c,
                           int32_t out_dtype, void* stream);

/* Host check of the metadata: 0 <= seq_lens[b] <= max_pages_per_seq*page_size
 * and every block_table entry a sequence uses lies in [0, num_pages).
 * LD_OK or LD_ERR_BAD_METADATA (or a pointer/shape error). */
int32_t ld_validate_metadata(const ld_problem* p, const int32_t* block_table_host, const int32_t* seq_lens_host);

/* Host copy of the split-KV planner ld_latent_decode runs on the device, for
 * tests and for callers that plan on the host.  Given the problem, host
 * seq_lens and the number of compute units, writes the chunk length (tokens,
 * a multiple of page_size, at most 512 pages) and, for every sequence, its split count and the
 * index of its first work unit.  Returns the number of work units via
 * *num_units.  splits_out and first_unit_out are int32 [batch]. */
int32_t ld_plan_host(const ld_problem* p, const int32_t* seq_lens_host, int32_t num_cus, int32_t* chunk_out,
                     int32_t* num_units, int32_t* splits_out, int32_t* first_unit_out);

#ifdef __cplusplus
}
#endif

#endif /* LATENT_DECODE_H */
