/*
 * fi_decode.h -- C ABI of the MI355X (gfx950) paged-KV decode attention
 * library (libfi_decode.so).
 *
 * The operation (FlashInfer README, "core features" items 1-3; hysenlabs
 * review, "Installing FlashInfer and running a first decode"; flash-attention
 * summary, "How it works"):
 *   for every request r and query head j, one query token q[r][j][:] attends
 *   over that request's keys with exact attention
 *       x_t = sm_scale * q . k_t,
 *       o   = sum_t softmax(x)_t * v_t,
 *       lse = ln sum_t exp(x_t)          (natural log),
 *   where q head j reads kv head j / G (G = num_qo_heads / num_kv_heads,
 *   grouped-query heads fused so each K/V row is read once per kv head), and
 *   the keys of request r are reached through a page table (the kv_indptr /
 *   kv_indices / last_page_len vocabulary of the "Pre-compiled cubins for
 *   FlashInfer" registry quickstart):
 *       n_r = kv_indptr[r+1] - kv_indptr[r] pages,
 *       kv_len_r = n_r == 0 ? 0 : (n_r - 1) * page_size + last_page_len[r],
 *       logical token t lives in page kv_indices[kv_indptr[r] + t / page_size]
 *       at slot t % page_size.
 *   An empty request yields o = 0 and lse = -inf.
 *
 * Layouts (all row-major, all device pointers unless marked host):
 *   q, o          [batch][num_qo_heads][head_dim], dtype q_dtype (o = q dtype)
 *                 (append plans: [total_q][num_qo_heads][head_dim])
 *   lse           [batch][num_qo_heads] fp32 (may be NULL)
 *   k_pages,
 *   v_pages       [num_pages][page_size][num_kv_heads][head_dim] ("NHD"),
 *                 dtype kv_dtype; separate K and V pools (fi_problem's
 *                 kv_layout also selects head-major "HND" pages or the
 *                 ragged layout)
 *   k_scale,
 *   v_scale       [num_kv_heads] fp32 for E4M3 KV (dequantised value =
 *                 decode(code) * scale[kv_head]; NULL means 1.0), ignored
 *                 for fp16/bf16 KV
 *
 * Plan / run (FlashInfer README, "core features" item 2: the plan stage
 * schedules variable-length work on the host to balance load; the run stage
 * executes it): fi_plan() turns the host-side lengths into a work list of
 * (request, kv head, token chunk) tiles and uploads it into a caller-owned
 * device workspace; fi_decode_run() / fi_cascade_decode() / fi_append_run()
 * then only enqueue kernels on the caller's stream -- no allocation, no
 * synchronisation, no host reads -- so they may be captured into a hipGraph
 * (README "core features" item 5).  Re-plan whenever kv_indptr or last_page_len change;
 * kv_indices contents and K/V data may change freely between runs.
 *
 * Ownership: the caller owns every device buffer and the stream.  The
 * library owns the plan object (host memory), released by fi_plan_destroy(),
 * and a small process-wide pool of pinned host buffers through which
 * fi_plan() uploads work lists: a buffer is reused by a later fi_plan() once
 * the upload that last used it has completed (checked with an event), so a
 * re-planning loop allocates no pinned memory after its first plans.
 *
 * Errors: every call returns an fi_status; nothing aborts, throws or prints
 * across the ABI.  Arguments are validated on the host before anything is
 * enqueued; on error nothing is launched and outputs are untouched, and
 * fi_last_error() returns a thread-local message.  Device-resident indices
 * (kv_indices, and the device copies of kv_indptr / last_page_len) are
 * trusted: they must describe the same tables that were planned.
 *
 * Supported: head_dim 64, 128 or 256; q in fp16 or bf16;
 * KV in the q dtype or OCP E4M3 (e4m3fn); 1 <= num_qo_heads / num_kv_heads
 * <= 16; any page_size >= 1; LLaMA-style RoPE on the fly (decode, cascade
 * levels and append); batch append (causal or not) on the same page tables.
 */
#ifndef FI_DECODE_H_
#define FI_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FI_OK = 0,
  FI_ERR_INVALID_ARG = 1,         /* bad pointer, shape or table */
  FI_ERR_UNSUPPORTED = 2,         /* valid but not built (dtype, head_dim, G) */
  FI_ERR_WORKSPACE_TOO_SMALL = 3, /* *workspace_needed says how much */
  FI_ERR_HIP = 4                  /* a HIP runtime call failed */
} fi_status;

typedef enum {
  FI_F16 = 0,
  FI_BF16 = 1,
  FI_E4M3 = 2, /* OCP 8-bit E4M3FN: bias 7, max 448, S.1111.111 = NaN */
  FI_F32 = 3
} fi_dtype;

/* One shared cascade level (host tables): num_groups groups of CONTIGUOUS
 * requests, group g = requests [qo_indptr[g], qo_indptr[g+1]) sharing the
 * prefix table kv_indptr[g] .. (pages as the per-request table, or rows in
 * the ragged layout) with last_page_len[g]. */
typedef struct {
  int32_t num_groups;
  const int32_t* qo_indptr;       /* host [num_groups+1], [0] = 0, [num_groups] = B */
  const int32_t* kv_indptr;       /* host [num_groups+1] */
  const int32_t* last_page_len;   /* host [num_groups] (NULL when ragged) */
} fi_cascade_level;

/* Plan tuning, for measurement: how the work is cut, never what is
 * computed.  A field left 0 takes the built-in default (the measured best);
 * fi_problem.tuning == NULL leaves every field at its default.  The library
 * reads no environment variable. */
typedef struct {
  int32_t heads_per_tile;       /* kv heads per decode workgroup: 1, 2, 4 or 8 */
  int32_t waves_per_cu;         /* decode waves the chunk search targets per CU
                                   (default: 16, or fewer when fi_plan finds the
                                   device keeps fewer of the decode kernel it
                                   will launch resident; one round of them, or
                                   two when the lengths are skewed) */
  int32_t chunk_min;            /* smallest decode chunk, tokens (32) */
  int32_t prefix_waves;         /* waves per multi-row tile: 4 or 8 (RoPE: 8) */
  int32_t prefix_tiles_per_cu;  /* cascade prefix tiles per CU (1) */
  int32_t prefix_chunk_min;     /* smallest cascade prefix chunk, tokens (256) */
  int32_t cascade_fold;         /* 0/1: a one-chunk suffix tile folds its prefix
                                   states in; -1: every cascade request goes
                                   through the merge kernel */
  int32_t fold_max_suffix;      /* longest suffix one fold chunk covers (1024) */
  int32_t append_tiles_pct;     /* append tiles per resident workgroup x 100 (125) */
  int32_t append_chunk_min;     /* smallest append key chunk, tokens (128) */
  int32_t decode_depth;         /* steps of K/V loads in flight: 0 = per kernel
                                   instance, 1, or 2 where built */
  int32_t prefix_split_p;       /* bf16 cascade prefix launches pass p to P.V
                                   with a bf16 residual: 0 = when a level has a
                                   prefix under 256 keys, 1 = always, -1 = never */
  int32_t rope_split_k;         /* RoPE with fp16 q: a key turned by its distance
                                   goes to the score as a high part plus a
                                   residual: 0 = when some request has fewer
                                   than 64 keys, 1 = always, -1 = never (one
                                   fp16 value, turned in packed fp16 against
                                   an fp16 table); bf16 q, and tiles of fewer
                                   than head_dim / 32 kv heads, always split */
  int32_t score_path;           /* plain decode: 0 = automatic (MFMA), 1 = MFMA
                                   for q.K^T and P.V, 2 = VALU dot products and
                                   FMAs (head_dim 128, <= 4 q heads per kv
                                   head; else FI_ERR_UNSUPPORTED) */
} fi_tuning;

/* Problem description; every pointer here is HOST memory, read during the
 * fi_plan() call only. */
typedef struct {
  int32_t batch;          /* number of requests B >= 0 */
  int32_t num_qo_heads;   /* Hq */
  int32_t num_kv_heads;   /* Hkv, divides Hq */
  int32_t head_dim;       /* D: 64, 128 or 256 */
  int32_t page_size;      /* tokens per page, >= 1 */
  fi_dtype q_dtype;       /* FI_F16 or FI_BF16; o has this dtype */
  fi_dtype kv_dtype;      /* q_dtype or FI_E4M3 */
  const int32_t* kv_indptr;     /* host [B+1], non-decreasing, [0] = 0 */
  const int32_t* last_page_len; /* host [B], in [1, page_size] for non-empty */
  /* Optional cascade level (FlashInfer README "core features" item 3 and the
   * "Cascade Inference: shared prefix batch decoding" news item): requests
   * are split into num_prefix_groups groups of CONTIGUOUS requests; group g
   * = requests [prefix_qo_indptr[g], prefix_qo_indptr[g+1]) shares the prefix
   * pages prefix_kv_indices[prefix_kv_indptr[g] ..) that precede each
   * request's own pages.  0 groups = plain decode. */
  int32_t num_prefix_groups;
  const int32_t* prefix_qo_indptr;     /* host [groups+1], [0]=0, [groups]=B */
  const int32_t* prefix_kv_indptr;     /* host [groups+1] */
  const int32_t* prefix_last_page_len; /* host [groups] */
  /* Tuning knob: tokens per split chunk (multiple of 16), 0 = automatic. */
  int32_t chunk_tokens;
  /* Position encoding (FlashInfer README decode example, pos_encoding_mode;
   * "core features" item 3, fused RoPE): FI_POS_NONE (0) or
   * FI_POS_ROPE_LLAMA, LLaMA-style RoPE applied on the fly to q and to the
   * cached (unrotated) keys: rotate-half over head_dim, the pair
   * (x_i, x_{i+D/2}) turned by angle_i = pos / rope_scale *
   * rope_theta^(-2 i / D); key t of a request's key list sits at position
   * t (with cascade levels: the groups' prefixes, outermost first, then the
   * request's own keys), the query at (number of keys) - 1; append query i
   * of n at kv_len - n + i.  A cascade plan with RoPE merges its prefix
   * states in a separate pass (no fold). */
  int32_t pos_encoding;
  float rope_theta;       /* <= 0: 1e4 */
  float rope_scale;       /* <= 0: 1 */
  /* Append mode (FlashInfer README append example:
   * single_prefill_with_kv_cache(q, k, v, causal=True), its queries being
   * the newest 128 tokens of the KV cache; batch form over qo_indptr):
   * qo_indptr != NULL gives request r the query tokens
   * [qo_indptr[r], qo_indptr[r+1]) of q [total_q][Hq][D], which are the LAST
   * n_r = qo_indptr[r+1] - qo_indptr[r] <= kv_len_r tokens of its keys:
   * query i sits at position kv_len_r - n_r + i and, with causal != 0,
   * attends keys 0 .. kv_len_r - n_r + i (all kv_len_r keys otherwise).
   * Run with fi_append_run.  Not combined with a cascade level
   * (FI_ERR_UNSUPPORTED); RoPE applies (above).  NULL = decode (one query
   * per request). */
  const int32_t* qo_indptr;   /* host [B+1], [0] = 0, non-decreasing, or NULL */
  int32_t causal;
  /* KV layout (README "core features" item 1: paged and ragged KV cache):
   * FI_KV_PAGED (0): NHD pages reached through kv_indptr / kv_indices /
   * last_page_len as described above.  FI_KV_RAGGED (1): each request's
   * tokens are contiguous rows kv_indptr[r] .. kv_indptr[r+1]-1 of K and V
   * [total_tokens][Hkv][D] (kv_indptr counts rows and need not start at 0;
   * page_size must be 1; last_page_len and the run calls' kv_indices /
   * last_page_len may be NULL).  A cascade level's prefix tables follow the
   * same layout, in the same K and V arrays.  FI_KV_PAGED_HND (2): pages as
   * FI_KV_PAGED but head-major, [num_pages][Hkv][page_size][D] (the other
   * value of the registry quickstart's kv_layout argument). */
  int32_t kv_layout;
  /* Several shared cascade levels (README "core features" item 3: cascade
   * attention over a hierarchical KV cache), outermost first: request r
   * attends over its group's prefix at every level in order, then its own
   * pages.  Give either these (num_prefix_groups = 0) or the single-level
   * fields above; run with fi_cascade_decode_levels.  At most 8 levels. */
  int32_t num_cascade_levels;
  const fi_cascade_level* cascade_levels;   /* host [num_cascade_levels] */
  /* Optional plan tuning (NULL: defaults). */
  const fi_tuning* tuning;
} fi_problem;

enum { FI_POS_NONE = 0, FI_POS_ROPE_LLAMA = 1 };
enum { FI_KV_PAGED = 0, FI_KV_RAGGED = 1, FI_KV_PAGED_HND = 2 };

typedef struct fi_plan_s* fi_plan_t;

/* Plan statistics, for tests and benchmarks. */
typedef struct {
  int64_t num_tiles;         /* decode work-list entries (workgroups) */
  int64_t num_prefix_tiles;  /* multi-row work-list entries (cascade prefix
                                tiles, or the tiles of an append plan) */
  int64_t num_partials;      /* partial (o, lse) states written by tiles */
  int64_t num_merge_units;   /* requests whose states are merged */
  int32_t chunk_tokens;      /* split chunk chosen (tokens) */
  int32_t prefix_chunk_tokens;
  int32_t heads_per_tile;    /* kv heads one decode workgroup handles */
  int32_t num_cus;
  size_t workspace_bytes;
  int64_t num_folded;        /* cascade requests whose one suffix tile folds in
                                their prefix states (no merge unit) */
  uint32_t prefix_split_p;   /* bit l: level l's prefix launch passes p with a
                                bf16 residual */
  int32_t staging_buffers;   /* pinned upload buffers the library holds for
                                all plans of the process (reused, not per plan) */
  int32_t rope_single;       /* RoPE plan whose turned keys are one fp16 value */
  int32_t valu_heads;        /* > 0: plain decode on the VALU (no MFMA) kernel */
  int32_t decode_waves_per_cu; /* decode waves per CU the chunking targeted: the
                                tuning's, else 16 or, when fewer, what the
                                current device keeps resident of the decode
                                kernel the run launches (16 without a device) */
} fi_plan_stats;

/* Plan stage (FlashInfer README "core features" item 2).
 * problem:        host description above.
 * num_cus:        compute units to balance for; 0 = query the current device.
 * workspace:      device buffer the plan's work list, merge map and partial
 *                 states live in; NULL = only report the size needed.
 * workspace_bytes: its size.
 * workspace_needed: out (may be NULL): bytes the plan needs.
 * stream:         hipStream_t the work list is uploaded on (NULL = default).
 * plan_out:       out: the plan (NULL when workspace is NULL).
 * Returns FI_ERR_WORKSPACE_TOO_SMALL (and sets *workspace_needed) when the
 * workspace is too small.  The workspace must stay allocated and untouched
 * by the caller while the plan is in use. */
fi_status fi_plan(const fi_problem* problem, int32_t num_cus, void* workspace,
                  size_t workspace_bytes, size_t* workspace_needed,
                  void* stream, fi_plan_t* plan_out);

/* Releases a plan (host memory only; the workspace stays the caller's). */
fi_status fi_plan_destroy(fi_plan_t plan);

/* Fills *stats (host) for a plan. */
fi_status fi_plan_get_stats(fi_plan_t plan, fi_plan_stats* stats);

/* Run stage: batch paged decode (FlashInfer README "core features" items 1
 * and 3: paged / vector-sparse attention, head-query fusion for GQA,
 * low-precision KV).  The plan must have been made without a cascade level.
 * kv_indptr, kv_indices, last_page_len are DEVICE copies of the planned
 * table.  sm_scale <= 0 selects 1/sqrt(head_dim).  lse may be NULL; when
 * every planned kv_len is 0, kv_indices, k_pages and v_pages may be NULL
 * (nothing is read; every row gets o = 0, lse = -inf).
 * Enqueues 1-2 kernels on stream. */
fi_status fi_decode_run(fi_plan_t plan, const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* kv_indptr,
                        const int32_t* kv_indices,
                        const int32_t* last_page_len, const float* k_scale,
                        const float* v_scale, float sm_scale, void* o,
                        float* lse, void* stream);

/* Run stage: cascade decode (README "core features" item 3, Cascade
 * Attention for a hierarchical KV cache): every request attends over its
 * group's shared prefix pages followed by its own pages; the prefix is read
 * once per (group, kv head) for all the group's query rows and the two
 * attention states are merged: by the request's suffix tile when its suffix
 * is one planned chunk, else by a merge pass.  The plan must have been made
 * with the same cascade level.  prefix_* and kv_* are DEVICE copies of the
 * planned tables.  Enqueues 2-3 kernels on stream (prefix, suffix, and a
 * merge when some request needs one). */
fi_status fi_cascade_decode(fi_plan_t plan, const void* q, const void* k_pages,
                            const void* v_pages,
                            const int32_t* prefix_kv_indptr,
                            const int32_t* prefix_kv_indices,
                            const int32_t* prefix_last_page_len,
                            const int32_t* kv_indptr,
                            const int32_t* kv_indices,
                            const int32_t* last_page_len,
                            const float* k_scale, const float* v_scale,
                            float sm_scale, void* o, float* lse, void* stream);

/* Run stage: cascade decode with the plan's num_levels shared levels
 * (fi_problem.cascade_levels, outermost first): level l's prefix tiles read
 * DEVICE tables level_kv_indptr[l] / level_kv_indices[l] /
 * level_last_page_len[l] (the three arrays are HOST arrays of num_levels
 * device pointers); the states of every level and of the request's own
 * pages are merged (folded into a one-chunk suffix tile, or by the merge
 * pass).  Enqueues one prefix kernel per level with tiles, the suffix
 * decode and the merge; capturable.  Errors as fi_cascade_decode, plus
 * FI_ERR_INVALID_ARG when num_levels differs from the plan's. */
fi_status fi_cascade_decode_levels(fi_plan_t plan, const void* q, const void* k_pages,
                                   const void* v_pages, int32_t num_levels,
                                   const int32_t* const* level_kv_indptr,
                                   const int32_t* const* level_kv_indices,
                                   const int32_t* const* level_last_page_len,
                                   const int32_t* kv_indptr, const int32_t* kv_indices,
                                   const int32_t* last_page_len, const float* k_scale,
                                   const float* v_scale, float sm_scale, void* o, float* lse,
                                   void* stream);

/* Run stage: batch append attention (README append example; see
 * fi_problem.qo_indptr): every query token of request r attends over r's
 * pages up to its causal limit (all of them without the mask).  The query
 * rows (token, q head) of one (request, kv head) are processed in 256-row
 * MFMA tiles over key chunks; tokens whose keys span several chunks are
 * merged by a merge pass.  The plan must have been made in append mode.
 * q: DEVICE [total_q][Hq][D] (q_dtype), o: DEVICE [total_q][Hq][D] (q_dtype),
 * lse: DEVICE [total_q][Hq] fp32 natural log, or NULL; kv_* are DEVICE
 * copies of the planned tables; k_scale / v_scale as fi_decode_run.
 * Enqueues 1-2 kernels on stream; capturable.  Errors: FI_ERR_INVALID_ARG
 * for a NULL plan / required pointer, non-finite sm_scale or a plan not made
 * in append mode. */
fi_status fi_append_run(fi_plan_t plan, const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* kv_indptr,
                        const int32_t* kv_indices, const int32_t* last_page_len,
                        const float* k_scale, const float* v_scale, float sm_scale,
                        void* o, float* lse, void* stream);

/* Plain batch decode for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): fi_plan + fi_decode_run in one call, with no workspace.  The
 * work list, merge map and fp32 partial states live in a static device
 * array of the library (32 MiB per GPU, held until the process ends); the
 * call allocates nothing -- no hipMalloc, no pinned or other host buffer --
 * and copies nothing from the host: a planner kernel derives the work list
 * from the device tables.
 * problem:  as for fi_plan (its host kv_indptr / last_page_len decide the
 *           split; the device copies must describe the same table); plain
 *           decode only -- no cascade level, append or RoPE
 *           (FI_ERR_UNSUPPORTED).  chunk_tokens 0 picks fi_plan's split, or
 *           longer chunks when its partial states would not fit the static
 *           array; a forced chunk_tokens whose states do not fit, or a batch
 *           whose work list alone does not, is FI_ERR_INVALID_ARG with the
 *           bytes needed in fi_last_error(), before anything is enqueued.
 * Other arguments as fi_decode_run.  Enqueues 2-3 kernels on stream
 * (planner, decode, merge when some request is split); capturable.  Every
 * call on one GPU shares that GPU's array: calls that overlap on a GPU (two
 * streams or threads) race and must be serialised by the caller. */
fi_status fi_decode_noalloc(const fi_problem* problem, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* kv_indptr,
                           const int32_t* kv_indices, const int32_t* last_page_len,
                           const float* k_scale, const float* v_scale, float sm_scale,
                           void* o, float* lse, void* stream);

/* Merge of attention states computed over DISJOINT key sets of the same
 * query rows (the split-KV / cascade recombination): with
 * M = max_i s_i, s = M + ln sum_i exp(s_i - M), v = sum_i exp(s_i - s) * v_i;
 * all s_i = -inf gives v = 0, s = -inf.
 * num_states:  1..64 states.
 * v_states:    HOST array of num_states DEVICE pointers, each [num_rows][head_dim]
 *              of v_dtype (FI_F16, FI_BF16 or FI_F32).
 * s_states:    HOST array of num_states DEVICE pointers, each [num_rows] fp32
 *              natural-log lse.
 * v_out:       DEVICE [num_rows][head_dim] of out_dtype; s_out DEVICE
 *              [num_rows] fp32 (may be NULL).  Rows are e.g. batch x heads.
 * Enqueues one kernel. */
fi_status fi_merge_states(int32_t num_states, const void* const* v_states,
                          const float* const* s_states, int64_t num_rows,
                          int32_t head_dim, fi_dtype v_dtype, void* v_out,
                          float* s_out, fi_dtype out_dtype, void* stream);

/* Human-readable name of a status, and the calling thread's last error. */
const char* fi_status_string(fi_status status);
const char* fi_last_error(void);

/* ---- test hooks --------------------------------------------------------
 * fi_debug_plan_tiles: runs the plan scheduler on the host only (no device
 * touched) and copies the decode work list into tiles_out (host, int32,
 * 8 words per tile: request, first kv head, t0, t1, partial slot base or -1,
 * kind, row0, row1); *num_tiles = entries.  If capacity_tiles is too small
 * only the count is returned.  prefix tiles follow the decode tiles.  For a
 * decode tile row0 is kv_indptr[request] (its page-table base); for a prefix
 * tile [row0, row1) is its range of the group's query rows. */
fi_status fi_debug_plan_tiles(const fi_problem* problem, int32_t num_cus,
                              int32_t* tiles_out, int64_t capacity_tiles,
                              int64_t* num_tiles);

/* fi_debug_gather: for every logical token of every request (request-major)
 * writes its physical token slot page * page_size + slot to out_slots
 * (device int64 [total tokens]): a plain per-token page-table lookup, the
 * reference point of the page-table reading (registry quickstart's
 * kv_indptr / kv_indices / last_page_len).  The kernels' own page walks are
 * checked by fi_debug_record_walk.  token_indptr: device [batch+1]
 * exclusive scan of kv_len. */
fi_status fi_debug_gather(int32_t batch, int32_t page_size,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          const int32_t* last_page_len,
                          const int64_t* token_indptr, int64_t* out_slots,
                          void* stream);

/* fi_debug_run_stage: enqueues ONE kernel of a planned run, with the launch
 * configuration the full run uses, so that kernel can be timed or checked
 * on its own.  Arguments as fi_cascade_decode; for a plan without a cascade
 * level the three prefix tables may be NULL.  stage 0 = the decode kernel
 * over the per-request pages, stage 1 = the cascade prefix kernel (plans
 * with prefix tiles only; for an append plan, its multi-row kernel over the
 * per-request pages), stage 2 = the merge of split requests' states
 * (nothing when the plan has no merge unit).  Rows whose state is not split
 * are written to o / lse as in the full run; split rows write their partial
 * states to the workspace, which stage 2 merges into o / lse.  Stages 1, 0, 2
 * in that order are the full run.  Errors as fi_cascade_decode, plus
 * FI_ERR_INVALID_ARG for another stage. */
fi_status fi_debug_run_stage(fi_plan_t plan, int32_t stage, const void* q,
                             const void* k_pages, const void* v_pages,
                             const int32_t* prefix_kv_indptr,
                             const int32_t* prefix_kv_indices,
                             const int32_t* prefix_last_page_len,
                             const int32_t* kv_indptr, const int32_t* kv_indices,
                             const int32_t* last_page_len, const float* k_scale,
                             const float* v_scale, float sm_scale, void* o,
                             float* lse, void* stream);

/* fi_debug_record_walk: runs ONE kernel of a planned run (stage 0 = the
 * decode kernel, 1 = the cascade prefix / append kernel) exactly as the run
 * launches it -- same work list, workgroup shape and loop -- in an instance
 * whose loader additionally stores, for every K vector it loads, the byte
 * offset of that 16-byte vector within the K pool:
 *   rec[((rec_base[i] + t) * num_kv_heads + h) * (row_bytes / 16) + c]
 *     = offset of bytes 16c .. 16c+15 of the K row of logical token t,
 *       kv head h,
 * with i the tile's request (decode, append) or prefix group (cascade
 * prefix) and row_bytes = head_dim * element size.  rec (device int64) and
 * rec_base (device int64 [batch+1] or [groups+1], the token start of each
 * key list in rec) are the caller's; entries no load reaches are left as
 * they were.  Outputs are written as by fi_debug_run_stage.  So the page
 * walk (page index, slot, layout strides, chunk boundaries, tail clamp) can
 * be compared bit for bit with a plain reading of the page table (registry
 * quickstart: kv_indptr / kv_indices / last_page_len, kv_layout).
 * Built for head_dim 128 with fp16 q + fp16 K/V or bf16 q + e4m3 K/V,
 * 8-wave multi-row tiles, no RoPE; otherwise FI_ERR_UNSUPPORTED.  Plans
 * with one cascade level at most. */
fi_status fi_debug_record_walk(fi_plan_t plan, int32_t stage, const void* q,
                               const void* k_pages, const void* v_pages,
                               const int32_t* prefix_kv_indptr,
                               const int32_t* prefix_kv_indices,
                               const int32_t* prefix_last_page_len,
                               const int32_t* kv_indptr, const int32_t* kv_indices,
                               const int32_t* last_page_len, const float* k_scale,
                               const float* v_scale, float sm_scale, void* o, float* lse,
                               int64_t* rec, const int64_t* rec_base, void* stream);

/* fi_debug_stream_read: reads `bytes` (multiple of 16) of device memory at
 * src with 16-byte loads from num_blocks workgroups of 256 threads and
 * writes one folded word per thread to sink (device uint32
 * [num_blocks * 256]).  A plain streaming read: the HBM bandwidth ceiling
 * and the byte-counter calibration that decode traffic is compared to. */
fi_status fi_debug_stream_read(const void* src, size_t bytes, uint32_t* sink,
                               int32_t num_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FI_DECODE_H_ */
