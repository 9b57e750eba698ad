// fi_internal.h -- types shared by the host runtime (plan.cpp, api.cpp) and
// the gfx950 kernels.  No HIP headers here: plan.cpp compiles with plain g++.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fi {

// the kernels are built for head_dim 64, 128 and 256
constexpr int kMaxGroup = 16;      // q heads per kv head one MFMA column tile holds
constexpr int kBlockTokens = 32;   // tokens per cascade-prefix step
constexpr int kChunkAlign = 16;    // decode chunks are whole 16-token steps
constexpr int kWavesPerTile = 8;   // waves (= kv heads) per decode workgroup
constexpr int kPrefixRowsPerWave = 32;   // 2 MFMA column tiles per wave
// query rows per wave of the multi-row kernel at head_dim D: two 16-row
// column tiles, one at D = 256 or with RoPE (registers)
constexpr int prefix_rows_per_wave(int D, bool rope = false) {
  return D == 256 || rope ? 16 : kPrefixRowsPerWave;
}
constexpr int kPrefixMaxWaves = 8;       // prefix workgroup: 4 or 8 waves
constexpr int kPrefixMaxChunk = 4096;    // prefix tokens per tile (page table in LDS)
constexpr int kMaxMergeStates = 64;
constexpr int kMaxLevels = 8;            // shared cascade levels
// bf16 P.V rounds p to 8 bits; over fewer keys than this (all of them of
// comparable weight, nothing else in the row) that rounding alone can move
// o past 2e-3 + 1e-2 |o|, so such prefixes take p with a bf16 residual
constexpr int kSplitPKeys = 256;
// RoPE with fp16 q: a key turned by its distance and rounded once to fp16
// moves a score by ~2^-12 relative per element; over a single key that alone
// reaches ~0.85e-3 in lse (CPU simulation, 8,000 rows), so plans whose
// shortest request has fewer keys than this keep the turned key's residual
constexpr int kRopeSingleKeys = 64;

enum TileKind : int32_t { kDecodeTile = 0, kPrefixTile = 1, kAppendTile = 2 };

// One entry of the work list (32 bytes, one workgroup each).
//   decode tile: request `req`, kv heads [kv_head0, kv_head0 + waves), tokens
//     [t0, t1) of the request's own pages; slot = partial-state slot of
//     kv_head0 (wave w writes slot + w) or -1 when the tile's states are final.
//   prefix tile: group `req`, kv head kv_head0, prefix tokens [t0, t1), q rows
//     [row0, row1) of the group (row = (r - first request) * G + j % G);
//     slot = the prefix chunk index.
// Work-list entry.  Decode tiles: row0 = kv_indptr[req] (the request's
// first page-table entry, known to the plan); row1 = number of earlier
// states (the request's cascade prefix chunks, slots slot_base + c * Hkv + h
// of its ReqInfo) the tile folds into its final output, 0 if none (then
// slot = -1 means the tile's own state is final).  Prefix tiles: query rows
// [row0, row1) of the group's G-row-per-request numbering.  Append tiles
// (the same multi-row kernel): request `req`, kv head kv_head0, keys
// [t0, t1) of the request, query rows [row0, row1) of its n query tokens
// (row = token * G + head in the group), slot = the key chunk index.
struct Tile {
  int32_t req, kv_head0, t0, t1, slot, kind, row0, row1;
};
static_assert(sizeof(Tile) == 32, "tile is 32 bytes");

// Per output row group (a request in decode and cascade plans, a query
// token in append plans): its partial states are slots slot_base + c * Hkv
// + h, for state index c in [0, n_states) (prefix chunks first) and kv head
// h.  n_states <= 1 means the producing tile writes the final output.
// kv_len: keys the query attends (its position + 1; the RoPE query
// position is kv_len - 1; append: the causal limit).
struct ReqInfo {
  int32_t slot_base, n_states;
  int32_t kv_len, pad;
};
static_assert(sizeof(ReqInfo) == 16, "request info is 16 bytes");

// RoPE table: for distance d < rows and frequency i < D / 2, the fp32 pair
// (cos, sin) of d / scale * theta^(-2 i / D); a row is D / 2 pairs.  Plans
// whose turned keys are one fp16 value keep fp16 rows (D / 2 cosines, then
// D / 2 sines: half as many bytes) in the same space.
constexpr int rope_row_bytes(int D) { return D / 2 * 8; }

// One merge work item: request r's states slot_base + c * Hkv + h,
// c < n_states (16 bytes, read with one load).
struct MergeUnit {
  int32_t req, slot_base, n_states, pad;
};

// Device workspace layout (byte offsets from the workspace base).
struct WorkspaceLayout {
  size_t tiles_off;        // Tile[num_tiles] then Tile[num_prefix_tiles]
  size_t req_info_off;     // ReqInfo[batch]
  size_t merge_reqs_off;   // MergeUnit[num_merge_units]
  size_t qo_indptr_off;    // int32[qo_len]: cascade group starts or append query starts
  size_t state_off_off;    // int32[num_levels * batch] (levels >= 2)
  size_t rope_qpos_off;    // int32[num_rope_qpos] (RoPE cascade / append plans)
  size_t partial_o_off;    // float[num_partials][G][D]
  size_t partial_lse_off;  // float[num_partials][G]   (log2 domain)
  size_t rope_off;         // float2[rope_rows][D / 2] (RoPE plans)
  size_t total;
};

// Host plan (built by plan.cpp, uploaded by api.cpp).
struct HostPlan {
  int32_t batch, Hq, Hkv, D, page_size, G;
  int32_t q_dtype, kv_dtype;
  int32_t num_groups;
  int32_t num_cus;
  int32_t chunk_tokens, prefix_chunk_tokens, heads_per_tile, prefix_waves;
  int64_t num_tiles, num_prefix_tiles, num_partials, num_merge_units;
  int64_t num_folded;   // requests whose decode tile folds in their prefix states
  int32_t append;       // append plan: multi-token queries over each request's keys
  int32_t merge_wide;   // many merge units with few states: the wide merge kernel
  int32_t ragged;       // ragged KV layout
  int32_t hnd;          // HND pages
  int32_t causal;       // append: causal mask
  int32_t has_keys;     // some request has kv_len > 0 (its own pages)
  int64_t total_q;      // append: query tokens (rows of o)
  int64_t num_req_info; // ReqInfo entries (batch, or total_q for append)
  int32_t qo_len;       // qo_indptr entries (levels' groups + 1 each, or batch + 1)
  // shared cascade levels, outermost first: level l's group starts are
  // qo_indptr[level_qo_start[l] ..], its prefix tiles are prefix tiles
  // level_tile_off[l] .. level_tile_off[l + 1] - 1, and a request's states
  // from it start at state index state_off[l * batch + r] (levels >= 2 only)
  int32_t num_levels;
  int32_t level_groups[kMaxLevels];
  int32_t level_qo_start[kMaxLevels];
  int64_t level_tile_off[kMaxLevels + 1];
  int32_t* state_off;   // num_levels * batch entries when num_levels >= 2
  int32_t decode_depth; // 0: the launcher's choice per instance; 1 or 2 forced
  // bf16 cascade prefix launches whose p goes to P.V as a bf16 high part
  // plus a residual (bit l set: level l has a prefix chunk shorter than
  // kSplitPKeys keys)
  uint32_t prefix_split_p;
  int32_t rope_single;  // RoPE, fp16 q or bf16 q over e4m3 K/V (fp16 compute): the
                        // turned key rounded once (no residual)
  int32_t decode_waves_per_cu;  // the decode wave target the chunking used
  int32_t valu_heads;   // plain decode on the VALU instance for this many q heads per
                        // kv head (1, 2 or 4), 0 = MFMA
  int32_t rope;         // FI_POS_ROPE_LLAMA or 0
  int32_t rope_rows;    // positions in the RoPE table (longest key list)
  // RoPE cascade / append plans: the position each query row is turned by
  // in the multi-row kernel, relative to the start of the key list its tile
  // reads -- cascade: [level * batch + request] = (the request's keys over
  // all levels - 1) - (keys of its earlier levels); append: [query token] =
  // its position in the request
  int32_t* rope_qpos;
  int64_t num_rope_qpos;
  float rope_theta, rope_scale;
  Tile* tiles;          // num_tiles + num_prefix_tiles entries
  ReqInfo* req_info;    // batch entries
  MergeUnit* merge_units;  // num_merge_units entries
  int32_t* qo_indptr;   // qo_len entries (cascade group starts / append query starts)
  WorkspaceLayout layout;
};

// Plan tuning: every field 0 selects the built-in default (the measured
// best); other values only change how the work is cut, never the result.
struct Tuning {
  int32_t heads_per_tile;       // kv heads per decode workgroup (1, 2, 4, 8)
  int32_t waves_per_cu;         // decode waves the chunk search targets per CU (16)
  int32_t chunk_min;            // smallest decode chunk in tokens (32)
  int32_t prefix_waves;         // waves per multi-row tile, 4 or 8
  int32_t prefix_tiles_per_cu;  // cascade prefix tiles per CU (1)
  int32_t prefix_chunk_min;     // smallest cascade prefix chunk in tokens (256)
  int32_t cascade_fold;         // 1 fold one-chunk suffixes (default), -1 never
  int32_t fold_max_suffix;      // longest suffix one fold chunk covers (1024)
  int32_t append_tiles_pct;     // append tiles per resident workgroup x 100 (125)
  int32_t append_chunk_min;     // smallest append key chunk in tokens (128)
  int32_t decode_depth;         // steps of K/V loads in flight, 1 or 2 (per instance)
  int32_t prefix_split_p;       // bf16 cascade prefix: 1 always split p, -1 never
  int32_t rope_split_k;         // RoPE, fp16 q: 1 always split the turned key, -1 never
  int32_t score_path;           // plain decode: 1 MFMA scores and P.V, 2 VALU (G <= 4, D 128)
};

// Builds the plan on the host.  Returns 0 or an fi_status code with `err`
// filled.  Memory of the arrays is malloc'ed; free with plan_free.
struct PlanInput {
  int32_t batch, Hq, Hkv, D, page_size;
  int32_t q_dtype, kv_dtype;
  const int32_t* kv_indptr;
  const int32_t* last_page_len;
  // shared cascade levels, outermost first (host tables)
  int32_t num_levels;
  struct Level {
    int32_t num_groups;
    const int32_t* qo_indptr;   // groups of contiguous requests
    const int32_t* p_indptr;
    const int32_t* p_last;
  } levels[kMaxLevels];
  int32_t chunk_tokens;
  int32_t num_cus;
  int32_t pos_encoding;
  float rope_theta, rope_scale;
  const int32_t* append_qo_indptr;   // host [batch + 1] or NULL (decode)
  int32_t causal;
  int32_t ragged;   // rows kv_indptr[r] + t, no page indices
  int32_t hnd;      // pages head-major: [page][Hkv][page_size][D]
  Tuning tune;
  // Waves per compute unit that the decode instance of a plan with these
  // arguments holds at once, for tiles of hpt kv heads (rope_form: 0 none,
  // 1 turned key as high part + residual, 2 as one fp16 value; fold: the
  // cascade fold instance), or 0 when unknown (no device): the default
  // decode wave target is min(16, this).  NULL: unknown.
  int (*resident_waves)(const void* ctx, int hpt, int rope_form, int fold) = nullptr;
  const void* resident_ctx = nullptr;
};
int plan_build(const PlanInput& in, HostPlan* out, char* err, size_t errlen);
void plan_free(HostPlan* p);
// Plain decode without host arrays or allocation: validates, picks the same
// split as plan_build (longer chunks when the partial states would not fit
// in max_bytes and chunk_tokens is 0) and fills the plan's sizes and a
// layout of at most max_bytes; the work list itself is written on the device
// (launch_device_plan).  tiles / req_info / merge_units stay NULL.
int plan_decode_static(const PlanInput& in, size_t max_bytes, HostPlan* out, char* err,
                       size_t errlen);

// ---- kernel parameter blocks (passed by value) ----------------------------
struct DecodeParams {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  const int32_t* kv_indptr;   // page table the tile tokens index (device)
  const int32_t* kv_indices;
  const float* k_scale;
  const float* v_scale;
  const Tile* tiles;
  const ReqInfo* req_info;
  float* partial_o;
  float* partial_lse;
  void* o;
  float* lse;
  float sm_scale_log2;        // sm_scale * log2(e)
  int32_t Hq, Hkv, G, page_size, ps_shift;  // ps_shift = log2(ps) or -1
  int32_t num_tiles;
  // prefix tiles only: first request of each group, device [groups+1]
  const int32_t* qo_indptr;
  // RoPE plans: the (cos, sin) table, rope_rows x D / 2 fp32 pairs
  const void* rope_table;
  int32_t rope_rows;
  int32_t rope_single;        // fp16 q or bf16 q over e4m3: turned keys as one fp16 value
  int32_t valu_heads;         // > 0: the VALU decode instance (q heads per kv head)
  // ragged KV: token t of a request is row kv_indptr[r] + t (page size 1,
  // kv_indices not read)
  int32_t ragged;
  // prefix tiles of a cascade with several levels: request r's states from
  // this level start at state index state_off[r] (NULL: 0)
  const int32_t* state_off;
  // RoPE multi-row tiles: the position query rows of request (cascade) or
  // query token (append) i are turned by, rope_qpos[i]
  const int32_t* rope_qpos;
  // K/V row of (page, slot, kv head) at page * page_bytes + slot *
  // slot_stride + head * head_stride bytes: NHD pages (slot_stride = Hkv
  // rows, head_stride = 1 row) or HND pages (slot_stride = 1 row,
  // head_stride = page_size rows)
  uint32_t page_bytes, slot_stride, head_stride;
  // test instances only: the byte offset of every K vector load, indexed by
  // (rec_base[request or group] + token, kv head, 16-byte chunk)
  int64_t* rec;
  const int64_t* rec_base;
};

struct MergeParams {
  const float* partial_o;
  const float* partial_lse;
  const MergeUnit* units;
  void* o;
  float* lse;
  int32_t Hq, Hkv, G;
  int32_t out_dtype;
};

struct MergeStatesParams {
  const void* v[kMaxMergeStates];
  const float* s[kMaxMergeStates];
  int32_t num_states;
  int64_t num_rows;
  int32_t head_dim;
  int32_t v_dtype, out_dtype;
  void* v_out;
  float* s_out;
};

}  // namespace fi
