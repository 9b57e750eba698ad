// api.cpp -- the extern "C" boundary of libfi_decode.so.
//
// Validates every argument on the host, then only enqueues kernels on the
// caller's stream (no allocation, no synchronisation in the run calls), so
// that fi_decode_run / fi_cascade_decode / fi_merge_states can be captured
// into a hipGraph (FlashInfer README, "core features" item 5).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "fi_decode.h"
#include "fi_internal.h"

namespace fi {
hipError_t launch_decode(const DecodeParams& p, int num_tiles, int waves, bool q_bf16,
                         int kv, bool fold, int depth, int head_dim, hipStream_t s);
hipError_t decode_occupancy(const DecodeParams& p, int waves, bool q_bf16, int kv, bool fold,
                            int depth, int head_dim, int* blocks);
hipError_t launch_prefix(const DecodeParams& p, int num_tiles, int waves, bool append,
                         bool split, bool q_bf16, int kv, int head_dim, hipStream_t s);
hipError_t launch_merge_partials(const MergeParams& p, int num_units, bool o_bf16, bool wide,
                                 int head_dim, hipStream_t s);
hipError_t launch_merge_states(const MergeStatesParams& p, hipStream_t s);
hipError_t launch_gather(const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int64_t* token_indptr, int batch, int page_size,
                         int ps_shift, int64_t* out, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s);
hipError_t launch_rope_table(void* table, int rows, int head_dim, float theta, float scale,
                             bool f16, hipStream_t s);
size_t scratch_capacity();
hipError_t scratch_address(void** out);
hipError_t launch_device_plan(const int32_t* kv_indptr, const int32_t* last_page_len,
                              int batch, int page_size, int chunk, int heads_per_tile, int Hkv,
                              void* tiles, void* req_info, void* units, int64_t tile_cap,
                              int64_t unit_cap, hipStream_t s);
}  // namespace fi

struct fi_plan_s {
  fi::HostPlan hp;
  char* workspace;
  size_t workspace_bytes;
};

namespace {

// ---- pinned upload buffers, shared by every plan of the process ------------
// fi_plan() writes the work list, request info and merge map into a pinned
// host buffer and copies it to the workspace asynchronously.  A buffer is
// taken again once the event recorded after its last copy has completed, so
// re-planning does not allocate pinned memory each time; at most kMaxStaging
// buffers per device are kept (beyond that fi_plan waits for the oldest copy).
struct Staging {
  void* ptr;
  size_t bytes;
  hipEvent_t done;   // recorded after the copy that last read the buffer
  int device;
  bool in_use;       // between acquire and the event record
  uint64_t last_use;
};
constexpr int kMaxStaging = 4;
std::mutex g_staging_mu;
std::vector<Staging> g_staging;
uint64_t g_staging_clock = 0;

// Returns a buffer of >= bytes on `device` whose previous copy is complete,
// or -1 with *err set.
int staging_acquire(size_t bytes, int device, hipError_t* err) {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  int n_dev = 0, oldest = -1;
  for (size_t i = 0; i < g_staging.size(); ++i) {
    Staging& b = g_staging[i];
    if (b.device != device) continue;
    ++n_dev;
    if (b.in_use) continue;
    if (b.bytes >= bytes && hipEventQuery(b.done) == hipSuccess) {
      b.in_use = true;
      return (int)i;
    }
    if (oldest < 0 || b.last_use < g_staging[oldest].last_use) oldest = (int)i;
  }
  if (n_dev >= kMaxStaging && oldest >= 0) {
    // reuse the least recently used buffer once its copy is done, growing it
    Staging& b = g_staging[oldest];
    hipError_t e = hipEventSynchronize(b.done);
    if (e == hipSuccess && b.bytes < bytes) {
      e = hipHostFree(b.ptr);
      b.ptr = nullptr;
      b.bytes = 0;
      if (e == hipSuccess) e = hipHostMalloc(&b.ptr, bytes, hipHostMallocDefault);
      if (e == hipSuccess) b.bytes = bytes;
    }
    if (e != hipSuccess) {
      *err = e;
      return -1;
    }
    b.in_use = true;
    return oldest;
  }
  Staging b{};
  b.device = device;
  hipError_t e = hipHostMalloc(&b.ptr, bytes, hipHostMallocDefault);
  if (e == hipSuccess) {
    e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
    if (e != hipSuccess) (void)hipHostFree(b.ptr);
  }
  if (e != hipSuccess) {
    *err = e;
    return -1;
  }
  b.bytes = bytes;
  b.in_use = true;
  g_staging.push_back(b);
  return (int)g_staging.size() - 1;
}

void* staging_ptr(int i) {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  return g_staging[i].ptr;
}

// Records the buffer's copy on `stream` and hands the buffer back; when
// `record` is false (the copy was never enqueued) it is free at once.
hipError_t staging_release(int i, hipStream_t stream, bool record) {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  Staging& b = g_staging[i];
  hipError_t e = record ? hipEventRecord(b.done, stream) : hipSuccess;
  if (e != hipSuccess) (void)hipStreamSynchronize(stream);   // copy done: free to reuse
  if (e != hipSuccess) (void)hipEventSynchronize(b.done);
  b.in_use = false;
  b.last_use = ++g_staging_clock;
  return e;
}

int staging_count() {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  return (int)g_staging.size();
}

thread_local std::string g_last_error;

fi_status fail(fi_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fi_status hip_fail(hipError_t e, const char* what) {
  return fail(FI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int ps_shift_of(int ps) {
  if (ps <= 0 || (ps & (ps - 1))) return -1;
  int s = 0;
  while ((1 << s) < ps) ++s;
  return s;
}

fi_status check_dtypes(fi_dtype q, fi_dtype kv) {
  if (q != FI_F16 && q != FI_BF16)
    return fail(FI_ERR_UNSUPPORTED, "q_dtype must be FI_F16 or FI_BF16 (got %d)", (int)q);
  if (kv != q && kv != FI_E4M3)
    return fail(FI_ERR_UNSUPPORTED, "kv_dtype must equal q_dtype or be FI_E4M3 (got %d)",
                (int)kv);
  return FI_OK;
}

fi::PlanInput to_input(const fi_problem* p, int num_cus) {
  fi::PlanInput in;
  in.batch = p->batch;
  in.Hq = p->num_qo_heads;
  in.Hkv = p->num_kv_heads;
  in.D = p->head_dim;
  in.page_size = p->page_size;
  in.q_dtype = p->q_dtype;
  in.kv_dtype = p->kv_dtype;
  in.kv_indptr = p->kv_indptr;
  in.last_page_len = p->last_page_len;
  // shared cascade levels: the single-level fields, or the level array
  in.num_levels = 0;
  if (p->num_cascade_levels > 0 && p->num_prefix_groups == 0) {
    in.num_levels = p->cascade_levels ? p->num_cascade_levels : -1;
    if (!p->cascade_levels) return in;
    for (int l = 0; l < p->num_cascade_levels && l < fi::kMaxLevels; ++l) {
      const fi_cascade_level& c = p->cascade_levels[l];
      in.levels[l] = {c.num_groups, c.qo_indptr, c.kv_indptr, c.last_page_len};
    }
  } else if (p->num_cascade_levels > 0 || p->num_prefix_groups != 0) {
    in.num_levels = 1;
    in.levels[0] = {p->num_prefix_groups, p->prefix_qo_indptr, p->prefix_kv_indptr,
                    p->prefix_last_page_len};
    if (p->num_cascade_levels > 0) in.num_levels = -1;   // both forms given: rejected
  }
  in.chunk_tokens = p->chunk_tokens;
  in.num_cus = num_cus;
  in.pos_encoding = p->pos_encoding;
  in.append_qo_indptr = p->qo_indptr;
  in.causal = p->causal;
  in.ragged = p->kv_layout == FI_KV_RAGGED;
  in.hnd = p->kv_layout == FI_KV_PAGED_HND;
  if (p->kv_layout < 0 || p->kv_layout > FI_KV_PAGED_HND) in.ragged = in.hnd = -1;
  in.rope_theta = p->rope_theta;
  in.rope_scale = p->rope_scale;
  memset(&in.tune, 0, sizeof(in.tune));
  if (p->tuning) {
    const fi_tuning& t = *p->tuning;
    in.tune = fi::Tuning{t.heads_per_tile,   t.waves_per_cu,     t.chunk_min,
                         t.prefix_waves,     t.prefix_tiles_per_cu, t.prefix_chunk_min,
                         t.cascade_fold,     t.fold_max_suffix,  t.append_tiles_pct,
                         t.append_chunk_min, t.decode_depth,     t.prefix_split_p,
                         t.rope_split_k,     t.score_path};
  }
  return in;
}

// Waves per compute unit that the current device holds at once of the decode
// instance a plan of *ctx (an fi_problem) launches with tiles of hpt kv heads
// (PlanInput::resident_waves); 0 when there is no device or the problem's
// fields are out of range (the plan validates them itself).
int resident_decode_waves(const void* ctx, int hpt, int rope_form, int fold) {
  const fi_problem* pr = static_cast<const fi_problem*>(ctx);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (pr->q_dtype != FI_F16 && pr->q_dtype != FI_BF16) return 0;
  const bool ragged = pr->kv_layout == FI_KV_RAGGED;
  const int ps = ragged ? 1 : pr->page_size;
  if (ps < 1) return 0;
  fi::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.ps_shift = ps_shift_of(ps);
  static const float kTableStandIn = 0.f;   // selects the RoPE instances only
  p.rope_table = rope_form ? &kTableStandIn : nullptr;
  p.rope_single = rope_form == 2 ? 1 : 0;
  const bool qbf = pr->q_dtype == FI_BF16;
  const int kv = pr->kv_dtype == FI_E4M3 ? 2 : (qbf ? 1 : 0);
  const int depth = pr->tuning ? pr->tuning->decode_depth : 0;
  int blocks = 0;
  if (fi::decode_occupancy(p, hpt, qbf, kv, fold != 0, depth, pr->head_dim, &blocks) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return blocks * hpt;
}

// device_occupancy: size the decode wave target by what the current device
// holds of the instance (fi_plan); the test hook plans without it.
fi_status build_host_plan(const fi_problem* problem, int num_cus, fi::HostPlan* hp,
                          bool device_occupancy = false) {
  if (!problem) return fail(FI_ERR_INVALID_ARG, "problem is NULL");
  fi_status st = check_dtypes(problem->q_dtype, problem->kv_dtype);
  if (st != FI_OK) return st;
  char err[256] = {0};
  int rc;
  try {   // no exception crosses the C ABI
    fi::PlanInput in = to_input(problem, num_cus);
    if (device_occupancy) {
      in.resident_waves = resident_decode_waves;
      in.resident_ctx = problem;
    }
    rc = fi::plan_build(in, hp, err, sizeof(err));
  } catch (const std::bad_alloc&) {
    fi::plan_free(hp);
    return fail(FI_ERR_INVALID_ARG, "out of host memory while planning");
  }
  if (rc != 0) {
    fi::plan_free(hp);
    return fail(rc == 2 ? FI_ERR_UNSUPPORTED : FI_ERR_INVALID_ARG, "%s", err);
  }
  return FI_OK;
}

fi::DecodeParams base_params(const fi_plan_s* pl, const void* q, const void* k,
                             const void* v, const float* ks, const float* vs,
                             float sm_scale, void* o, float* lse) {
  const fi::HostPlan& hp = pl->hp;
  fi::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k_pages = k;
  p.v_pages = v;
  p.k_scale = hp.kv_dtype == FI_E4M3 ? ks : nullptr;
  p.v_scale = hp.kv_dtype == FI_E4M3 ? vs : nullptr;
  p.tiles = reinterpret_cast<const fi::Tile*>(pl->workspace + hp.layout.tiles_off);
  p.req_info = reinterpret_cast<const fi::ReqInfo*>(pl->workspace + hp.layout.req_info_off);
  p.partial_o = reinterpret_cast<float*>(pl->workspace + hp.layout.partial_o_off);
  p.partial_lse = reinterpret_cast<float*>(pl->workspace + hp.layout.partial_lse_off);
  p.o = o;
  p.lse = lse;
  const float sc = sm_scale > 0.f ? sm_scale : 1.0f / std::sqrt((float)hp.D);
  p.sm_scale_log2 = sc * 1.4426950408889634f;
  p.Hq = hp.Hq;
  p.Hkv = hp.Hkv;
  p.G = hp.G;
  p.page_size = hp.page_size;
  p.ps_shift = ps_shift_of(hp.page_size);
  p.num_tiles = (int32_t)hp.num_tiles;
  if (hp.rope) {
    p.rope_table = pl->workspace + hp.layout.rope_off;
    p.rope_rows = hp.rope_rows;
    p.rope_single = hp.rope_single;
  }
  p.ragged = hp.ragged;
  p.valu_heads = hp.valu_heads;
  {
    const uint32_t rowb = (uint32_t)hp.D * (hp.kv_dtype == FI_E4M3 ? 1u : 2u);
    const uint32_t ps = (uint32_t)hp.page_size, hkv = (uint32_t)hp.Hkv;
    p.page_bytes = ps * hkv * rowb;
    p.slot_stride = hp.hnd ? rowb : hkv * rowb;
    p.head_stride = hp.hnd ? ps * rowb : rowb;
  }
  return p;
}

fi_status launch_merge(const fi_plan_s* pl, void* o, float* lse, hipStream_t s) {
  const fi::HostPlan& hp = pl->hp;
  if (hp.num_merge_units == 0) return FI_OK;
  fi::MergeParams m;
  m.partial_o = reinterpret_cast<const float*>(pl->workspace + hp.layout.partial_o_off);
  m.partial_lse = reinterpret_cast<const float*>(pl->workspace + hp.layout.partial_lse_off);
  m.units = reinterpret_cast<const fi::MergeUnit*>(pl->workspace + hp.layout.merge_reqs_off);
  m.o = o;
  m.lse = lse;
  m.Hq = hp.Hq;
  m.Hkv = hp.Hkv;
  m.G = hp.G;
  m.out_dtype = hp.q_dtype;
  hipError_t e = fi::launch_merge_partials(m, (int)hp.num_merge_units, hp.q_dtype == FI_BF16,
                                          hp.merge_wide != 0, hp.D, s);
  return e == hipSuccess ? FI_OK : hip_fail(e, "merge launch");
}

}  // namespace

extern "C" {

const char* fi_status_string(fi_status st) {
  switch (st) {
    case FI_OK: return "FI_OK";
    case FI_ERR_INVALID_ARG: return "FI_ERR_INVALID_ARG";
    case FI_ERR_UNSUPPORTED: return "FI_ERR_UNSUPPORTED";
    case FI_ERR_WORKSPACE_TOO_SMALL: return "FI_ERR_WORKSPACE_TOO_SMALL";
    case FI_ERR_HIP: return "FI_ERR_HIP";
  }
  return "unknown fi_status";
}

const char* fi_last_error(void) { return g_last_error.c_str(); }

fi_status fi_plan(const fi_problem* problem, int32_t num_cus, void* workspace,
                  size_t workspace_bytes, size_t* workspace_needed, void* stream,
                  fi_plan_t* plan_out) {
  g_last_error.clear();
  if (plan_out) *plan_out = nullptr;
  if (num_cus < 0) return fail(FI_ERR_INVALID_ARG, "num_cus must be >= 0");
  if (num_cus == 0) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "querying the compute unit count");
    num_cus = cus;
  }
  fi::HostPlan hp;
  fi_status st = build_host_plan(problem, num_cus, &hp, true);
  if (st != FI_OK) return st;
  if (workspace_needed) *workspace_needed = hp.layout.total;
  if (!workspace) {
    fi::plan_free(&hp);
    return FI_OK;
  }
  if (!plan_out) {
    fi::plan_free(&hp);
    return fail(FI_ERR_INVALID_ARG, "plan_out is NULL");
  }
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) {
    fi::plan_free(&hp);
    return fail(FI_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  if (workspace_bytes < hp.layout.total) {
    size_t need = hp.layout.total;
    fi::plan_free(&hp);
    return fail(FI_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the plan needs %zu",
                workspace_bytes, need);
  }
  const size_t meta_bytes = hp.layout.partial_o_off;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  int sb = -1;
  if (e == hipSuccess) sb = staging_acquire(std::max<size_t>(meta_bytes, 256), dev, &e);
  if (sb < 0) {
    fi::plan_free(&hp);
    return hip_fail(e, "pinned staging buffer for the plan upload");
  }
  void* staging = staging_ptr(sb);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  char* st8 = reinterpret_cast<char*>(staging);
  memset(st8, 0, meta_bytes);
  memcpy(st8 + hp.layout.tiles_off, hp.tiles,
         sizeof(fi::Tile) * (hp.num_tiles + hp.num_prefix_tiles));
  memcpy(st8 + hp.layout.req_info_off, hp.req_info, sizeof(fi::ReqInfo) * hp.num_req_info);
  memcpy(st8 + hp.layout.merge_reqs_off, hp.merge_units,
         sizeof(fi::MergeUnit) * hp.num_merge_units);
  memcpy(st8 + hp.layout.qo_indptr_off, hp.qo_indptr, sizeof(int32_t) * hp.qo_len);
  if (hp.num_levels >= 2)
    memcpy(st8 + hp.layout.state_off_off, hp.state_off,
           sizeof(int32_t) * (size_t)hp.num_levels * hp.batch);
  if (hp.num_rope_qpos > 0)
    memcpy(st8 + hp.layout.rope_qpos_off, hp.rope_qpos, sizeof(int32_t) * hp.num_rope_qpos);
  e = hipMemcpyAsync(workspace, staging, meta_bytes, hipMemcpyHostToDevice, hs);
  const bool copied = e == hipSuccess;
  if (e == hipSuccess && hp.rope)   // the (cos, sin) table, built on the device
    e = fi::launch_rope_table(reinterpret_cast<char*>(workspace) + hp.layout.rope_off,
                              hp.rope_rows, hp.D, hp.rope_theta, hp.rope_scale,
                              hp.rope_single != 0, hs);
  const hipError_t er = staging_release(sb, hs, copied);
  if (e == hipSuccess) e = er;
  if (e != hipSuccess) {
    fi::plan_free(&hp);
    return hip_fail(e, "uploading the plan");
  }
  fi_plan_s* pl = new (std::nothrow) fi_plan_s;
  if (!pl) {
    fi::plan_free(&hp);
    return fail(FI_ERR_INVALID_ARG, "out of host memory for the plan object");
  }
  pl->hp = hp;
  pl->workspace = reinterpret_cast<char*>(workspace);
  pl->workspace_bytes = workspace_bytes;
  *plan_out = pl;
  return FI_OK;
}

fi_status fi_plan_destroy(fi_plan_t plan) {
  if (!plan) return FI_OK;
  fi::plan_free(&plan->hp);
  delete plan;
  return FI_OK;
}

fi_status fi_plan_get_stats(fi_plan_t plan, fi_plan_stats* s) {
  if (!plan || !s) return fail(FI_ERR_INVALID_ARG, "plan and stats must be non-NULL");
  const fi::HostPlan& hp = plan->hp;
  s->num_tiles = hp.num_tiles;
  s->num_prefix_tiles = hp.num_prefix_tiles;
  s->num_partials = hp.num_partials;
  s->num_merge_units = hp.num_merge_units;
  s->chunk_tokens = hp.chunk_tokens;
  s->prefix_chunk_tokens = hp.prefix_chunk_tokens;
  s->heads_per_tile = hp.heads_per_tile;
  s->num_cus = hp.num_cus;
  s->workspace_bytes = hp.layout.total;
  s->num_folded = hp.num_folded;
  s->prefix_split_p = hp.prefix_split_p;
  s->rope_single = hp.rope_single;
  s->valu_heads = hp.valu_heads;
  s->decode_waves_per_cu = hp.decode_waves_per_cu;
  s->staging_buffers = staging_count();
  return FI_OK;
}

namespace {

enum Stage { kStagePrefix = 1, kStageDecode = 2, kStageMerge = 4 };

// Device tables of the shared cascade levels, outermost first.
struct LevelTables {
  int n = 0;
  const int32_t* indptr[fi::kMaxLevels] = {};
  const int32_t* indices[fi::kMaxLevels] = {};
  const int32_t* last[fi::kMaxLevels] = {};
};

LevelTables one_level(const int32_t* indptr, const int32_t* indices, const int32_t* last) {
  LevelTables t;
  t.n = 1;
  t.indptr[0] = indptr;
  t.indices[0] = indices;
  t.last[0] = last;
  return t;
}

// Shared argument checks of the run calls; level tables are required only
// for levels with groups.
fi_status check_run_args(const fi::HostPlan& hp, const void* q, const void* k_pages,
                         const void* v_pages, const LevelTables& lv,
                         const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int32_t* last_page_len, float sm_scale, const void* o) {
  if (!q || !o || !kv_indptr || (!hp.ragged && !last_page_len))
    return fail(FI_ERR_INVALID_ARG, "q, o, kv_indptr and last_page_len must be non-NULL");
  if (!hp.append && lv.n < hp.num_levels)
    return fail(FI_ERR_INVALID_ARG, "the plan has %d cascade levels, %d sets of tables given",
                hp.num_levels, lv.n);
  for (int l = 0; l < hp.num_levels && !hp.append; ++l) {
    if (hp.level_groups[l] == 0) continue;
    if (!lv.indptr[l] || (!hp.ragged && !lv.last[l]))
      return fail(FI_ERR_INVALID_ARG,
                  "the prefix indptr / last_page_len tables must be non-NULL (level %d)", l);
    if (!hp.ragged && !lv.indices[l] &&
        hp.level_tile_off[l + 1] > hp.level_tile_off[l])
      return fail(FI_ERR_INVALID_ARG, "the index tables must be non-NULL (level %d)", l);
  }
  // (a batch whose every key list is empty reads no K/V and no index)
  if ((hp.has_keys || (!hp.append && hp.num_prefix_tiles > 0)) && (!k_pages || !v_pages))
    return fail(FI_ERR_INVALID_ARG, "k_pages and v_pages must be non-NULL");
  // append tiles read the per-request table
  const bool own_rows = hp.num_tiles > 0 || (hp.append && hp.num_prefix_tiles > 0);
  if (!hp.ragged && !kv_indices && own_rows && hp.has_keys)
    return fail(FI_ERR_INVALID_ARG, "the index tables must be non-NULL");
  if (!(sm_scale == sm_scale) || std::isinf(sm_scale))
    return fail(FI_ERR_INVALID_ARG, "sm_scale must be finite");
  return FI_OK;
}

// Enqueues the selected stages of a planned run on stream s, in order
// prefix (level by level) -> decode -> merge (a folded suffix tile reads
// the prefix states, so the prefix kernels always complete first).
fi_status enqueue_run(fi_plan_t plan, int stages, const void* q, const void* k_pages,
                      const void* v_pages, const LevelTables& lv, const int32_t* kv_indptr,
                      const int32_t* kv_indices, const float* k_scale, const float* v_scale,
                      float sm_scale, void* o, float* lse, hipStream_t s,
                      int64_t* rec = nullptr, const int64_t* rec_base = nullptr) {
  const fi::HostPlan& hp = plan->hp;
  const bool qbf = hp.q_dtype == FI_BF16;
  const int kv = hp.kv_dtype == FI_E4M3 ? 2 : (qbf ? 1 : 0);
  fi::DecodeParams p = base_params(plan, q, k_pages, v_pages, k_scale, v_scale, sm_scale, o, lse);
  p.rec = rec;
  p.rec_base = rec_base;
  hipError_t e = hipSuccess;
  const bool do_prefix = (stages & kStagePrefix) && hp.num_prefix_tiles > 0;
  const bool do_decode = (stages & kStageDecode) && hp.num_tiles > 0;
  const int32_t* qo_all = reinterpret_cast<const int32_t*>(plan->workspace + hp.layout.qo_indptr_off);
  if (do_prefix && hp.append) {
    // append tiles read the request's own table; row -> query token = the
    // request's first token (planned copy of qo_indptr) + row / G
    fi::DecodeParams pp = p;
    pp.kv_indptr = kv_indptr;
    pp.kv_indices = kv_indices;
    pp.qo_indptr = qo_all;
    if (hp.num_rope_qpos > 0)
      pp.rope_qpos = reinterpret_cast<const int32_t*>(plan->workspace + hp.layout.rope_qpos_off);
    e = fi::launch_prefix(pp, (int)hp.num_prefix_tiles, hp.prefix_waves, true, false, qbf, kv,
                          hp.D, s);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  } else if (do_prefix) {
    // prefix tiles of level l read that level's table; row -> request = the
    // group's first request (planned copy of the level's qo_indptr) + row / G
    for (int l = 0; l < hp.num_levels; ++l) {
      const int64_t n = hp.level_tile_off[l + 1] - hp.level_tile_off[l];
      if (n == 0) continue;
      fi::DecodeParams pp = p;
      pp.kv_indptr = lv.indptr[l];
      pp.kv_indices = lv.indices[l];
      pp.qo_indptr = qo_all + hp.level_qo_start[l];
      pp.state_off = hp.num_levels >= 2
                         ? reinterpret_cast<const int32_t*>(plan->workspace +
                                                            hp.layout.state_off_off) +
                               (int64_t)l * hp.batch
                         : nullptr;
      pp.num_tiles = (int32_t)(hp.num_tiles + hp.level_tile_off[l]);
      if (hp.num_rope_qpos > 0)
        pp.rope_qpos =
            reinterpret_cast<const int32_t*>(plan->workspace + hp.layout.rope_qpos_off) +
            (int64_t)l * hp.batch;
      e = fi::launch_prefix(pp, (int)n, hp.prefix_waves, false, (hp.prefix_split_p >> l) & 1u,
                            qbf, kv, hp.D, s);
      if (e != hipSuccess) return hip_fail(e, "prefix launch");
    }
  }
  if (do_decode) {
    p.kv_indptr = kv_indptr;
    p.kv_indices = kv_indices;
    e = fi::launch_decode(p, (int)hp.num_tiles, hp.heads_per_tile, qbf, kv, hp.num_folded > 0,
                          hp.decode_depth, hp.D, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  if (stages & kStageMerge) return launch_merge(plan, o, lse, s);
  return FI_OK;
}

}  // namespace

fi_status fi_decode_run(fi_plan_t plan, const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* kv_indptr,
                        const int32_t* kv_indices, const int32_t* last_page_len,
                        const float* k_scale, const float* v_scale, float sm_scale,
                        void* o, float* lse, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const fi::HostPlan& hp = plan->hp;
  if (hp.num_groups != 0)
    return fail(FI_ERR_INVALID_ARG, "plan has a cascade level: use fi_cascade_decode");
  if (hp.append) return fail(FI_ERR_INVALID_ARG, "append plan: use fi_append_run");
  if (hp.batch == 0) return FI_OK;
  const LevelTables none;
  fi_status st = check_run_args(hp, q, k_pages, v_pages, none, kv_indptr, kv_indices,
                                last_page_len, sm_scale, o);
  if (st != FI_OK) return st;
  return enqueue_run(plan, kStageDecode | kStageMerge, q, k_pages, v_pages, none, kv_indptr,
                     kv_indices, k_scale, v_scale, sm_scale, o, lse,
                     reinterpret_cast<hipStream_t>(stream));
}

fi_status fi_cascade_decode(fi_plan_t plan, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* prefix_kv_indptr,
                            const int32_t* prefix_kv_indices,
                            const int32_t* prefix_last_page_len, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* last_page_len,
                            const float* k_scale, const float* v_scale, float sm_scale,
                            void* o, float* lse, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const fi::HostPlan& hp = plan->hp;
  if (hp.append) return fail(FI_ERR_INVALID_ARG, "append plan: use fi_append_run");
  if (hp.num_groups == 0)
    return fail(FI_ERR_INVALID_ARG, "plan has no cascade level: use fi_decode_run");
  if (hp.num_levels != 1)
    return fail(FI_ERR_INVALID_ARG, "plan has %d cascade levels: use fi_cascade_decode_levels",
                hp.num_levels);
  if (hp.batch == 0) return FI_OK;
  const LevelTables lv = one_level(prefix_kv_indptr, prefix_kv_indices, prefix_last_page_len);
  fi_status st = check_run_args(hp, q, k_pages, v_pages, lv, kv_indptr, kv_indices,
                                last_page_len, sm_scale, o);
  if (st != FI_OK) return st;
  return enqueue_run(plan, kStagePrefix | kStageDecode | kStageMerge, q, k_pages, v_pages, lv,
                     kv_indptr, kv_indices, k_scale, v_scale, sm_scale, o, lse,
                     reinterpret_cast<hipStream_t>(stream));
}

fi_status fi_cascade_decode_levels(fi_plan_t plan, const void* q, const void* k_pages,
                                   const void* v_pages, int32_t num_levels,
                                   const int32_t* const* level_kv_indptr,
                                   const int32_t* const* level_kv_indices,
                                   const int32_t* const* level_last_page_len,
                                   const int32_t* kv_indptr, const int32_t* kv_indices,
                                   const int32_t* last_page_len, const float* k_scale,
                                   const float* v_scale, float sm_scale, void* o, float* lse,
                                   void* stream) {
  g_last_error.clear();
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const fi::HostPlan& hp = plan->hp;
  if (hp.append) return fail(FI_ERR_INVALID_ARG, "append plan: use fi_append_run");
  if (num_levels != hp.num_levels)
    return fail(FI_ERR_INVALID_ARG, "the plan has %d cascade levels, got %d", hp.num_levels,
                num_levels);
  if (num_levels > 0 && (!level_kv_indptr || !level_kv_indices || !level_last_page_len))
    return fail(FI_ERR_INVALID_ARG, "the level table arrays must be non-NULL");
  if (hp.batch == 0) return FI_OK;
  LevelTables lv;
  lv.n = num_levels;
  for (int l = 0; l < num_levels; ++l) {
    lv.indptr[l] = level_kv_indptr[l];
    lv.indices[l] = level_kv_indices[l];
    lv.last[l] = level_last_page_len[l];
  }
  fi_status st = check_run_args(hp, q, k_pages, v_pages, lv, kv_indptr, kv_indices,
                                last_page_len, sm_scale, o);
  if (st != FI_OK) return st;
  return enqueue_run(plan, kStagePrefix | kStageDecode | kStageMerge, q, k_pages, v_pages, lv,
                     kv_indptr, kv_indices, k_scale, v_scale, sm_scale, o, lse,
                     reinterpret_cast<hipStream_t>(stream));
}

fi_status fi_append_run(fi_plan_t plan, const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* kv_indptr,
                        const int32_t* kv_indices, const int32_t* last_page_len,
                        const float* k_scale, const float* v_scale, float sm_scale,
                        void* o, float* lse, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const fi::HostPlan& hp = plan->hp;
  if (!hp.append) return fail(FI_ERR_INVALID_ARG, "plan is not an append plan");
  if (hp.total_q == 0) return FI_OK;
  const LevelTables none;
  fi_status st = check_run_args(hp, q, k_pages, v_pages, none, kv_indptr, kv_indices,
                                last_page_len, sm_scale, o);
  if (st != FI_OK) return st;
  return enqueue_run(plan, kStagePrefix | kStageMerge, q, k_pages, v_pages, none, kv_indptr,
                     kv_indices, k_scale, v_scale, sm_scale, o, lse,
                     reinterpret_cast<hipStream_t>(stream));
}

fi_status fi_debug_run_stage(fi_plan_t plan, int32_t stage, const void* q, const void* k_pages,
                             const void* v_pages, const int32_t* prefix_kv_indptr,
                             const int32_t* prefix_kv_indices,
                             const int32_t* prefix_last_page_len, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* last_page_len,
                             const float* k_scale, const float* v_scale, float sm_scale,
                             void* o, float* lse, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const fi::HostPlan& hp = plan->hp;
  if (stage < 0 || stage > 2)
    return fail(FI_ERR_INVALID_ARG,
                "stage must be 0 (decode kernel), 1 (prefix kernel) or 2 (merge kernel)");
  if (stage == 1 && hp.num_prefix_tiles == 0)
    return fail(FI_ERR_INVALID_ARG, "the plan has no cascade prefix or append tiles");
  if (hp.num_levels > 1)
    return fail(FI_ERR_INVALID_ARG, "stage hook: plans with one cascade level at most");
  if (hp.batch == 0 || (hp.append && hp.total_q == 0)) return FI_OK;
  const LevelTables lv = hp.num_levels == 1
                             ? one_level(prefix_kv_indptr, prefix_kv_indices, prefix_last_page_len)
                             : LevelTables();
  fi_status st = check_run_args(hp, q, k_pages, v_pages, lv, kv_indptr, kv_indices,
                                last_page_len, sm_scale, o);
  if (st != FI_OK) return st;
  const int which = stage == 0 ? kStageDecode : stage == 1 ? kStagePrefix : kStageMerge;
  return enqueue_run(plan, which, q, k_pages, v_pages, lv, kv_indptr, kv_indices, k_scale,
                     v_scale, sm_scale, o, lse, reinterpret_cast<hipStream_t>(stream));
}

fi_status fi_debug_record_walk(fi_plan_t plan, int32_t stage, const void* q,
                               const void* k_pages, const void* v_pages,
                               const int32_t* prefix_kv_indptr,
                               const int32_t* prefix_kv_indices,
                               const int32_t* prefix_last_page_len, const int32_t* kv_indptr,
                               const int32_t* kv_indices, const int32_t* last_page_len,
                               const float* k_scale, const float* v_scale, float sm_scale,
                               void* o, float* lse, int64_t* rec, const int64_t* rec_base,
                               void* stream) {
  g_last_error.clear();
  if (!plan) return fail(FI_ERR_INVALID_ARG, "plan is NULL");
  const fi::HostPlan& hp = plan->hp;
  if (stage != 0 && stage != 1)
    return fail(FI_ERR_INVALID_ARG, "stage must be 0 (decode kernel) or 1 (multi-row kernel)");
  if (!rec || !rec_base) return fail(FI_ERR_INVALID_ARG, "rec and rec_base must be non-NULL");
  if (stage == 1 && hp.num_prefix_tiles == 0)
    return fail(FI_ERR_INVALID_ARG, "the plan has no cascade prefix or append tiles");
  if (hp.num_levels > 1)
    return fail(FI_ERR_INVALID_ARG, "record hook: plans with one cascade level at most");
  if (hp.batch == 0 || (hp.append && hp.total_q == 0)) return FI_OK;
  const LevelTables lv = hp.num_levels == 1
                             ? one_level(prefix_kv_indptr, prefix_kv_indices, prefix_last_page_len)
                             : LevelTables();
  fi_status st = check_run_args(hp, q, k_pages, v_pages, lv, kv_indptr, kv_indices,
                                last_page_len, sm_scale, o);
  if (st != FI_OK) return st;
  // the record instances that are built
  const bool f16 = hp.q_dtype == FI_F16 && hp.kv_dtype == FI_F16;
  const bool fp8 = hp.q_dtype == FI_BF16 && hp.kv_dtype == FI_E4M3;
  const int depth = hp.decode_depth ? hp.decode_depth
                                    : (hp.num_folded > 0 && hp.heads_per_tile <= 4 ? 2 : 1);
  if (hp.D != 128 || hp.rope || !(f16 || fp8) ||
      (stage == 1 && (hp.prefix_waves != 8 || (fp8 && hp.append))) ||
      (stage == 0 && fp8 && depth == 2))
    return fail(FI_ERR_UNSUPPORTED,
                "record hook: head_dim 128, fp16 q + fp16 K/V or bf16 q + e4m3 K/V (one step "
                "in flight, no append), 8-wave multi-row tiles, no RoPE");
  return enqueue_run(plan, stage == 0 ? kStageDecode : kStagePrefix, q, k_pages, v_pages, lv,
                     kv_indptr, kv_indices, k_scale, v_scale, sm_scale, o, lse,
                     reinterpret_cast<hipStream_t>(stream), rec, rec_base);
}

fi_status fi_decode_noalloc(const fi_problem* problem, const void* q, const void* k_pages,
                           const void* v_pages, const int32_t* kv_indptr,
                           const int32_t* kv_indices, const int32_t* last_page_len,
                           const float* k_scale, const float* v_scale, float sm_scale, void* o,
                           float* lse, void* stream) {
  g_last_error.clear();
  if (!problem) return fail(FI_ERR_INVALID_ARG, "problem is NULL");
  fi_status st = check_dtypes(problem->q_dtype, problem->kv_dtype);
  if (st != FI_OK) return st;
  // sizes first (host only): nothing touches the device before they pass
  int num_cus = 0, dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "querying the compute unit count");
  fi_plan_s pl;   // on the stack: the plan's sizes, its work list in scratch
  char err[320] = {0};
  fi::PlanInput in = to_input(problem, num_cus);
  in.resident_waves = resident_decode_waves;
  in.resident_ctx = problem;
  const int rc = fi::plan_decode_static(in, fi::scratch_capacity(), &pl.hp, err, sizeof(err));
  if (rc != 0) return fail(rc == 2 ? FI_ERR_UNSUPPORTED : FI_ERR_INVALID_ARG, "%s", err);
  const fi::HostPlan& hp = pl.hp;
  if (hp.batch == 0) return FI_OK;
  const LevelTables none;
  st = check_run_args(hp, q, k_pages, v_pages, none, kv_indptr, kv_indices, last_page_len,
                      sm_scale, o);
  if (st != FI_OK) return st;
  void* base = nullptr;
  e = fi::scratch_address(&base);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (static scratch)");
  pl.workspace = reinterpret_cast<char*>(base);
  pl.workspace_bytes = fi::scratch_capacity();
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  e = fi::launch_device_plan(kv_indptr, hp.ragged ? nullptr : last_page_len, hp.batch,
                             hp.page_size, hp.chunk_tokens, hp.heads_per_tile, hp.Hkv,
                             pl.workspace + hp.layout.tiles_off,
                             pl.workspace + hp.layout.req_info_off,
                             pl.workspace + hp.layout.merge_reqs_off, hp.num_tiles,
                             hp.num_merge_units, hs);
  if (e != hipSuccess) return hip_fail(e, "device planner launch");
  return enqueue_run(&pl, kStageDecode | kStageMerge, q, k_pages, v_pages, none, kv_indptr,
                     kv_indices, k_scale, v_scale, sm_scale, o, lse, hs);
}

fi_status fi_merge_states(int32_t num_states, const void* const* v_states,
                          const float* const* s_states, int64_t num_rows, int32_t head_dim,
                          fi_dtype v_dtype, void* v_out, float* s_out, fi_dtype out_dtype,
                          void* stream) {
  g_last_error.clear();
  if (num_states < 1 || num_states > fi::kMaxMergeStates)
    return fail(FI_ERR_INVALID_ARG, "num_states must be in [1, %d]", fi::kMaxMergeStates);
  if (num_rows < 0 || head_dim <= 0)
    return fail(FI_ERR_INVALID_ARG, "num_rows must be >= 0 and head_dim > 0");
  auto ok_dt = [](fi_dtype d) { return d == FI_F16 || d == FI_BF16 || d == FI_F32; };
  if (!ok_dt(v_dtype) || !ok_dt(out_dtype))
    return fail(FI_ERR_UNSUPPORTED, "merge dtypes must be FI_F16, FI_BF16 or FI_F32");
  if (num_rows == 0) return FI_OK;
  if (!v_states || !s_states || !v_out)
    return fail(FI_ERR_INVALID_ARG, "v_states, s_states and v_out must be non-NULL");
  fi::MergeStatesParams p;
  memset(&p, 0, sizeof(p));
  for (int i = 0; i < num_states; ++i) {
    if (!v_states[i] || !s_states[i])
      return fail(FI_ERR_INVALID_ARG, "state %d has a NULL pointer", i);
    p.v[i] = v_states[i];
    p.s[i] = s_states[i];
  }
  p.num_states = num_states;
  p.num_rows = num_rows;
  p.head_dim = head_dim;
  p.v_dtype = v_dtype;
  p.out_dtype = out_dtype;
  p.v_out = v_out;
  p.s_out = s_out;
  hipError_t e = fi::launch_merge_states(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FI_OK : hip_fail(e, "merge_states launch");
}

fi_status fi_debug_plan_tiles(const fi_problem* problem, int32_t num_cus, int32_t* tiles_out,
                              int64_t capacity_tiles, int64_t* num_tiles) {
  g_last_error.clear();
  if (!num_tiles) return fail(FI_ERR_INVALID_ARG, "num_tiles is NULL");
  fi::HostPlan hp;
  fi_status st = build_host_plan(problem, num_cus > 0 ? num_cus : 256, &hp);
  if (st != FI_OK) return st;
  const int64_t n = hp.num_tiles + hp.num_prefix_tiles;
  *num_tiles = n;
  if (tiles_out && capacity_tiles >= n)
    memcpy(tiles_out, hp.tiles, sizeof(fi::Tile) * n);
  fi::plan_free(&hp);
  return FI_OK;
}

fi_status fi_debug_gather(int32_t batch, int32_t page_size, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* last_page_len,
                          const int64_t* token_indptr, int64_t* out_slots, void* stream) {
  g_last_error.clear();
  (void)last_page_len;
  if (batch < 0 || page_size < 1) return fail(FI_ERR_INVALID_ARG, "bad batch or page_size");
  if (batch == 0) return FI_OK;
  if (!kv_indptr || !kv_indices || !token_indptr || !out_slots)
    return fail(FI_ERR_INVALID_ARG, "NULL pointer");
  hipError_t e = fi::launch_gather(kv_indptr, kv_indices, token_indptr, batch, page_size,
                                   ps_shift_of(page_size), out_slots,
                                   reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FI_OK : hip_fail(e, "gather launch");
}

fi_status fi_debug_stream_read(const void* src, size_t bytes, uint32_t* sink,
                               int32_t num_blocks, void* stream) {
  g_last_error.clear();
  if (!src || !sink || num_blocks <= 0 || bytes % 16 != 0)
    return fail(FI_ERR_INVALID_ARG, "stream_read: NULL pointer, no blocks, or bytes %% 16");
  hipError_t e = fi::launch_stream_read(src, (int64_t)bytes, sink, num_blocks,
                                        reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FI_OK : hip_fail(e, "stream_read launch");
}

}  // extern "C"
