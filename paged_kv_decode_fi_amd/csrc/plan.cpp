// plan.cpp -- host plan scheduler (pure C++, no HIP).
//
// FlashInfer README, "core features" item 2: attention over variable-length
// requests is split into a plan stage, which schedules the work on the host
// to avoid load imbalance, and a run stage.  The README names stream-K as an
// inspiration: long work is cut into pieces processed by different
// workgroups and fixed up afterwards; here the fix-up is the merge of
// (o, lse) attention states.
//
// Work model.  Each (request r, kv head h) has L_r keys.  A decode tile is one
// workgroup of W waves = W consecutive kv heads of one request over one
// token chunk [t0, t1) (W = 8 when Hkv allows; fewer for small problems,
// and 4 where narrower tiles even out the load over the CUs).
// The chunk length c is one value for the whole batch: the smallest
// multiple of the 16-token step, at least c_min, such that the waves
// launched stay within target = num_cus * waves_per_cu, one round of the
// waves the launched instance keeps resident (more chunks than that only
// adds partial states to merge) -- or two rounds when lengths are so skewed
// that one round would leave the long requests' tiles running alone.
// Tiles are placed for in-order dispatch (dispatch_order): the longest run
// first and each CU's share of the work evens out.
//
// Cascade: the shared prefix of group g is attended once per (g, kv head) by
// prefix tiles covering prefix_rows query rows each (rows = the group's
// requests x the G q heads of that kv head); the prefix is cut into chunks
// so that there is about one prefix tile per CU.  A request whose own suffix
// is one decode chunk folds the prefix chunks' states into its decode tile's
// output; others are merged by the merge kernel.
//
// Append (FlashInfer README append example; batch form over qo_indptr):
// request r's n_r query tokens are the last n_r of its L_r keys.  Query rows
// (token, head in the group) of one (request, kv head) are cut into tiles of
// prefix_rows rows; each row tile needs the keys up to its last row's causal
// limit, cut into chunks of one length for the batch (one tile per CU when
// there is not already that much work).  Query tokens with several chunks
// get partial states and a merge unit each.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <vector>

#include "fi_internal.h"

namespace fi {
namespace {

// a tuning field, or the default when it is 0
int tune_or(int32_t v, int dflt) { return v != 0 ? v : dflt; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Decode tiles for the dispatcher.  When every tile of a launch is resident
// at once, the hardware hands workgroup i to CU i mod num_cus, so position
// j * num_cus + c is CU c's j-th tile and the CU holding the most work ends
// the kernel.  Longest processing time first: each tile, longest first,
// goes to the least-loaded CU that still has a free position (ceil(n /
// num_cus) positions for the first n mod num_cus CUs, one fewer for the
// rest, so the positions are 0 .. n - 1).  w: work per tile, non-increasing.
// Returns each tile's position in *pos (when pos != NULL) and the most
// loaded CU's work over the mean.
double dispatch_order(const std::vector<int64_t>& w, int num_cus, std::vector<int64_t>* pos) {
  const int64_t n = (int64_t)w.size();
  if (pos) pos->resize(n);
  if (n == 0 || num_cus <= 0) return 1.0;
  if (n <= num_cus) {   // one tile per CU: the order stays
    if (pos)
      for (int64_t i = 0; i < n; ++i) (*pos)[i] = i;
    int64_t total = 0;
    for (int64_t x : w) total += x;
    return total > 0 ? (double)w[0] * num_cus / (double)total : 1.0;
  }
  const int64_t rounds = ceil_div(n, num_cus), full = n - (rounds - 1) * num_cus;
  std::vector<int64_t> load(num_cus, 0), cnt(num_cus, 0);
  // min-heap of (load, cu) over CUs with a free position
  std::vector<std::pair<int64_t, int>> heap;
  heap.reserve(num_cus);
  for (int c = 0; c < num_cus; ++c) heap.push_back({0, c});
  auto cmp = [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) {
    return a > b;
  };
  std::make_heap(heap.begin(), heap.end(), cmp);
  int64_t total = 0;
  for (int64_t i = 0; i < n; ++i) {
    std::pop_heap(heap.begin(), heap.end(), cmp);
    const int c = heap.back().second;
    heap.pop_back();
    if (pos) (*pos)[i] = cnt[c] * num_cus + c;   // CU c's tiles stay longest first
    load[c] += w[i];
    total += w[i];
    if (++cnt[c] < (c < full ? rounds : rounds - 1)) {
      heap.push_back({load[c], c});
      std::push_heap(heap.begin(), heap.end(), cmp);
    }
  }
  const int64_t mx = *std::max_element(load.begin(), load.end());
  return total > 0 ? (double)mx * num_cus / (double)total : 1.0;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// kv_len from a CSR page table row (ragged: last == NULL, indptr counts
// tokens)
int64_t table_len(const int32_t* indptr, const int32_t* last, int i, int ps) {
  int64_t n = (int64_t)indptr[i + 1] - indptr[i];
  if (!last) return n;
  return n == 0 ? 0 : (n - 1) * ps + last[i];
}

#define PLAN_FAIL(code, ...)                 \
  do {                                       \
    snprintf(err, errlen, __VA_ARGS__);      \
    return code;                             \
  } while (0)

// Decode split policy: kv heads per tile and the chunk length, from the
// requests' lengths len(r) (no allocation; also used by the allocation-free
// entry point).
//  * heads per tile: the largest of tune.heads_per_tile (default 8; 4 with
//    RoPE: smaller workgroups of the register-heavier RoPE instances), 4,
//    2, 1 dividing Hkv; halved (down to 2) for small problems; halved once
//    more for uneven work (below, once the chunk is known).
//  * chunk: the smallest multiple of the 16-token step, at least chunk_min,
//    whose waves stay within num_cus * waves_per_cu (one round of resident
//    waves), or the longest request when that is already enough work.
//    waves_per_cu: tune.waves_per_cu, else 16 or, when fewer, the waves per
//    CU that the instance to be launched holds at once (resident(hpt); 0 =
//    unknown) -- a target past what is resident splits the work into a
//    second round of workgroups.  When that chunk is over 1.25x the mean
//    tokens per resident workgroup (skewed lengths: many short requests
//    force long chunks of the long ones, which then run alone at the end),
//    the chunk is sized for two rounds instead, so the long requests' tiles
//    fill in behind the short ones.
template <class LenFn, class ResidentFn>
void decode_split(const PlanInput& in, int num_cus, bool rope, LenFn len, ResidentFn resident,
                  int* hpt_out, int64_t* chunk_out, int* waves_per_cu_out) {
  const int B = in.batch, Hkv = in.Hkv;
  const int hpt_default = rope ? kWavesPerTile / 2 : kWavesPerTile;
  const bool hpt_forced = in.tune.heads_per_tile > 0;
  int hpt = (int)std::min<int64_t>(kWavesPerTile,
                                   std::max<int64_t>(1, tune_or(in.tune.heads_per_tile, hpt_default)));
  // (head_dim 256 with RoPE: the step's K/V rows of 8 heads and the
  // table rows exceed the LDS, so at most 4)
  if (rope && in.D == 256) hpt = std::min(hpt, kWavesPerTile / 2);
  while (hpt & (hpt - 1)) hpt &= hpt - 1;
  while (Hkv % hpt) hpt >>= 1;
  const int64_t c_min = round_up(std::max(tune_or(in.tune.chunk_min, 32), kChunkAlign),
                                 kChunkAlign);
  if (!hpt_forced) {
    // small problems (fewer than 2 tiles per CU even at the minimum chunk):
    // fewer heads per tile, so more, smaller workgroups spread the latency
    auto tiles_at_min = [&](int h) {
      int64_t t = 0;
      for (int r = 0; r < B; ++r) t += std::max<int64_t>(1, ceil_div(len(r), c_min));
      return t * (Hkv / h);
    };
    while (hpt > 2 && tiles_at_min(hpt) < 2 * (int64_t)num_cus) hpt >>= 1;
  }
  int64_t waves_per_cu = 16;
  if (in.tune.waves_per_cu > 0) {
    waves_per_cu = in.tune.waves_per_cu;
  } else {
    const int res = resident(hpt);
    if (res > 0) waves_per_cu = std::max<int64_t>(hpt, std::min<int64_t>(16, res));
  }
  const int64_t target_waves = std::max<int64_t>(1, num_cus * waves_per_cu);
  int64_t Lmax = 0;
  for (int r = 0; r < B; ++r) Lmax = std::max(Lmax, len(r));
  auto waves_for = [&](int64_t c) {
    int64_t w = 0;
    for (int r = 0; r < B; ++r) w += std::max<int64_t>(1, ceil_div(len(r), c));
    return w * Hkv;   // hpt waves per tile, Hkv / hpt tiles per chunk
  };
  int64_t chunk;
  if (in.chunk_tokens > 0) {
    chunk = in.chunk_tokens;
  } else {
    const int64_t hi = std::max<int64_t>(round_up(std::max<int64_t>(Lmax, 1), kChunkAlign),
                                         kChunkAlign);
    const int64_t lo = std::min(c_min, hi);
    auto chunk_for = [&](int64_t target) -> int64_t {
      if (waves_for(hi) >= target) return hi;   // enough work without splitting
      // smallest c in [lo, hi] (multiple of the step) with waves(c) <= target
      int64_t a = lo / kChunkAlign, b = hi / kChunkAlign;
      while (a < b) {
        int64_t mid = (a + b) / 2;
        if (waves_for(mid * kChunkAlign) <= target) b = mid; else a = mid + 1;
      }
      return a * kChunkAlign;
    };
    chunk = chunk_for(target_waves);
    // mean tokens per resident workgroup (Hkv / hpt tiles per chunk)
    int64_t tokens = 0;
    for (int r = 0; r < B; ++r) tokens += std::max<int64_t>(0, len(r));
    const double slots = (double)target_waves / hpt;
    const double mean = (double)tokens * (Hkv / hpt) / slots;
    if (in.tune.waves_per_cu == 0 && (double)chunk > 1.25 * mean)
      chunk = chunk_for(2 * target_waves);
  }
  // Narrower tiles for uneven work.  The hardware hands workgroups to the
  // CUs in turn, so the tiles' placement (dispatch_order) decides how much
  // work each CU holds, and the CU holding the most ends the kernel.  Tiles
  // of half the kv heads cut the same chunks into twice as many workgroups,
  // which evens that out when a few long requests dominate, at a measured
  // cost of ~4 % per byte (each token's K/V rows of the tile are half as
  // long a contiguous run).  They are taken when the modelled most-loaded
  // CU, relative to the mean, drops by more than that (skewed128: 1.138 ->
  // 1.045, step 217.7 -> 210.7 us; batch64_gqa4: 1.094 -> 1.064, 95.5 ->
  // 96.6 us measured, so kept at 8 heads).
  if (!hpt_forced && !rope && hpt == kWavesPerTile && in.chunk_tokens == 0 &&
      Hkv % (hpt / 2) == 0 && resident(hpt / 2) == resident(hpt)) {
    std::vector<int64_t> steps;   // per (request, chunk): 16-token steps
    for (int r = 0; r < B; ++r) {
      const int64_t L = len(r);
      if (L <= 0) continue;
      const int64_t nc = ceil_div(L, chunk), nst = ceil_div(L, (int64_t)kChunkAlign);
      for (int64_t c = 0; c < nc; ++c) steps.push_back(nst / nc + (c < nst % nc ? 1 : 0));
    }
    std::sort(steps.begin(), steps.end(), std::greater<int64_t>());
    auto imbalance = [&](int h) {   // the tiles of h kv heads, as dispatch_order places them
      std::vector<int64_t> w;
      for (int64_t st : steps)
        for (int k = 0; k < Hkv / h; ++k) w.push_back(st);
      return dispatch_order(w, num_cus, nullptr);
    };
    if (!steps.empty() && num_cus > 0 && imbalance(hpt / 2) * 1.04 < imbalance(hpt)) hpt /= 2;
  }
  *hpt_out = hpt;
  *chunk_out = chunk;
  *waves_per_cu_out = (int)waves_per_cu;
}

int plan_append(const PlanInput& in, const std::vector<int64_t>& lens, int num_cus,
                HostPlan* out, char* err, size_t errlen) {
  const int B = in.batch, Hkv = in.Hkv, G = in.Hq / in.Hkv;
  const int32_t* qo = in.append_qo_indptr;
  if (B > 0 && qo[0] != 0) PLAN_FAIL(1, "qo_indptr[0] must be 0");
  for (int r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r];
    if (n < 0) PLAN_FAIL(1, "qo_indptr decreases at request %d", r);
    if (n > lens[r])
      PLAN_FAIL(1, "request %d has %lld query tokens but %lld keys (the queries are the "
                   "last tokens of the cache)", r, (long long)n, (long long)lens[r]);
  }
  const int64_t total_q = B > 0 ? qo[B] : 0;
  const bool causal = in.causal != 0;
  // 4-wave (128-row) tiles when no (request, kv head) has more rows: an
  // 8-wave tile would leave half its waves without rows; two 4-wave
  // workgroups fit a CU
  int64_t rows_max = 0;
  for (int r = 0; r < B; ++r) rows_max = std::max<int64_t>(rows_max, (int64_t)(qo[r + 1] - qo[r]) * G);
  // (at head_dim 256 the 4-wave instance holds a CU alone: 8 waves; RoPE
  // tiles are built with 8 waves only)
  const bool rope = in.pos_encoding == 1;
  const int rpw = prefix_rows_per_wave(in.D, rope);
  const int waves =
      rope ? 8
           : tune_or(in.tune.prefix_waves, rows_max <= 4 * rpw && in.D != 256 ? 4 : 8) == 4 ? 4
                                                                                           : 8;
  const int64_t R = (int64_t)rpw * waves;   // rows per tile
  const int64_t slots_per_cu = waves == 4 ? 2 : 1;
  // row tiles: (request, rows [row0, row1), keys needed by the last row)
  struct RowTile {
    int r;
    int64_t row0, row1, keys;
  };
  std::vector<RowTile> rts;
  for (int r = 0; r < B; ++r) {
    const int64_t n = (int64_t)qo[r + 1] - qo[r], rows = n * G;
    for (int64_t a = 0; a < rows; a += R) {
      const int64_t b = std::min(a + R, rows), i_last = (b - 1) / G;
      rts.push_back(RowTile{r, a, b, causal ? lens[r] - n + i_last + 1 : lens[r]});
    }
  }
  int64_t kmax = 0;
  for (const RowTile& t : rts) kmax = std::max(kmax, t.keys);
  auto tiles_for = [&](int64_t c) {
    int64_t w = 0;
    for (const RowTile& t : rts) w += ceil_div(t.keys, c);
    return w * Hkv;
  };
  int64_t chunk;
  const int64_t hi = std::min<int64_t>(round_up(std::max<int64_t>(kmax, 1), kBlockTokens),
                                       kPrefixMaxChunk);
  if (in.chunk_tokens > 0) {
    chunk = std::min<int64_t>(round_up(in.chunk_tokens, kBlockTokens), kPrefixMaxChunk);
  } else {
    // about append_tiles_pct / 100 (1.25) tiles per resident workgroup, so
    // unequal requests even out; chunks of at least append_chunk_min keys
    const int64_t want = std::max<int64_t>(
        1, (int64_t)num_cus * slots_per_cu * tune_or(in.tune.append_tiles_pct, 125) / 100);
    if (rts.empty() || tiles_for(hi) >= want) {
      chunk = hi;
    } else {
      // smallest c in [lo, hi] (whole 32-token steps) with tiles(c) <= want
      const int64_t lo = std::min<int64_t>(
          round_up(std::max(tune_or(in.tune.append_chunk_min, 128), kBlockTokens), kBlockTokens),
          hi);
      int64_t a = lo / kBlockTokens, b = hi / kBlockTokens;
      while (a < b) {
        const int64_t mid = (a + b) / 2;
        if (tiles_for(mid * kBlockTokens) <= want) b = mid; else a = mid + 1;
      }
      chunk = a * kBlockTokens;
    }
  }

  // per request: its longest row tile's keys cut into ceil(keys / chunk)
  // chunks of near-equal length (whole 32-token steps), so no tile is a
  // short remainder; every row tile of the request uses the same boundaries
  // (up to its own last key), so the row tiles of a chunk read the same K/V
  std::vector<int64_t> req_cl(B, kBlockTokens);
  for (const RowTile& t : rts) {
    const int64_t nc = ceil_div(t.keys, chunk);
    req_cl[t.r] = std::max(req_cl[t.r], round_up(ceil_div(t.keys, nc), kBlockTokens));
  }
  auto chunk_len = [&](const RowTile& t) { return req_cl[t.r]; };
  auto n_chunks = [&](const RowTile& t) { return ceil_div(t.keys, req_cl[t.r]); };
  // per query token: states (chunks of its row tile), slots, merge units
  out->req_info = (ReqInfo*)malloc(sizeof(ReqInfo) * (size_t)std::max<int64_t>(total_q, 1));
  if (!out->req_info) PLAN_FAIL(1, "out of host memory");
  std::vector<MergeUnit> mu;
  int64_t slots = 0, max_states = 0;
  for (const RowTile& t : rts) {
    const int64_t n = (int64_t)qo[t.r + 1] - qo[t.r];
    const int64_t nc = n_chunks(t);
    max_states = std::max(max_states, nc);
    for (int64_t i = t.row0 / G; i <= (t.row1 - 1) / G; ++i) {
      ReqInfo& ri = out->req_info[qo[t.r] + i];
      ri.n_states = (int32_t)nc;
      ri.slot_base = -1;
      ri.kv_len = (int32_t)(causal ? lens[t.r] - n + i + 1 : lens[t.r]);
      ri.pad = 0;
      if (nc >= 2) {
        ri.slot_base = (int32_t)slots;
        slots += nc * Hkv;
        mu.push_back(MergeUnit{(int32_t)(qo[t.r] + i), ri.slot_base, (int32_t)nc, 0});
      }
      if (slots > (int64_t)0x7fffffff / (G * in.D))
        PLAN_FAIL(2, "too many partial states; raise chunk_tokens");
    }
  }
  // tiles: groups = (request, chunk, kv head), each holding its row tiles;
  // groups longest first (the kernel takes tiles in list order), and in
  // rounds of 8 groups the list interleaves row tiles (group x's row tile k
  // at 8 k + x of the round), so the row tiles of one group land on blocks
  // 8 apart -- the same XCD, dispatched together, sharing the chunk in L2
  struct Group {
    int64_t len;
    std::vector<Tile> tiles;
  };
  std::vector<Group> groups;
  for (size_t k = 0; k < rts.size();) {
    size_t e = k;
    while (e < rts.size() && rts[e].r == rts[k].r) ++e;
    int64_t ncmax = 0;
    for (size_t j = k; j < e; ++j) ncmax = std::max(ncmax, n_chunks(rts[j]));
    for (int64_t c = 0; c < ncmax; ++c)
      for (int h = 0; h < Hkv; ++h) {
        Group gr{0, {}};
        for (size_t j = k; j < e; ++j) {
          if (c >= n_chunks(rts[j])) continue;
          const int64_t cl = chunk_len(rts[j]);
          Tile t;
          t.req = rts[j].r;
          t.kv_head0 = h;
          t.t0 = (int32_t)std::min<int64_t>(c * cl, rts[j].keys);
          t.t1 = (int32_t)std::min<int64_t>((c + 1) * cl, rts[j].keys);
          t.slot = (int32_t)c;
          t.kind = kAppendTile;
          t.row0 = (int32_t)rts[j].row0;
          t.row1 = (int32_t)rts[j].row1;
          if (t.t1 <= t.t0) continue;
          gr.len = std::max<int64_t>(gr.len, t.t1 - t.t0);
          gr.tiles.push_back(t);
        }
        if (!gr.tiles.empty()) groups.push_back(std::move(gr));
      }
    k = e;
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group& a, const Group& b) { return a.len > b.len; });
  std::vector<Tile> at;
  for (size_t g0 = 0; g0 < groups.size(); g0 += 8) {
    const size_t g1 = std::min(groups.size(), g0 + 8);
    size_t kmax = 0;
    for (size_t g = g0; g < g1; ++g) kmax = std::max(kmax, groups[g].tiles.size());
    for (size_t k = 0; k < kmax; ++k)
      for (size_t g = g0; g < g1; ++g)
        if (k < groups[g].tiles.size()) at.push_back(groups[g].tiles[k]);
  }
  out->qo_indptr = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B + 1));
  out->merge_units = (MergeUnit*)malloc(sizeof(MergeUnit) * std::max<size_t>(mu.size(), 1));
  out->tiles = (Tile*)malloc(sizeof(Tile) * std::max<size_t>(at.size(), 1));
  if (!out->qo_indptr || !out->merge_units || !out->tiles) PLAN_FAIL(1, "out of host memory");
  for (int r = 0; r <= B; ++r) out->qo_indptr[r] = B > 0 ? qo[r] : 0;
  std::copy(mu.begin(), mu.end(), out->merge_units);
  std::copy(at.begin(), at.end(), out->tiles);

  out->batch = B; out->Hq = in.Hq; out->Hkv = Hkv; out->D = in.D;
  out->has_keys = std::any_of(lens.begin(), lens.end(), [](int64_t L) { return L > 0; });
  out->page_size = in.page_size; out->G = G; out->q_dtype = in.q_dtype;
  out->kv_dtype = in.kv_dtype; out->num_groups = 0; out->num_cus = num_cus;
  out->chunk_tokens = (int32_t)chunk;
  out->prefix_chunk_tokens = (int32_t)chunk;
  out->heads_per_tile = 1;
  out->prefix_waves = waves;
  out->num_tiles = 0;
  out->num_prefix_tiles = (int64_t)at.size();
  out->num_partials = slots;
  out->num_merge_units = (int64_t)mu.size();
  out->append = 1;
  out->causal = causal ? 1 : 0;
  out->ragged = in.ragged;
  out->hnd = in.hnd;
  out->merge_wide = mu.size() >= 128 && max_states <= 8;
  out->total_q = total_q;
  out->num_req_info = total_q;
  out->qo_len = B + 1;

  WorkspaceLayout& L = out->layout;
  size_t off = 0;
  L.tiles_off = off;
  off = align256(off + sizeof(Tile) * at.size());
  L.req_info_off = off;
  off = align256(off + sizeof(ReqInfo) * (size_t)std::max<int64_t>(total_q, 1));
  L.merge_reqs_off = off;
  off = align256(off + sizeof(MergeUnit) * std::max<size_t>(mu.size(), 1));
  L.qo_indptr_off = off;
  off = align256(off + sizeof(int32_t) * (size_t)(B + 1));
  // RoPE: query token i of request r (n tokens, L keys) sits at L - n + i
  // and key t at t; both are turned by those positions
  if (rope) {
    out->num_rope_qpos = total_q;
    out->rope_qpos = (int32_t*)malloc(sizeof(int32_t) * (size_t)std::max<int64_t>(total_q, 1));
    if (!out->rope_qpos) PLAN_FAIL(1, "out of host memory");
    for (int r = 0; r < B; ++r) {
      const int64_t n = (int64_t)qo[r + 1] - qo[r];
      for (int64_t i = 0; i < n; ++i) out->rope_qpos[qo[r] + i] = (int32_t)(lens[r] - n + i);
    }
  }
  L.rope_qpos_off = off;
  off = align256(off + sizeof(int32_t) * (size_t)out->num_rope_qpos);
  L.partial_o_off = off;
  off = align256(off + sizeof(float) * (size_t)slots * G * in.D);
  L.partial_lse_off = off;
  off = align256(off + sizeof(float) * (size_t)slots * G);
  out->rope = rope ? 1 : 0;
  out->rope_theta = in.rope_theta > 0.f ? in.rope_theta : 1e4f;
  out->rope_scale = in.rope_scale > 0.f ? in.rope_scale : 1.f;
  int64_t Lmax = 0;
  for (int r = 0; r < B; ++r) Lmax = std::max(Lmax, lens[r]);
  out->rope_rows = rope ? (int32_t)std::max<int64_t>(Lmax, kChunkAlign) : 0;
  L.rope_off = off;
  off = align256(off + (size_t)rope_row_bytes(in.D) * (size_t)out->rope_rows);
  L.total = off;
  return 0;
}

}  // namespace

// Checks the dimensions, layout, tuning and the per-request table (no
// allocation): 0 or an fi_status code with `err` filled.
int check_problem(const PlanInput& in, char* err, size_t errlen) {
  const int B = in.batch, Hkv = in.Hkv, ps = in.page_size;
  if (B < 0) PLAN_FAIL(1, "batch must be >= 0 (got %d)", B);
  if (in.Hq <= 0 || Hkv <= 0 || in.Hq % Hkv != 0)
    PLAN_FAIL(1, "num_qo_heads (%d) must be a positive multiple of num_kv_heads (%d)",
              in.Hq, Hkv);
  const int G = in.Hq / Hkv;
  if (G > kMaxGroup)
    PLAN_FAIL(2, "group size %d > %d q heads per kv head is not built", G, kMaxGroup);
  if (in.D != 64 && in.D != 128 && in.D != 256)
    PLAN_FAIL(2, "head_dim %d not built (64, 128 or 256)", in.D);
  if (ps <= 0) PLAN_FAIL(1, "page_size must be >= 1 (got %d)", ps);
  if ((in.ragged != 0 && in.ragged != 1) || (in.hnd != 0 && in.hnd != 1) ||
      (in.ragged && in.hnd))
    PLAN_FAIL(1, "kv_layout must be FI_KV_PAGED, FI_KV_RAGGED or FI_KV_PAGED_HND");
  if ((int64_t)ps * Hkv * in.D * 2 > 0x7fffffff)
    PLAN_FAIL(2, "a page of %d tokens x %d kv heads is too large", ps, Hkv);
  if (in.ragged && ps != 1) PLAN_FAIL(1, "a ragged KV layout has page_size 1 (got %d)", ps);
  const int32_t* last_tab = in.ragged ? nullptr : in.last_page_len;
  if (B > 0 && (!in.kv_indptr || (!in.ragged && !in.last_page_len)))
    PLAN_FAIL(1, "kv_indptr and last_page_len (host) are required");
  if (in.chunk_tokens < 0 || in.chunk_tokens % kChunkAlign != 0)
    PLAN_FAIL(1, "chunk_tokens must be 0 or a positive multiple of %d", kChunkAlign);
  {
    const Tuning& tu = in.tune;
    const int32_t counts[] = {tu.heads_per_tile, tu.waves_per_cu, tu.chunk_min,
                              tu.prefix_waves, tu.prefix_tiles_per_cu, tu.prefix_chunk_min,
                              tu.fold_max_suffix, tu.append_tiles_pct, tu.append_chunk_min};
    for (int32_t c : counts)
      if (c < 0) PLAN_FAIL(1, "tuning values must be >= 0 (0 = default)");
    if (tu.decode_depth < 0 || tu.decode_depth > 2)
      PLAN_FAIL(1, "tuning decode_depth must be 0 (automatic), 1 or 2");
    if (tu.cascade_fold < -1 || tu.cascade_fold > 1 || tu.prefix_split_p < -1 ||
        tu.prefix_split_p > 1 || tu.rope_split_k < -1 || tu.rope_split_k > 1)
      PLAN_FAIL(1, "tuning cascade_fold, prefix_split_p and rope_split_k must be -1, 0 or 1");
    if (tu.score_path < 0 || tu.score_path > 2)
      PLAN_FAIL(1, "tuning score_path must be 0 (automatic), 1 (MFMA) or 2 (VALU)");
  }
  // paged tables index kv_indices from 0; a ragged table's entries are the
  // requests' first rows in K / V, anywhere
  if (B > 0 && !in.ragged && in.kv_indptr[0] != 0) PLAN_FAIL(1, "kv_indptr[0] must be 0");
  if (B > 0 && in.kv_indptr[0] < 0) PLAN_FAIL(1, "kv_indptr[0] must be >= 0");
  for (int r = 0; r < B; ++r) {
    if (in.kv_indptr[r + 1] < in.kv_indptr[r])
      PLAN_FAIL(1, "kv_indptr decreases at request %d", r);
    int64_t n = (int64_t)in.kv_indptr[r + 1] - in.kv_indptr[r];
    if (n > 0 && last_tab && (last_tab[r] < 1 || last_tab[r] > ps))
      PLAN_FAIL(1, "last_page_len[%d] = %d outside [1, %d]", r, last_tab[r], ps);
    if (table_len(in.kv_indptr, last_tab, r, ps) > (int64_t)0x7fffffff - 64)
      PLAN_FAIL(1, "request %d too long", r);
  }
  return 0;
}

int plan_build(const PlanInput& in, HostPlan* out, char* err, size_t errlen) {
  memset(out, 0, sizeof(*out));
  const int B = in.batch, Hkv = in.Hkv, ps = in.page_size;
  {
    const int rc = check_problem(in, err, errlen);
    if (rc) return rc;
  }
  const int G = in.Hq / Hkv;
  const int32_t* last_tab = in.ragged ? nullptr : in.last_page_len;
  std::vector<int64_t> lens(B);
  for (int r = 0; r < B; ++r) lens[r] = table_len(in.kv_indptr, last_tab, r, ps);
  // ---- shared (cascade) levels, outermost first; each splits the requests
  // into groups of contiguous requests sharing a prefix table
  const int NL = in.num_levels;
  if (NL < 0)
    PLAN_FAIL(1, "cascade levels: give either the single-level prefix fields or a non-NULL "
                 "level array, not both");
  if (NL > kMaxLevels) PLAN_FAIL(2, "%d cascade levels (at most %d are built)", NL, kMaxLevels);
  std::vector<std::vector<int64_t>> plens(NL);       // [level][group] prefix tokens
  std::vector<std::vector<int>> group_of(NL, std::vector<int>(B, -1));
  int NG = 0;                                         // groups over all levels
  for (int l = 0; l < NL; ++l) {
    const PlanInput::Level& lv = in.levels[l];
    const int ng = lv.num_groups;
    if (ng < 0) PLAN_FAIL(1, "num_prefix_groups must be >= 0 (level %d)", l);
    NG += ng;
    plens[l].assign(ng, 0);
    if (ng == 0) continue;
    if (!lv.qo_indptr || !lv.p_indptr || (!in.ragged && !lv.p_last))
      PLAN_FAIL(1, "cascade level %d needs prefix_qo_indptr, prefix_kv_indptr, "
                   "prefix_last_page_len (host)", l);
    if (lv.qo_indptr[0] != 0 || lv.qo_indptr[ng] != B)
      PLAN_FAIL(1, "prefix_qo_indptr must start at 0 and end at batch (level %d)", l);
    if (!in.ragged && lv.p_indptr[0] != 0)
      PLAN_FAIL(1, "prefix_kv_indptr[0] must be 0 (level %d)", l);
    if (lv.p_indptr[0] < 0) PLAN_FAIL(1, "prefix_kv_indptr[0] must be >= 0 (level %d)", l);
    for (int g = 0; g < ng; ++g) {
      if (lv.qo_indptr[g + 1] < lv.qo_indptr[g])
        PLAN_FAIL(1, "prefix_qo_indptr decreases at group %d (level %d)", g, l);
      if (lv.p_indptr[g + 1] < lv.p_indptr[g])
        PLAN_FAIL(1, "prefix_kv_indptr decreases at group %d (level %d)", g, l);
      int64_t n = (int64_t)lv.p_indptr[g + 1] - lv.p_indptr[g];
      if (n > 0 && !in.ragged && (lv.p_last[g] < 1 || lv.p_last[g] > ps))
        PLAN_FAIL(1, "prefix_last_page_len[%d] outside [1, %d] (level %d)", g, ps, l);
      plens[l][g] = table_len(lv.p_indptr, in.ragged ? nullptr : lv.p_last, g, ps);
      for (int r = lv.qo_indptr[g]; r < lv.qo_indptr[g + 1]; ++r) group_of[l][r] = g;
    }
  }
  auto has_prefix = [&](int r) {
    for (int l = 0; l < NL; ++l)
      if (group_of[l][r] >= 0 && plens[l][group_of[l][r]] > 0) return true;
    return false;
  };
  const int num_cus = in.num_cus > 0 ? in.num_cus : 256;
  if (in.pos_encoding != 0 && in.pos_encoding != 1)
    PLAN_FAIL(1, "pos_encoding must be FI_POS_NONE or FI_POS_ROPE_LLAMA (got %d)",
              in.pos_encoding);
  const bool rope = in.pos_encoding == 1;
  if (rope && (!(in.rope_theta == in.rope_theta) || !(in.rope_scale == in.rope_scale) ||
               in.rope_theta > 1e30f || in.rope_scale > 1e30f))
    PLAN_FAIL(1, "rope_theta and rope_scale must be finite");
  if (in.append_qo_indptr) {
    if (NG > 0) PLAN_FAIL(2, "append with a cascade level is not built");
    return plan_append(in, lens, num_cus, out, err, errlen);
  }
  // RoPE with cascade levels: every key's index in its request's whole key
  // list (earlier levels, then own pages) must fit the table's int32 rows
  std::vector<int64_t> total_len(lens);
  for (int r = 0; r < B; ++r) {
    for (int l = 0; l < NL; ++l)
      if (group_of[l][r] >= 0) total_len[r] += plens[l][group_of[l][r]];
    if (rope && total_len[r] > (int64_t)0x7fffffff - 64)
      PLAN_FAIL(1, "request %d: its keys over all cascade levels are too many", r);
  }

  // ---- decode chunk length and heads per tile
  // fp16 q (or bf16 q over e4m3 K/V, which the decode kernel then computes
  // in fp16): the turned key as one fp16 value when every request is long
  // enough for its rounding to stay well inside the lse bar (plain decode:
  // a cascade's multi-row tiles read the fp32 table); (the step's fp16 table
  // rows are copied by one 16-byte vector per thread: 2 D bytes x 16 rows
  // need 32 D / 16 threads, so tiles of hpt >= D / 32 waves)
  int64_t shortest = -1;
  for (int r = 0; r < B; ++r)
    if (lens[r] > 0) shortest = shortest < 0 ? lens[r] : std::min(shortest, lens[r]);
  auto rope_single_at = [&](int h) {
    return rope && (in.q_dtype == 0 || in.kv_dtype == 2) && NL == 0 && h * 32 >= in.D &&
           (in.tune.rope_split_k < 0 || (in.tune.rope_split_k == 0 && shortest >= kRopeSingleKeys));
  };
  const bool fold_ok = in.tune.cascade_fold >= 0 && !rope;   // no RoPE fold instance
  auto resident = [&](int h) {
    if (!in.resident_waves) return 0;
    return in.resident_waves(in.resident_ctx, h, !rope ? 0 : rope_single_at(h) ? 2 : 1,
                             NG > 0 && fold_ok ? 1 : 0);
  };
  const bool hpt_forced = in.tune.heads_per_tile > 0;
  int hpt;
  int64_t chunk;
  int wpc = 16;
  decode_split(in, num_cus, rope, [&](int r) { return lens[r]; }, resident, &hpt, &chunk, &wpc);
  out->decode_waves_per_cu = wpc;
  // Cascade: a request with prefix states whose suffix is one chunk folds
  // those states into its decode tile's output, so no merge pass is needed.
  // When every such suffix is short (<= tune.fold_max_suffix tokens, default
  // 1024), cover each with one chunk, 2 kv heads per tile (small tiles, two
  // steps of loads in flight), provided that still gives >= 4 waves per CU.
  if (NG > 0 && fold_ok && in.chunk_tokens == 0 && !hpt_forced) {
    int64_t ls_max = 0;
    for (int r = 0; r < B; ++r)
      if (has_prefix(r)) ls_max = std::max(ls_max, lens[r]);
    const int hpt_f = Hkv % 2 == 0 ? 2 : 1;
    if (ls_max > 0 && ls_max <= tune_or(in.tune.fold_max_suffix, 1024)) {
      const int64_t chunk_f = round_up(ls_max, kChunkAlign);
      int64_t w = 0;
      for (int r = 0; r < B; ++r) w += std::max<int64_t>(1, ceil_div(lens[r], chunk_f));
      if (w * Hkv >= 4 * (int64_t)num_cus) {
        hpt = hpt_f;
        chunk = chunk_f;
      }
    }
  }
  const int64_t head_groups = Hkv / hpt;   // decode tiles per (request, chunk)

  // ---- cascade prefix chunking
  // (RoPE multi-row tiles are built with 8 waves only)
  const int prefix_waves =
      rope ? kPrefixMaxWaves : tune_or(in.tune.prefix_waves, kPrefixMaxWaves) == 4 ? 4 : 8;
  const int64_t prefix_rows = (int64_t)prefix_rows_per_wave(in.D, rope) * prefix_waves;
  int64_t prefix_chunk = 0;
  std::vector<std::vector<int64_t>> n_pchunks(NL);   // [level][group] chunks
  int64_t prefix_row_tiles = 0;  // sum over levels and groups of row tiles x Hkv
  int64_t Lpmax = 0;
  for (int l = 0; l < NL; ++l)
    for (int g = 0; g < in.levels[l].num_groups; ++g) {
      const int64_t rows =
          (int64_t)(in.levels[l].qo_indptr[g + 1] - in.levels[l].qo_indptr[g]) * G;
      if (plens[l][g] > 0) prefix_row_tiles += ceil_div(rows, prefix_rows) * Hkv;
      Lpmax = std::max(Lpmax, plens[l][g]);
    }
  if (prefix_row_tiles > 0) {
    const int64_t want =
        std::max<int64_t>(1, (int64_t)num_cus * std::max(1, tune_or(in.tune.prefix_tiles_per_cu, 1)));
    int64_t n_split = std::max<int64_t>(1, ceil_div(want, prefix_row_tiles));
    prefix_chunk = round_up(ceil_div(Lpmax, n_split), kBlockTokens);
    prefix_chunk = std::max<int64_t>(prefix_chunk, tune_or(in.tune.prefix_chunk_min, 256));
    prefix_chunk = round_up(prefix_chunk, kBlockTokens);
    // a prefix tile stages its chunk's page indices in LDS (<= 4096 + 2)
    prefix_chunk = std::min<int64_t>(prefix_chunk, kPrefixMaxChunk);
  }
  for (int l = 0; l < NL; ++l) {
    n_pchunks[l].assign(in.levels[l].num_groups, 0);
    for (int g = 0; g < in.levels[l].num_groups; ++g)
      n_pchunks[l][g] =
          (plens[l][g] > 0 && prefix_chunk > 0) ? ceil_div(plens[l][g], prefix_chunk) : 0;
  }
  // request r's prefix states: level by level, outermost first
  std::vector<int64_t> np_of(B, 0);
  std::vector<int32_t> state_off((size_t)std::max(NL, 1) * std::max(B, 1), 0);
  for (int r = 0; r < B; ++r)
    for (int l = 0; l < NL; ++l) {
      state_off[(size_t)l * B + r] = (int32_t)np_of[r];
      if (group_of[l][r] >= 0) np_of[r] += n_pchunks[l][group_of[l][r]];
    }

  // ---- states per request, slots
  // A request with prefix states and a suffix that is one decode chunk is
  // "folded": its decode tile reads the prefix states and writes the final
  // output, so only the prefix states need slots and no merge unit is made
  // (tune.cascade_fold = -1 sends every such request through the merge kernel).
  std::vector<int64_t> n_dchunks(B);
  std::vector<char> folded(B, 0);
  for (int r = 0; r < B; ++r) n_dchunks[r] = lens[r] > 0 ? ceil_div(lens[r], chunk) : 0;
  out->req_info = (ReqInfo*)malloc(sizeof(ReqInfo) * std::max(B, 1));
  if (!out->req_info) PLAN_FAIL(1, "out of host memory");
  int64_t slots = 0, n_merge = 0;
  for (int r = 0; r < B; ++r) {
    const int64_t np = np_of[r];
    int64_t ns = n_dchunks[r] + np;
    folded[r] = fold_ok && np > 0 && n_dchunks[r] == 1;
    out->req_info[r].n_states = (int32_t)ns;
    out->req_info[r].slot_base = -1;
    out->req_info[r].kv_len = (int32_t)lens[r];
    out->req_info[r].pad = 0;
    if (ns >= 2) {
      out->req_info[r].slot_base = (int32_t)slots;
      slots += (folded[r] ? np : ns) * Hkv;
      if (!folded[r]) ++n_merge;
    }
    if (slots > (int64_t)0x7fffffff / (G * in.D))
      PLAN_FAIL(2, "too many partial states; raise chunk_tokens");
  }
  out->merge_units = (MergeUnit*)malloc(sizeof(MergeUnit) * std::max<int64_t>(n_merge, 1));
  if (!out->merge_units) PLAN_FAIL(1, "out of host memory");
  {
    int64_t k = 0;
    for (int r = 0; r < B; ++r)
      if (out->req_info[r].n_states >= 2 && !folded[r])
        out->merge_units[k++] = MergeUnit{r, out->req_info[r].slot_base,
                                          out->req_info[r].n_states, 0};
  }

  // ---- decode tiles
  std::vector<Tile> dt;
  for (int r = 0; r < B; ++r) {
    const int64_t c_off = np_of[r];
    const ReqInfo& ri = out->req_info[r];
    int64_t nc = n_dchunks[r];
    bool need_empty = (nc == 0 && ri.n_states == 0);
    // the request's steps shared out over its nc chunks as evenly as whole
    // steps allow (the first ones one step longer), so no chunk is a short
    // remainder: each is at most the chunk length and at least one step
    const int64_t nsteps = ceil_div(lens[r], (int64_t)kChunkAlign);
    const int64_t per = nc > 0 ? nsteps / nc : 0, extra = nc > 0 ? nsteps % nc : 0;
    auto bound = [&](int64_t c) {
      return std::min<int64_t>((int64_t)kChunkAlign * (c * per + std::min(c, extra)), lens[r]);
    };
    for (int64_t c = 0; c < std::max<int64_t>(nc, need_empty ? 1 : 0); ++c) {
      for (int64_t hg = 0; hg < head_groups; ++hg) {
        Tile t;
        t.req = r;
        t.kv_head0 = (int32_t)(hg * hpt);
        t.t0 = (int32_t)bound(c);
        t.t1 = (int32_t)bound(c + 1);
        t.slot = ri.n_states >= 2 && !folded[r]
                     ? (int32_t)(ri.slot_base + (c_off + c) * Hkv + t.kv_head0) : -1;
        t.kind = kDecodeTile;
        t.row0 = in.kv_indptr[r];   // the request's first page-table entry
        t.row1 = folded[r] ? (int32_t)c_off : 0;   // prefix states to fold in
        dt.push_back(t);
      }
    }
  }
  std::stable_sort(dt.begin(), dt.end(), [](const Tile& a, const Tile& b) {
    return (a.t1 - a.t0) > (b.t1 - b.t0);
  });
  {
    std::vector<int64_t> w(dt.size()), pos;
    for (size_t i = 0; i < dt.size(); ++i) w[i] = dt[i].t1 - dt[i].t0;
    dispatch_order(w, num_cus, &pos);
    std::vector<Tile> placed(dt.size());
    for (size_t i = 0; i < dt.size(); ++i) placed[pos[i]] = dt[i];
    dt.swap(placed);
  }
  // ---- prefix tiles, level by level: chunk-major, row tiles of one
  // (group, head, chunk) adjacent so they run together and share the chunk's
  // K/V in cache
  std::vector<Tile> pt;
  out->num_levels = NL;
  int32_t qo_entries = 0;
  for (int l = 0; l < NL; ++l) {
    out->level_tile_off[l] = (int64_t)pt.size();
    out->level_qo_start[l] = qo_entries;
    out->level_groups[l] = in.levels[l].num_groups;
    qo_entries += in.levels[l].num_groups + 1;
    for (int g = 0; g < in.levels[l].num_groups; ++g) {
      const int64_t rows =
          (int64_t)(in.levels[l].qo_indptr[g + 1] - in.levels[l].qo_indptr[g]) * G;
      if (plens[l][g] == 0 || rows == 0) continue;
      const int64_t nrt = ceil_div(rows, prefix_rows);
      for (int64_t pc = 0; pc < n_pchunks[l][g]; ++pc)
        for (int h = 0; h < Hkv; ++h)
          for (int64_t rt = 0; rt < nrt; ++rt) {
            Tile t;
            t.req = g;
            t.kv_head0 = h;
            t.t0 = (int32_t)(pc * prefix_chunk);
            t.t1 = (int32_t)std::min<int64_t>((pc + 1) * prefix_chunk, plens[l][g]);
            t.slot = (int32_t)pc;   // chunk of this level; + state_off[l][r]
            t.kind = kPrefixTile;
            t.row0 = (int32_t)(rt * prefix_rows);
            t.row1 = (int32_t)std::min<int64_t>((rt + 1) * prefix_rows, rows);
            pt.push_back(t);
          }
    }
  }
  out->level_tile_off[NL] = (int64_t)pt.size();
  // bf16 K/V: a level whose shortest prefix has fewer than kSplitPKeys keys
  // runs the prefix instance that passes p to P.V with a residual
  out->prefix_split_p = 0;
  for (int l = 0; l < NL && in.q_dtype == 1 && in.kv_dtype == 1; ++l) {
    int64_t shortest = -1;
    for (int g = 0; g < in.levels[l].num_groups; ++g)
      if (plens[l][g] > 0 && in.levels[l].qo_indptr[g + 1] > in.levels[l].qo_indptr[g])
        shortest = shortest < 0 ? plens[l][g] : std::min(shortest, plens[l][g]);
    const bool split = in.tune.prefix_split_p > 0 ||
                       (in.tune.prefix_split_p == 0 && shortest >= 0 && shortest < kSplitPKeys);
    if (split) out->prefix_split_p |= 1u << l;
  }
  out->qo_indptr = (int32_t*)malloc(sizeof(int32_t) * (size_t)std::max(qo_entries, 1));
  out->state_off = (int32_t*)malloc(sizeof(int32_t) * state_off.size());
  if (!out->qo_indptr || !out->state_off) PLAN_FAIL(1, "out of host memory");
  out->qo_indptr[0] = 0;
  for (int l = 0; l < NL; ++l)
    for (int g = 0; g <= in.levels[l].num_groups; ++g)
      out->qo_indptr[out->level_qo_start[l] + g] = in.levels[l].qo_indptr[g];
  std::copy(state_off.begin(), state_off.end(), out->state_off);
  out->num_tiles = (int64_t)dt.size();
  out->num_prefix_tiles = (int64_t)pt.size();
  out->tiles = (Tile*)malloc(sizeof(Tile) * std::max<size_t>(dt.size() + pt.size(), 1));
  if (!out->tiles) PLAN_FAIL(1, "out of host memory");
  std::copy(dt.begin(), dt.end(), out->tiles);
  std::copy(pt.begin(), pt.end(), out->tiles + dt.size());

  out->batch = B; out->Hq = in.Hq; out->Hkv = Hkv; out->D = in.D;
  out->has_keys = std::any_of(lens.begin(), lens.end(), [](int64_t L) { return L > 0; });
  out->page_size = ps; out->G = G; out->q_dtype = in.q_dtype;
  out->kv_dtype = in.kv_dtype; out->num_groups = NG; out->num_cus = num_cus;
  out->chunk_tokens = (int32_t)chunk;
  out->prefix_chunk_tokens = (int32_t)prefix_chunk;
  out->heads_per_tile = hpt;
  out->prefix_waves = prefix_waves;
  out->num_partials = slots;
  out->num_merge_units = n_merge;
  {
    int32_t ms = 0;
    for (int64_t k = 0; k < n_merge; ++k) ms = std::max(ms, out->merge_units[k].n_states);
    out->merge_wide = n_merge >= 128 && ms <= 8;   // many units, few states each
  }
  out->num_folded = 0;
  for (int r = 0; r < B; ++r) out->num_folded += folded[r] ? 1 : 0;
  out->decode_depth = in.tune.decode_depth;
  out->num_req_info = B;
  out->qo_len = std::max(qo_entries, 1);
  out->ragged = in.ragged;
  out->hnd = in.hnd;

  WorkspaceLayout& L = out->layout;
  size_t off = 0;
  L.tiles_off = off;
  off = align256(off + sizeof(Tile) * (dt.size() + pt.size()));
  L.req_info_off = off;
  off = align256(off + sizeof(ReqInfo) * (size_t)std::max(B, 1));
  L.merge_reqs_off = off;
  off = align256(off + sizeof(MergeUnit) * (size_t)std::max<int64_t>(n_merge, 1));
  L.qo_indptr_off = off;
  off = align256(off + sizeof(int32_t) * (size_t)out->qo_len);
  L.state_off_off = off;
  off = align256(off + sizeof(int32_t) * state_off.size());
  // RoPE with cascade levels: request r's rows in level l's tiles are turned
  // by their position counted from the start of that level's prefix
  if (rope && NL > 0) {
    out->num_rope_qpos = (int64_t)NL * B;
    out->rope_qpos = (int32_t*)malloc(sizeof(int32_t) * (size_t)std::max<int64_t>(NL * B, 1));
    if (!out->rope_qpos) PLAN_FAIL(1, "out of host memory");
    for (int r = 0; r < B; ++r) {
      int64_t before = 0;   // keys of the request's earlier levels
      for (int l = 0; l < NL; ++l) {
        out->rope_qpos[(size_t)l * B + r] = (int32_t)std::max<int64_t>(total_len[r] - 1 - before, 0);
        if (group_of[l][r] >= 0) before += plens[l][group_of[l][r]];
      }
    }
  }
  L.rope_qpos_off = off;
  off = align256(off + sizeof(int32_t) * (size_t)out->num_rope_qpos);
  L.partial_o_off = off;
  off = align256(off + sizeof(float) * (size_t)slots * G * in.D);
  L.partial_lse_off = off;
  off = align256(off + sizeof(float) * (size_t)slots * G);
  out->rope = rope ? 1 : 0;
  out->rope_theta = in.rope_theta > 0.f ? in.rope_theta : 1e4f;
  out->rope_scale = in.rope_scale > 0.f ? in.rope_scale : 1.f;
  // distances / positions 0 .. (longest key list over all levels) - 1, and
  // at least the 16 rows every decode tile stages
  int64_t Ltot = 0;
  for (int r = 0; r < B; ++r) Ltot = std::max(Ltot, total_len[r]);
  out->rope_rows = rope ? (int32_t)std::max<int64_t>(Ltot, kChunkAlign) : 0;
  // score path of plain decode: MFMA (default) or the VALU instance
  if (in.tune.score_path == 2) {
    if (rope || NG > 0 || in.D != 128 || G > 4)
      PLAN_FAIL(2, "the VALU score path serves plain decode at head_dim 128 with at most 4 "
                   "q heads per kv head");
    out->valu_heads = G == 1 ? 1 : G == 2 ? 2 : 4;
  }
  out->rope_single = rope_single_at(hpt);
  L.rope_off = off;
  off = align256(off + (size_t)rope_row_bytes(in.D) * (size_t)out->rope_rows);
  L.total = off;
  return 0;
}

int plan_decode_static(const PlanInput& in, size_t max_bytes, HostPlan* out, char* err,
                       size_t errlen) {
  memset(out, 0, sizeof(*out));
  {
    const int rc = check_problem(in, err, errlen);
    if (rc) return rc;
  }
  if (in.num_levels != 0 || in.append_qo_indptr || in.pos_encoding != 0)
    PLAN_FAIL(2, "the allocation-free entry point runs plain decode only (no cascade level, "
                 "append or RoPE)");
  const int B = in.batch, Hkv = in.Hkv, ps = in.page_size, G = in.Hq / in.Hkv;
  const int num_cus = in.num_cus > 0 ? in.num_cus : 256;
  const int32_t* last_tab = in.ragged ? nullptr : in.last_page_len;
  auto len = [&](int r) { return table_len(in.kv_indptr, last_tab, r, ps); };
  int hpt;
  int64_t chunk;
  decode_split(
      in, num_cus, false, len,
      [&](int h) { return in.resident_waves ? in.resident_waves(in.resident_ctx, h, 0, 0) : 0; },
      &hpt, &chunk, &out->decode_waves_per_cu);
  // the work list in scratch: tiles, request info, merge units, partial
  // states (the same counts the device planner derives from the tables)
  auto layout = [&](int64_t c, WorkspaceLayout* L, int64_t* tiles, int64_t* units,
                    int64_t* slots, int32_t* max_states) {
    *tiles = *units = *slots = 0;
    *max_states = 0;
    for (int r = 0; r < B; ++r) {
      const int64_t nc = len(r) > 0 ? ceil_div(len(r), c) : 0;
      *tiles += std::max<int64_t>(nc, 1) * (Hkv / hpt);
      if (nc >= 2) {
        *slots += nc * Hkv;
        *units += 1;
        *max_states = std::max<int32_t>(*max_states, (int32_t)nc);
      }
    }
    size_t off = 0;
    L->tiles_off = off;
    off = align256(off + sizeof(Tile) * (size_t)*tiles);
    L->req_info_off = off;
    off = align256(off + sizeof(ReqInfo) * (size_t)std::max(B, 1));
    L->merge_reqs_off = off;
    off = align256(off + sizeof(MergeUnit) * (size_t)std::max<int64_t>(*units, 1));
    L->qo_indptr_off = off;
    L->state_off_off = off;
    L->partial_o_off = off;
    off = align256(off + sizeof(float) * (size_t)*slots * G * in.D);
    L->partial_lse_off = off;
    off = align256(off + sizeof(float) * (size_t)*slots * G);
    L->rope_off = off;
    L->total = off;
  };
  WorkspaceLayout L;
  int64_t tiles, units, slots;
  int32_t max_states;
  layout(chunk, &L, &tiles, &units, &slots, &max_states);
  if (L.total > max_bytes && in.chunk_tokens == 0) {
    // fewer, longer chunks until the partial states fit (unsplit needs none)
    int64_t Lmax = 16;
    for (int r = 0; r < B; ++r) Lmax = std::max(Lmax, len(r));
    while (L.total > max_bytes && chunk < Lmax) {
      chunk = std::min<int64_t>(round_up(2 * chunk, kChunkAlign), round_up(Lmax, kChunkAlign));
      layout(chunk, &L, &tiles, &units, &slots, &max_states);
    }
  }
  if (L.total > max_bytes)
    PLAN_FAIL(1, "the allocation-free entry point needs %zu bytes of device scratch for this "
                 "batch (chunk %lld tokens); its static buffer holds %zu (use a larger "
                 "chunk_tokens, a smaller batch, or fi_plan with a workspace)",
              L.total, (long long)chunk, max_bytes);
  if (slots > (int64_t)0x7fffffff / (G * in.D) || tiles > 0x7fffffff)
    PLAN_FAIL(2, "too many tiles or partial states; raise chunk_tokens");
  out->batch = B; out->Hq = in.Hq; out->Hkv = Hkv; out->D = in.D;
  out->page_size = ps; out->G = G; out->q_dtype = in.q_dtype; out->kv_dtype = in.kv_dtype;
  out->num_cus = num_cus;
  out->chunk_tokens = (int32_t)chunk;
  out->heads_per_tile = hpt;
  out->prefix_waves = kPrefixMaxWaves;
  out->num_tiles = tiles;
  out->num_partials = slots;
  out->num_merge_units = units;
  out->merge_wide = units >= 128 && max_states <= 8;
  out->num_req_info = B;
  out->qo_len = 1;
  out->ragged = in.ragged;
  out->hnd = in.hnd;
  out->decode_depth = in.tune.decode_depth;
  for (int r = 0; r < B && !out->has_keys; ++r) out->has_keys = len(r) > 0;
  out->layout = L;
  return 0;
}

void plan_free(HostPlan* p) {
  if (!p) return;
  free(p->tiles);
  free(p->req_info);
  free(p->merge_units);
  free(p->qo_indptr);
  free(p->state_off);
  free(p->rope_qpos);
  p->rope_qpos = nullptr;
  p->qo_indptr = nullptr;
  p->state_off = nullptr;
  p->tiles = nullptr;
  p->req_info = nullptr;
  p->merge_units = nullptr;
}

}  // namespace fi
