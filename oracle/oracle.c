/*
 * oracle.c -- plain, slow, fp64 CPU oracle for paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (one query token per head, exact attention):
 *   FlashInfer README, "core features" item 1: single/batch attention over
 *   sparse (paged) or dense KV storage; "vector-sparse" = page size 1.
 *   Dao-AILab/flash-attention summary, "How it works": the method is EXACT
 *   attention, so the plain definition softmax(q.K^T * scale).V is the
 *   reference and every faster schedule may only change rounding.
 *   hysenlabs review, "Installing FlashInfer and running a first decode":
 *   q is [num_qo_heads, head_dim], k and v are [kv_len, num_kv_heads,
 *   head_dim]; here K/V live in pages [num_pages][page_size][Hkv][D] that a
 *   request reaches through kv_indptr / kv_indices / last_page_len (the
 *   paged-call vocabulary of the "Pre-compiled cubins for FlashInfer"
 *   registry quickstart).
 *   FlashInfer README, "core features" item 3: grouped-query heads share a
 *   kv head (head-query fusion), low-precision KV, cascade attention over a
 *   hierarchical (shared prefix + per-request suffix) KV cache.
 *
 * Readings of points the pages leave open (each one is listed in the design
 * notes as well):
 *   - q head j reads kv head j / G with G = Hq / Hkv (contiguous groups);
 *   - logical token t of a request lives in page kv_indices[indptr[r] + t/ps]
 *     at slot t mod ps; the last page holds last_page_len[r] valid tokens;
 *   - lse is the natural-log log-sum-exp of the scaled scores;
 *   - an empty request gives o = 0, lse = -inf;
 *   - fp8 is OCP E4M3FN (bias 7, max 448, S.1111.111 is NaN, no inf),
 *     dequantised value = decode(code) * scale[kv_head];
 *   - softmax is taken in two passes (max, then sums), in fp64, with dot
 *     products summed over d in ascending order;
 *   - "LLaMA style RoPE on-the-fly" (README decode example with
 *     pos_encoding_mode="ROPE_LLAMA"; "core features" item 3, fused-RoPE
 *     attention) -- the pages give no formula; read as rotate-half: for
 *     i < D/2, angle_i = (pos / rope_scale) * rope_theta^(-2 i / D) and the
 *     pair (x_i, x_{i+D/2}) turns by angle_i; key t of a request's key list
 *     (cascade: the group's prefix tokens, then the request's own) sits at
 *     position t, the query at position L - 1 (the token being decoded is
 *     the last one in the cache); V is not rotated.
 *   - page layout: NHD pages [num_pages][page_size][Hkv][D] by default; HND
 *     (the other value of the registry quickstart's kv_layout argument)
 *     stores each page head-major, [num_pages][Hkv][page_size][D];
 *   - append attention (README example: single_prefill_with_kv_cache with
 *     causal=True, whose queries are the newest 128 tokens of the KV cache;
 *     the README also points to batch forms of decode, append and
 *     prefill): request r has
 *     n_r = qo_indptr[r+1] - qo_indptr[r] query tokens, which are the LAST
 *     n_r of its L keys, so query i (0-based) sits at position L - n_r + i;
 *     with the causal mask it attends keys 0 .. L - n_r + i, without it all
 *     L keys.  n_r <= L is required.  Query rows are stored token-major
 *     ([total_q][Hq][D]) and so are o and lse.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_LEVELS 8

/* dtype codes used by this file's own entry points */
enum { OR_F16 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_F32 = 3, OR_F64 = 4 };

/* ---- scalar decoders, written from the format definitions ---------------- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1.0 + (double)f / 1024.0, e - 15);
  return s ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 (8 exponent bits, bias
 * 127, 7 fraction bits). */
double oracle_bf16_to_f64(uint16_t b) {
  int s = (b >> 15) & 1, e = (b >> 7) & 0xff, f = b & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* f * 2^-126 * 2^-7 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1.0 + (double)f / 128.0, e - 127);
  return s ? -v : v;
}

/* OCP 8-bit float E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; the
 * all-ones exponent still encodes normal numbers except mantissa 111 (NaN);
 * there is no infinity.  Largest finite value 1.75 * 2^8 = 448. */
double oracle_e4m3_to_f64(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 0xf, m = c & 0x7;
  double v;
  if (e == 15 && m == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

static double load_elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case OR_F16: return oracle_f16_to_f64(((const uint16_t*)base)[i]);
    case OR_BF16: return oracle_bf16_to_f64(((const uint16_t*)base)[i]);
    case OR_E4M3: return oracle_e4m3_to_f64(((const uint8_t*)base)[i]);
    case OR_F32: return (double)((const float*)base)[i];
    default: return ((const double*)base)[i];
  }
}

/* ---- the page-table walk --------------------------------------------------
 * Number of valid tokens of request r: (n_pages - 1) * ps + last_page_len,
 * or 0 when the request owns no page.  Ragged layout (FlashInfer README
 * "core features" item 1 and the hysenlabs review's feature list name a
 * ragged KV cache next to the paged one; read as each request's tokens
 * stored contiguously, rows indptr[r] .. indptr[r+1]-1 of one
 * [total_tokens][Hkv][D] array): indices == NULL and last == NULL, and
 * indptr counts tokens. */
static int64_t request_len(const int32_t* indptr, const int32_t* last, int r,
                           int ps) {
  int64_t n = (int64_t)indptr[r + 1] - indptr[r];
  if (!last) return n;   /* ragged */
  return n == 0 ? 0 : (n - 1) * ps + last[r];
}

/* Physical token slot (page * ps + slot) of logical token t of request r
 * (ragged: its row indptr[r] + t). */
static int64_t token_slot(const int32_t* indptr, const int32_t* indices,
                          int r, int64_t t, int ps) {
  if (!indices) return (int64_t)indptr[r] + t;
  int64_t page = indices[indptr[r] + t / ps];
  return page * ps + t % ps;
}

/* Writes the physical slot of every logical token of every request, in
 * request order then token order; returns the number written.  Test hook
 * that the GPU gather is compared against bit for bit. */
int64_t oracle_gather_map(int batch, int page_size, const int32_t* kv_indptr,
                          const int32_t* kv_indices,
                          const int32_t* last_page_len, int64_t* out) {
  int64_t k = 0;
  for (int r = 0; r < batch; ++r) {
    int64_t L = request_len(kv_indptr, last_page_len, r, page_size);
    for (int64_t t = 0; t < L; ++t)
      out[k++] = token_slot(kv_indptr, kv_indices, r, t, page_size);
  }
  return k;
}

/* ---- one (query row, key list) attention, the plain definition -----------
 * x_t = sm_scale * sum_d q[d] * k_t[d]   (d ascending)
 * M = max_t x_t ; l = sum_t exp(x_t - M) ; o[d] = sum_t exp(x_t - M) v_t[d] / l
 * lse = M + ln l ; empty key list: o = 0, lse = -inf.
 * Keys are given as element offsets (of the first element of each row) into
 * the K and V pools. */
typedef struct {
  const void* k_pool;
  const void* v_pool;
  int kv_dtype;
  int D;
  double k_scale, v_scale;
} kv_src;

/* Rotate-half RoPE of one D-vector at position pos (see the readings
 * above): out_i = x_i cos a_i - x_{i+D/2} sin a_i,
 * out_{i+D/2} = x_{i+D/2} cos a_i + x_i sin a_i, a_i = (pos / scale) *
 * theta^(-2 i / D).  out may not alias x. */
void oracle_rope_rotate(const double* x, int D, double pos, double theta, double scale,
                        double* out) {
  const int half = D / 2;
  for (int i = 0; i < half; ++i) {
    const double a = (pos / scale) * pow(theta, -2.0 * i / D);
    const double c = cos(a), s = sin(a);
    out[i] = x[i] * c - x[i + half] * s;
    out[i + half] = x[i + half] * c + x[i] * s;
  }
}

typedef struct {
  int on;
  double theta, scale;
} rope_t;

/* One query row over keys 0 .. L-1 of row_off; with RoPE the query sits at
 * position qpos. */
static void attend_row(const double* q, const int64_t* row_off, int64_t L,
                       const kv_src* src, double sm_scale, const rope_t* rope,
                       double qpos, double* x /*[L]*/, double* o, double* lse) {
  const int D = src->D;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (L == 0) {
    *lse = -INFINITY;
    return;
  }
  double qr[512], kr[512], kraw[512];   /* D <= 512 */
  if (rope->on)
    oracle_rope_rotate(q, D, qpos, rope->theta, rope->scale, qr);
  else
    for (int d = 0; d < D; ++d) qr[d] = q[d];
  double M = -INFINITY;
  for (int64_t t = 0; t < L; ++t) {
    for (int d = 0; d < D; ++d)
      kraw[d] = load_elem(src->k_pool, src->kv_dtype, row_off[t] + d) * src->k_scale;
    if (rope->on)
      oracle_rope_rotate(kraw, D, (double)t, rope->theta, rope->scale, kr);
    else
      for (int d = 0; d < D; ++d) kr[d] = kraw[d];
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qr[d] * kr[d];
    x[t] = sm_scale * dot;
    if (x[t] > M) M = x[t];
  }
  double l = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    double p = exp(x[t] - M);
    l += p;
    for (int d = 0; d < D; ++d)
      o[d] += p * (load_elem(src->v_pool, src->kv_dtype, row_off[t] + d) *
                   src->v_scale);
  }
  for (int d = 0; d < D; ++d) o[d] /= l;
  *lse = M + log(l);
}

/* ---- batch driver ---------------------------------------------------------
 * Work item = (request r, kv head h); a pool of threads takes items from an
 * atomic counter.  The arithmetic of an item does not depend on which thread
 * runs it. */
typedef struct {
  int batch, Hq, Hkv, D, ps, q_dtype, kv_dtype;
  const void* q;
  const void* k_pages;
  const void* v_pages;
  /* level 0: per-request table (always present) */
  const int32_t *indptr, *indices, *last;
  /* optional shared levels, outermost first: level l splits the requests
   * into groups of contiguous requests, each sharing a prefix table */
  int n_levels;
  struct {
    int n_groups;
    const int32_t *qo_indptr, *p_indptr, *p_indices, *p_last;
  } lv[ORACLE_MAX_LEVELS];
  const float *k_scale, *v_scale;
  double sm_scale;
  rope_t rope;
  /* append mode (app_qo_indptr != NULL): query tokens per request */
  const int32_t* app_qo_indptr;
  int causal;
  int hnd; /* pages head-major: [page][Hkv][ps][D] */
  const uint8_t* unit_mask; /* [batch*Hkv] or NULL: 1 = compute this item */
  double* o;                /* [batch][Hq][D] */
  double* lse;              /* [batch][Hq] */
  int64_t next;
  int64_t max_len;
} job_t;

static int group_of(const job_t* J, int l, int r) {
  for (int g = 0; g < J->lv[l].n_groups; ++g)
    if (r >= J->lv[l].qo_indptr[g] && r < J->lv[l].qo_indptr[g + 1]) return g;
  return -1;
}

/* Element offset of the row of (physical token slot, kv head): NHD pages
 * keep a token's heads together, HND pages a head's tokens. */
static int64_t row_offset(const job_t* J, int64_t slot, int h) {
  if (!J->hnd) return (slot * J->Hkv + h) * (int64_t)J->D;
  const int64_t page = slot / J->ps, sl = slot % J->ps;
  return ((page * J->Hkv + h) * J->ps + sl) * (int64_t)J->D;
}

static void run_item(const job_t* J, int r, int h, int64_t* rows, double* x,
                     double* qv) {
  const int G = J->Hq / J->Hkv, D = J->D;
  int64_t L = 0;
  /* key list = (prefix tokens of the request's group at each shared level,
   * outermost first) ++ (its own tokens); decode has no mask, so the order
   * only fixes the summation order (and, with RoPE, the positions). */
  for (int l = 0; l < J->n_levels; ++l) {
    const int g = group_of(J, l, r);
    if (g < 0) continue;
    const int64_t Lp = request_len(J->lv[l].p_indptr, J->lv[l].p_last, g, J->ps);
    for (int64_t t = 0; t < Lp; ++t)
      rows[L++] = row_offset(
          J, token_slot(J->lv[l].p_indptr, J->lv[l].p_indices, g, t, J->ps), h);
  }
  int64_t Ls = request_len(J->indptr, J->last, r, J->ps);
  for (int64_t t = 0; t < Ls; ++t)
    rows[L++] = row_offset(J, token_slot(J->indptr, J->indices, r, t, J->ps), h);
  kv_src src = {J->k_pages, J->v_pages, J->kv_dtype, D,
                J->k_scale ? (double)J->k_scale[h] : 1.0,
                J->v_scale ? (double)J->v_scale[h] : 1.0};
  if (J->app_qo_indptr) {
    /* append: query token i of the request at position L - n + i */
    const int64_t q0 = J->app_qo_indptr[r], n = J->app_qo_indptr[r + 1] - q0;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t pos = L - n + i;
      const int64_t keys = J->causal ? pos + 1 : L;
      for (int j = h * G; j < (h + 1) * G; ++j) {
        int64_t qo = ((q0 + i) * J->Hq + j) * D;
        for (int d = 0; d < D; ++d) qv[d] = load_elem(J->q, J->q_dtype, qo + d);
        attend_row(qv, rows, keys, &src, J->sm_scale, &J->rope, (double)pos, x,
                   J->o + qo, J->lse + (q0 + i) * J->Hq + j);
      }
    }
    return;
  }
  for (int j = h * G; j < (h + 1) * G; ++j) {
    int64_t qo = ((int64_t)r * J->Hq + j) * D;
    for (int d = 0; d < D; ++d) qv[d] = load_elem(J->q, J->q_dtype, qo + d);
    attend_row(qv, rows, L, &src, J->sm_scale, &J->rope, (double)(L - 1), x, J->o + qo,
               J->lse + (int64_t)r * J->Hq + j);
  }
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (J->max_len + 1));
  double* x = (double*)malloc(sizeof(double) * (J->max_len + 1));
  double* qv = (double*)malloc(sizeof(double) * J->D);
  const int64_t n_items = (int64_t)J->batch * J->Hkv;
  for (;;) {
    int64_t it = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
    if (it >= n_items) break;
    if (J->unit_mask && !J->unit_mask[it]) continue;
    run_item(J, (int)(it / J->Hkv), (int)(it % J->Hkv), rows, x, qv);
  }
  free(rows);
  free(x);
  free(qv);
  return NULL;
}

static int run_job(job_t* J, int num_threads) {
  if (J->Hkv <= 0 || J->Hq % J->Hkv != 0 || J->ps <= 0 || J->D <= 0 || J->D > 512 ||
      (J->D & 1))
    return -1;
  if (J->rope.on && !(J->rope.theta > 0.0 && J->rope.scale > 0.0)) return -1;
  /* a level is either paged (indices and last) or ragged (neither) */
  if ((J->indices == NULL) != (J->last == NULL)) return -1;
  if (J->n_levels < 0 || J->n_levels > ORACLE_MAX_LEVELS) return -1;
  for (int l = 0; l < J->n_levels; ++l)
    if ((J->lv[l].p_indices == NULL) != (J->lv[l].p_last == NULL)) return -1;
  J->max_len = 0;
  for (int r = 0; r < J->batch; ++r) {
    int64_t L = request_len(J->indptr, J->last, r, J->ps);
    if (J->app_qo_indptr) {
      const int64_t n = (int64_t)J->app_qo_indptr[r + 1] - J->app_qo_indptr[r];
      if (n < 0 || n > L) return -1;
    }
    for (int l = 0; l < J->n_levels; ++l) {
      const int g = group_of(J, l, r);
      if (g >= 0) L += request_len(J->lv[l].p_indptr, J->lv[l].p_last, g, J->ps);
    }
    if (L > J->max_len) J->max_len = L;
  }
  J->next = 0;
  if (num_threads < 1) num_threads = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * num_threads);
  int started = 0;
  for (int i = 0; i < num_threads; ++i)
    if (pthread_create(&th[i], NULL, worker, J) == 0) ++started;
  if (started == 0) worker(J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  return 0;
}

/* Paged decode: o[b][j][:], lse[b][j] for every request b and q head j (or
 * only for the (b, kv head) items unit_mask selects).  Returns 0 on success. */
int oracle_decode(int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                  int page_size, int q_dtype, int kv_dtype, const void* q,
                  const void* k_pages, const void* v_pages,
                  const int32_t* kv_indptr, const int32_t* kv_indices,
                  const int32_t* last_page_len, const float* k_scale,
                  const float* v_scale, double sm_scale,
                  const uint8_t* unit_mask, double* o, double* lse,
                  int num_threads, int rope, double rope_theta, double rope_scale,
                  int hnd) {
  job_t J;
  memset(&J, 0, sizeof(J));
  J.hnd = hnd;
  J.rope.on = rope; J.rope.theta = rope_theta; J.rope.scale = rope_scale;
  J.batch = batch; J.Hq = num_qo_heads; J.Hkv = num_kv_heads; J.D = head_dim;
  J.ps = page_size; J.q_dtype = q_dtype; J.kv_dtype = kv_dtype;
  J.q = q; J.k_pages = k_pages; J.v_pages = v_pages;
  J.indptr = kv_indptr; J.indices = kv_indices; J.last = last_page_len;
  J.k_scale = k_scale; J.v_scale = v_scale; J.sm_scale = sm_scale;
  J.unit_mask = unit_mask; J.o = o; J.lse = lse;
  return run_job(&J, num_threads);
}

/* Cascade decode: request r of group g (qo_indptr[g] <= r < qo_indptr[g+1])
 * attends over the group's shared prefix pages followed by its own pages,
 * i.e. exactly the flat decode over the concatenated key list. */
int oracle_cascade(int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                   int page_size, int q_dtype, int kv_dtype, const void* q,
                   const void* k_pages, const void* v_pages, int n_groups,
                   const int32_t* prefix_qo_indptr,
                   const int32_t* prefix_kv_indptr,
                   const int32_t* prefix_kv_indices,
                   const int32_t* prefix_last_page_len,
                   const int32_t* kv_indptr, const int32_t* kv_indices,
                   const int32_t* last_page_len, const float* k_scale,
                   const float* v_scale, double sm_scale,
                   const uint8_t* unit_mask, double* o, double* lse,
                   int num_threads, int rope, double rope_theta, double rope_scale,
                  int hnd) {
  job_t J;
  memset(&J, 0, sizeof(J));
  J.hnd = hnd;
  J.rope.on = rope; J.rope.theta = rope_theta; J.rope.scale = rope_scale;
  J.batch = batch; J.Hq = num_qo_heads; J.Hkv = num_kv_heads; J.D = head_dim;
  J.ps = page_size; J.q_dtype = q_dtype; J.kv_dtype = kv_dtype;
  J.q = q; J.k_pages = k_pages; J.v_pages = v_pages;
  J.indptr = kv_indptr; J.indices = kv_indices; J.last = last_page_len;
  J.n_levels = n_groups > 0 ? 1 : 0;
  J.lv[0].n_groups = n_groups; J.lv[0].qo_indptr = prefix_qo_indptr;
  J.lv[0].p_indptr = prefix_kv_indptr; J.lv[0].p_indices = prefix_kv_indices;
  J.lv[0].p_last = prefix_last_page_len;
  J.k_scale = k_scale; J.v_scale = v_scale; J.sm_scale = sm_scale;
  J.unit_mask = unit_mask; J.o = o; J.lse = lse;
  return run_job(&J, num_threads);
}

/* Multi-level cascade: n_levels shared levels, outermost first; level l has
 * n_groups[l] groups of contiguous requests (qo_indptr[l]) with prefix
 * tables indptr[l] / indices[l] / last[l]; request r attends over the
 * prefix of its group at every level, in level order, then its own pages --
 * the flat decode over the concatenated key list. */
int oracle_cascade_levels(int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                          int page_size, int q_dtype, int kv_dtype, const void* q,
                          const void* k_pages, const void* v_pages, int n_levels,
                          const int32_t* n_groups, const int32_t* const* qo_indptr,
                          const int32_t* const* p_indptr, const int32_t* const* p_indices,
                          const int32_t* const* p_last, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* last_page_len,
                          const float* k_scale, const float* v_scale, double sm_scale,
                          const uint8_t* unit_mask, double* o, double* lse,
                          int num_threads, int rope, double rope_theta, double rope_scale,
                          int hnd) {
  if (n_levels < 0 || n_levels > ORACLE_MAX_LEVELS) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.hnd = hnd;
  J.rope.on = rope; J.rope.theta = rope_theta; J.rope.scale = rope_scale;
  J.batch = batch; J.Hq = num_qo_heads; J.Hkv = num_kv_heads; J.D = head_dim;
  J.ps = page_size; J.q_dtype = q_dtype; J.kv_dtype = kv_dtype;
  J.q = q; J.k_pages = k_pages; J.v_pages = v_pages;
  J.indptr = kv_indptr; J.indices = kv_indices; J.last = last_page_len;
  J.n_levels = n_levels;
  for (int l = 0; l < n_levels; ++l) {
    J.lv[l].n_groups = n_groups[l]; J.lv[l].qo_indptr = qo_indptr[l];
    J.lv[l].p_indptr = p_indptr[l]; J.lv[l].p_indices = p_indices[l];
    J.lv[l].p_last = p_last[l];
  }
  J.k_scale = k_scale; J.v_scale = v_scale; J.sm_scale = sm_scale;
  J.unit_mask = unit_mask; J.o = o; J.lse = lse;
  return run_job(&J, num_threads);
}

/* Append attention: request r's qo_indptr[r+1] - qo_indptr[r] query tokens
 * are the last ones of its key list (see the readings at the top); o and lse
 * are [total_q][Hq][D] and [total_q][Hq], rows in query-token order. */
int oracle_append(int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                  int page_size, int q_dtype, int kv_dtype, const void* q,
                  const void* k_pages, const void* v_pages, const int32_t* qo_indptr,
                  const int32_t* kv_indptr, const int32_t* kv_indices,
                  const int32_t* last_page_len, const float* k_scale,
                  const float* v_scale, double sm_scale, int causal,
                  const uint8_t* unit_mask, double* o, double* lse,
                  int num_threads, int rope, double rope_theta, double rope_scale,
                  int hnd) {
  if (!qo_indptr) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.hnd = hnd;
  J.rope.on = rope; J.rope.theta = rope_theta; J.rope.scale = rope_scale;
  J.batch = batch; J.Hq = num_qo_heads; J.Hkv = num_kv_heads; J.D = head_dim;
  J.ps = page_size; J.q_dtype = q_dtype; J.kv_dtype = kv_dtype;
  J.q = q; J.k_pages = k_pages; J.v_pages = v_pages;
  J.indptr = kv_indptr; J.indices = kv_indices; J.last = last_page_len;
  J.k_scale = k_scale; J.v_scale = v_scale; J.sm_scale = sm_scale;
  J.app_qo_indptr = qo_indptr; J.causal = causal != 0;
  J.unit_mask = unit_mask; J.o = o; J.lse = lse;
  return run_job(&J, num_threads);
}

/* Merge of attention states over disjoint key sets.  Since
 * exp(lse) = sum of exp(score) over the keys, the union of sets i has
 * lse = M + ln sum_i exp(lse_i - M) with M = max_i lse_i, and
 * o = sum_i exp(lse_i - lse) * o_i.  If every lse_i is -inf the union is
 * empty: o = 0, lse = -inf.
 * states: o_in [n_states][n_rows][D] (dtype v_dtype), lse_in [n_states][n_rows]
 * (fp32 or fp64 per s_dtype); outputs fp64. */
int oracle_merge(int n_states, int64_t n_rows, int D, int v_dtype,
                 const void* o_in, int s_dtype, const void* lse_in,
                 double* o_out, double* lse_out) {
  for (int64_t row = 0; row < n_rows; ++row) {
    double M = -INFINITY;
    for (int i = 0; i < n_states; ++i) {
      double s = load_elem(lse_in, s_dtype, (int64_t)i * n_rows + row);
      if (s > M) M = s;
    }
    double* o = o_out + row * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
      lse_out[row] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int i = 0; i < n_states; ++i)
      sum += exp(load_elem(lse_in, s_dtype, (int64_t)i * n_rows + row) - M);
    double lse = M + log(sum);
    for (int i = 0; i < n_states; ++i) {
      double w = exp(load_elem(lse_in, s_dtype, (int64_t)i * n_rows + row) - lse);
      for (int d = 0; d < D; ++d)
        o[d] += w * load_elem(o_in, v_dtype,
                              ((int64_t)i * n_rows + row) * D + d);
    }
    lse_out[row] = lse;
  }
  return 0;
}
