// fi_prefix.h -- the multi-row attention kernel (cascade prefix tiles and
// batch-append tiles) for gfx950.  Included by prefix.hip (instances
// without RoPE) and prefix_rope.hip (RoPE instances), which compile in
// parallel.
//
// Many query rows against one chunk of one key list, K/V staged in LDS and
// shared by every wave of the workgroup: the G heads of every request of a
// cascade group against the group's shared prefix (FlashInfer README "core
// features" item 3, cascade attention), or the query tokens of an append
// request against its own keys (README append example, causal mask).
#pragma once

#include <type_traits>

#include "fi_device.h"

namespace fi {

// ============================================================================
// cascade prefix tiles: many query rows x one prefix chunk of one kv head.
// ============================================================================
// Workgroup = WAVES waves; wave w owns query rows row0 + 16 RT w + 16 rt + n
// (rt < RT: 2 row tiles, 1 at head_dim 256 or with RoPE) as the N columns of
// its MFMAs, so each K/V element staged in LDS serves 16 RT WAVES rows.  The
// tile's slice of the page table is copied to LDS once.  Per 32-token step
// the workgroup loads the step's K and V rows of the tile's kv head two steps
// ahead into registers, stores them to one of two LDS buffers after
// computing from the other, one barrier per step.  Scores: MFMA 16x16x32
// with every K operand of the step read from LDS up front; the V^T operands
// (transpose reads) are issued before the softmax so their latency hides
// under it.  Softmax: the probabilities are formed against the running max
// m; only when a lane's sum of them exceeds kPrefixLazySum (or is not
// finite: the first step, where m = -inf) does the wave take the exact row
// max, rescale and recompute, so the common step carries no max reduction.
// P.V: MFMA 16x16x32.  The prefix is reused across row tiles, so its loads
// use the default (cached) policy, and the block -> tile map puts all row
// tiles of one (head, chunk) on the same XCD (workgroups are dispatched to
// the 8 XCDs round-robin) so they share that XCD's L2.
//
// The same kernel runs append tiles (APPEND): the rows are the query tokens
// of one request (token-major, G heads each) over that request's own pages;
// row i may attend keys below its limit (ReqInfo.kv_len of its token: its
// causal limit, or all keys without the mask), so a step that reaches past
// the smallest limit of the wave's rows masks per row, and a wave skips
// steps past the largest limit of its rows.
//
// RoPE (ROPE instances): rows of one tile sit at different positions, so the
// decode kernel's relative form (turning each key by its distance from the
// one query) does not apply; the rotation is taken in its absolute form
// instead.  Each query row is turned by its position relative to the start
// of the tile's key list (p.rope_qpos of its request or query token) and
// each key by its index in that list -- the dot product depends only on the
// difference.  Both are turned in fp32 from the plan's fp32 (cos, sin) table
// and kept as a 16-bit high part plus a 16-bit residual, and each score is
// the sum of three MFMAs (high.high, high.residual, residual.high), so the
// turned operands enter the scores at about fp32 accuracy.  The keys are
// turned once per workgroup while they are staged: a K unit is dims 4j..4j+3
// and their rotate-half partners D/2 + 4j.. of one token, loaded together
// with the table's (cos, sin) of those four frequencies at the token's
// index, and written to LDS as a high row and a residual row.
constexpr int kPStep = 32;
constexpr float kPrefixLazySum = 256.f;

template <int KV, int D, bool ROPE = false>
struct PStage {
  // K row bytes kept in LDS: as stored (e4m3 stays 8-bit), or, with RoPE,
  // the turned key as 16-bit values (two rows: high part and residual)
  static constexpr int ROWB = (KV == kKvE4M3 && !ROPE) ? D : 2 * D;
  static constexpr int KPARTS = ROPE ? 2 : 1;
  // K LDS row stride: 16-bit rows padded by 32 bytes (the score operand
  // reads then show no bank conflict; at 16 bytes they took 28 % of the
  // LDS-active cycles), e4m3 rows by 16
  static constexpr int KS = ROWB + ((KV == kKvE4M3 && !ROPE) ? 16 : 32);
  static constexpr int VS = 2 * D + 32;                     // V LDS row stride (16-bit values)
  static constexpr int VOFF = KPARTS * kPStep * KS;         // V rows after the K rows
  static constexpr int BUF = VOFF + kPStep * VS;
  static constexpr int PTAB = kPrefixMaxChunk + 2;          // page-table slots (page_size 1)
  static constexpr int LDS = 2 * BUF + 4 * PTAB;
};

// XCD-aware map: block b runs on XCD b % 8; give each XCD a contiguous range
// of the (chunk, head, row tile)-ordered tile list.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int x = b & 7, k = b >> 3, per = n >> 3, rem = n & 7;
  return x * per + min(x, rem) + k;
}

// MODE: kPrefixPlain / kPrefixSplitP (cascade prefix tiles) or kPrefixAppend.
enum { kPrefixPlain = 0, kPrefixSplitP = 1, kPrefixAppend = 2 };

// Turns the 16-bit pairs (x_e, y_e) = (element e of xa, element e of ya),
// e < 4, forward by the angles whose (cos, sin) are cs[e]: x' = x c - y s,
// y' = y c + x s, in fp32; writes each result as a 16-bit high part and a
// 16-bit residual.
template <bool BF16>
__device__ __forceinline__ void rope_turn4(u32x2 xa, u32x2 ya, const float2 (&cs)[4],
                                           u32x2& xh, u32x2& xl, u32x2& yh, u32x2& yl) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float rx[2], ry[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float c = cs[2 * k + e].x, sn = cs[2 * k + e].y;
      const float x = e ? hi16<BF16>(xa[k]) : lo16<BF16>(xa[k]);
      const float y = e ? hi16<BF16>(ya[k]) : lo16<BF16>(ya[k]);
      rx[e] = __builtin_fmaf(x, c, -(y * sn));
      ry[e] = __builtin_fmaf(y, c, x * sn);
    }
    xh[k] = pack2<BF16>(rx[0], rx[1]);
    yh[k] = pack2<BF16>(ry[0], ry[1]);
    xl[k] = residual2<BF16>(xh[k], rx[0], rx[1]);
    yl[k] = residual2<BF16>(yh[k], ry[0], ry[1]);
  }
}

// REC: as decode_kernel's (the token base is that of the tile's group, or of
// its request for append tiles).
template <int KV, bool QBF16, int WAVES, bool PS_POW2, int MODE, int D, bool ROPE = false,
          bool REC = false>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 && D != 256 ? 2 : 1) void prefix_kernel(
    DecodeParams p) {
  static_assert(!(ROPE && REC), "the record instances have no RoPE");
  constexpr bool APPEND = MODE == kPrefixAppend;
  // row tiles (16 query rows each) per wave: two, one at D = 256 or with
  // RoPE (registers: the turned q and K operands are twice as wide)
  constexpr int RT = prefix_rows_per_wave(D, ROPE) / 16;
  using S = PStage<KV, D, ROPE>;
  // bf16 K/V: P.V takes p as a bf16 high part plus a bf16 residual in append
  // tiles and in the split-p cascade instance -- bf16 keeps 8 bits of p, and
  // when a few keys carry comparable weight (the first rows of a prefill, a
  // short shared prefix) that rounding alone moves o past the accuracy bar.
  // The plan picks the split instance for a cascade level whose shortest
  // prefix is under kSplitPKeys keys; long prefixes keep one bf16 p (the
  // residual products cost the MFMA-bound kernel more than a tenth, and over
  // that many keys the rounding averages out).
  constexpr bool SPLITP = MODE != kPrefixPlain && KV == kKvBF16;
  // RoPE at D = 256 (registers): K operands read per k slice, and one set of
  // loads in flight (issued at the start of the step before the one it feeds)
  constexpr bool KUP = !(ROPE && D == 256);
  constexpr bool ONE_SET = ROPE && D == 256;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS];
  int* ptab = reinterpret_cast<int*>(lds + 2 * S::BUF);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  // cascade: contiguous tile ranges per XCD; append: the plan interleaves
  // its list so that block b and b + 8 (same XCD) share a key chunk
  const Tile tile =
      p.tiles[p.num_tiles + (APPEND ? (int)blockIdx.x : xcd_tile(blockIdx.x, gridDim.x))];
  const int grp = tile.req, h = tile.kv_head0, t0 = tile.t0, t1 = tile.t1;
  const int G = p.G;
  const int qo0 = p.qo_indptr[grp];
  const int page_base = p.kv_indptr[grp];
  const int ps = p.page_size, ps_shift = p.ps_shift;
  auto page_idx = [&](int t) { return PS_POW2 ? (t >> ps_shift) : (t / ps); };
  const int nsteps = (t1 - t0 + kPStep - 1) / kPStep;
  if (nsteps <= 0) return;   // the plan emits no empty prefix tiles
  const int pfirst = page_idx(t0);
  {
    const int np = page_idx(t1 - 1) - pfirst + 1;   // <= chunk / page_size + 1 < PTAB
    for (int i = tid; i < np; i += 64 * WAVES)
      ptab[i] = p.ragged ? page_base + pfirst + i : p.kv_indices[page_base + pfirst + i];
  }
  const float2* rtab = reinterpret_cast<const float2*>(p.rope_table);

  // query rows of this lane's column tiles (B operands of the scores); with
  // RoPE the turned row as a high part (qop) and a residual (qlo)
  u32x4 qop[RT][D / 32];
  u32x4 qlo[ROPE ? RT : 1][D / 32];
  bool rok[RT];
  int rreq[RT], rj[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = tile.row0 + 16 * RT * wave + 16 * rt + n;   // < row0 + 16 RT WAVES
    rok[rt] = row < tile.row1;
    const int rr = rok[rt] ? row : tile.row0;
    rreq[rt] = qo0 + rr / G;
    rj[rt] = h * G + rr % G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)rreq[rt] * p.Hq + rj[rt]) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
      qop[rt][s] = rok[rt] ? v : u32x4{0, 0, 0, 0};
    }
    if constexpr (ROPE) {
      // operand s holds dims 32 s + 8 g .. +7; s + D / 64 their partners
      const int64_t qd = rok[rt] ? p.rope_qpos[rreq[rt]] : 0;   // < rope_rows
#pragma unroll
      for (int s = 0; s < D / 64; ++s) {
        const float2* cs = rtab + qd * (D / 2) + 32 * s + 8 * g;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float2 c4[4] = {cs[4 * hh], cs[4 * hh + 1], cs[4 * hh + 2], cs[4 * hh + 3]};
          const u32x2 xa = {qop[rt][s][2 * hh], qop[rt][s][2 * hh + 1]};
          const u32x2 ya = {qop[rt][s + D / 64][2 * hh], qop[rt][s + D / 64][2 * hh + 1]};
          u32x2 xh, xl, yh, yl;
          rope_turn4<QBF16>(xa, ya, c4, xh, xl, yh, yl);
          qop[rt][s][2 * hh] = xh.x;
          qop[rt][s][2 * hh + 1] = xh.y;
          qlo[rt][s][2 * hh] = xl.x;
          qlo[rt][s][2 * hh + 1] = xl.y;
          qop[rt][s + D / 64][2 * hh] = yh.x;
          qop[rt][s + D / 64][2 * hh + 1] = yh.y;
          qlo[rt][s + D / 64][2 * hh] = yl.x;
          qlo[rt][s + D / 64][2 * hh + 1] = yl.y;
        }
      }
    }
  }
  // key limit of each of this lane's rows within the tile (t1, or the
  // row's causal limit), and over the wave's valid rows the smallest (steps
  // reaching past it mask per row) and the largest (steps from there on
  // have no key for any row: skipped)
  int lim[RT], lo = 0x7fffffff, hi = -0x7fffffff - 1;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lim[rt] = APPEND ? min(p.req_info[rreq[rt]].kv_len, t1) : t1;
    if (rok[rt]) {
      lo = min(lo, lim[rt]);
      hi = max(hi, lim[rt]);
    }
  }
#pragma unroll
  for (int k = 1; k < 16; k <<= 1) {
    lo = min(lo, __shfl_xor(lo, k));
    hi = max(hi, __shfl_xor(hi, k));
  }
  const int wave_lo = __builtin_amdgcn_readfirstlane(lo);
  const int wave_hi = __builtin_amdgcn_readfirstlane(hi);
  float c = p.sm_scale_log2;
  if (KV == kKvE4M3 && p.k_scale) c *= p.k_scale[h];

  // cooperative loader: a step is 32 rows of K and 32 rows of V, i.e.
  // 2 x 32 x VR 16-byte vectors (VR per row).  Thread tid loads vectors
  // idx = tid + u T (T threads, u < NL): pool idx / (32 VR) (0 = K, 1 = V),
  // token (idx % (32 VR)) / VR, chunk idx % VR.  RoPE instances load K as
  // KU units (above) of 2 x 4 elements plus 4 table pairs, NLK per thread,
  // and V as NLV 16-byte vectors per thread.
  constexpr bool F8 = KV == kKvE4M3;
  constexpr int HROW = F8 ? D : 2 * D;              // K / V row bytes in memory
  constexpr int VR = HROW / 16;
  constexpr int T = 64 * WAVES;
  constexpr int PV = 32 * VR;                       // vectors per pool per step
  constexpr int NL = ROPE ? 1 : (2 * PV + T - 1) / T;
  constexpr int KU = kPStep * D / 8;                // RoPE: K units per step
  constexpr int NLK = ROPE ? (KU + T - 1) / T : 1;
  constexpr int NLV = ROPE ? (PV + T - 1) / T : 1;
  using KPart = typename std::conditional<F8, uint32_t, u32x2>::type;   // 4 elements
  struct RopeSet {
    KPart a[NLK], b[NLK];   // dims 4 j .. +3 and their partners D/2 + 4 j ..
    float2 cs[NLK][4];      // (cos, sin) of frequencies 4 j .. +3 at the key's index
    u32x4 v[NLV];
  };
  const char* kbase = reinterpret_cast<const char*>(p.k_pages) + (int64_t)h * p.head_stride;
  const char* vbase = reinterpret_cast<const char*>(p.v_pages) + (int64_t)h * p.head_stride;
  const int last = t1 - 1;
  auto row_off = [&](int t) {   // byte offset of token t's row of this kv head
    const int pi = page_idx(t);
    const uint32_t sl = PS_POW2 ? (uint32_t)(t & (ps - 1)) : (uint32_t)(t - pi * ps);
    const uint32_t page = (uint32_t)ptab[pi - pfirst];
    return (uint64_t)page * p.page_bytes + sl * p.slot_stride;
  };
  // byte offsets of this thread's NL vectors of the step at tb: the page
  // lookup (an LDS read of the tile's page table) is taken a step before
  // the loads that use it, so no step starts waiting on it
  auto offs = [&](int tb, uint64_t (&o)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + u * T;
      if (2 * PV % T != 0 && idx >= 2 * PV) continue;
      const int q = idx % PV;
      o[u] = row_off(min(tb + q / VR, last)) + 16 * (q % VR);
    }
  };
  auto load_at = [&](int tb, const uint64_t (&o)[NL], u32x4 (&vec)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + u * T;
      if (2 * PV % T != 0 && idx >= 2 * PV) continue;
      vec[u] = ld_global<u32x4>(idx < PV ? kbase : vbase, o[u]);
      if constexpr (REC) {
        const int q = idx % PV;
        if (idx < PV)
          p.rec[((p.rec_base[grp] + min(tb + q / VR, last)) * p.Hkv + h) * VR + q % VR] =
              (int64_t)(o[u] + (uint64_t)h * p.head_stride);
      }
    }
    (void)tb;
  };
  auto load = [&](int tb, u32x4 (&vec)[NL]) {
    uint64_t o[NL];
    offs(tb, o);
    load_at(tb, o, vec);
  };
  auto load_rope = [&](int tb, RopeSet& st) {
#pragma unroll
    for (int u = 0; u < NLK; ++u) {
      const int idx = tid + u * T;
      if (KU % T != 0 && idx >= KU) continue;
      const int j = idx % (D / 8), t = min(tb + idx / (D / 8), last);
      const uint64_t off = row_off(t) + (F8 ? 4 : 8) * j;
      st.a[u] = ld_global<KPart>(kbase, off);
      st.b[u] = ld_global<KPart>(kbase, off + (F8 ? 1 : 2) * (D / 2));
      const float2* cs = rtab + (int64_t)t * (D / 2) + 4 * j;   // t < rope_rows
#pragma unroll
      for (int e = 0; e < 4; ++e) st.cs[u][e] = cs[e];
    }
#pragma unroll
    for (int u = 0; u < NLV; ++u) {
      const int idx = tid + u * T;
      if (PV % T != 0 && idx >= PV) continue;
      const int t = min(tb + idx / VR, last);
      st.v[u] = ld_global<u32x4>(vbase, row_off(t) + 16 * (idx % VR));
    }
  };
  // one 16-byte V vector (token tok, chunk chk) to LDS (e4m3: as 16-bit)
  auto store_v = [&](uint8_t* vt, int tok, int chk, const u32x4& w) {
    if constexpr (F8) {
      const u32x2 a = e4m3x4_to_16<QBF16>(w.x), b = e4m3x4_to_16<QBF16>(w.y);
      const u32x2 c2 = e4m3x4_to_16<QBF16>(w.z), d = e4m3x4_to_16<QBF16>(w.w);
      uint8_t* dv = vt + tok * S::VS + 32 * chk;
      *reinterpret_cast<u32x4*>(dv) = u32x4{a.x, a.y, b.x, b.y};
      *reinterpret_cast<u32x4*>(dv + 16) = u32x4{c2.x, c2.y, d.x, d.y};
    } else {
      *reinterpret_cast<u32x4*>(vt + tok * S::VS + 16 * chk) = w;
    }
  };
  auto store = [&](int buf, const u32x4 (&vec)[NL]) {
    uint8_t* kt = lds + buf * S::BUF;
    uint8_t* vt = kt + S::VOFF;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + u * T;
      if (2 * PV % T != 0 && idx >= 2 * PV) continue;
      const int q = idx % PV;
      const int tok = q / VR, chk = q % VR;
      if (idx < PV)
        *reinterpret_cast<u32x4*>(kt + tok * S::KS + 16 * chk) = vec[u];
      else
        store_v(vt, tok, chk, vec[u]);
    }
  };
  auto store_rope = [&](int buf, const RopeSet& st) {
    uint8_t* kh = lds + buf * S::BUF;
    uint8_t* kl = kh + kPStep * S::KS;
    uint8_t* vt = kh + S::VOFF;
#pragma unroll
    for (int u = 0; u < NLK; ++u) {
      const int idx = tid + u * T;
      if (KU % T != 0 && idx >= KU) continue;
      const int tok = idx / (D / 8), j = idx % (D / 8);
      u32x2 xa, ya;
      if constexpr (F8) {
        xa = e4m3x4_to_16<QBF16>(st.a[u]);
        ya = e4m3x4_to_16<QBF16>(st.b[u]);
      } else {
        xa = st.a[u];
        ya = st.b[u];
      }
      u32x2 xh, xl, yh, yl;
      rope_turn4<QBF16>(xa, ya, st.cs[u], xh, xl, yh, yl);
      const int o0 = tok * S::KS + 8 * j, o1 = o0 + D;   // dims 4 j and D/2 + 4 j
      *reinterpret_cast<u32x2*>(kh + o0) = xh;
      *reinterpret_cast<u32x2*>(kh + o1) = yh;
      *reinterpret_cast<u32x2*>(kl + o0) = xl;
      *reinterpret_cast<u32x2*>(kl + o1) = yl;
    }
#pragma unroll
    for (int u = 0; u < NLV; ++u) {
      const int idx = tid + u * T;
      if (PV % T != 0 && idx >= PV) continue;
      store_v(vt, idx / VR, idx % VR, st.v[u]);
    }
  };

  float m[RT], l[RT];
  f32x4 oacc[RT][D / 16];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int b = 0; b < D / 16; ++b) oacc[rt][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 32-token step from LDS buffer buf; a step reaching past the
  // smallest row limit masks tokens at or past each row's limit (a uniform
  // branch around the masking only: one copy of the step body keeps the
  // accumulators in place across iterations)
  auto compute = [&](int tb, int buf, bool tail) {
    const uint8_t* kt = lds + buf * S::BUF;
    const uint8_t* vt = kt + S::VOFF;
    // ---- K operands of both token tiles (tokens 16 tt + n), all k slices
    // (RoPE: the high part; its residual rows follow the high rows), read
    // up front -- or, RoPE at D = 256 (registers), one k slice at a time
    // inside the score loop
    u32x4 kop[2][KUP ? D / 32 : 1];
    u32x4 kol[ROPE ? 2 : 1][KUP ? D / 32 : 1];
    auto read_k = [&](int tt, int s, u32x4& hi_part, u32x4& lo_part) {
      const uint8_t* krow = kt + (16 * tt + n) * S::KS;
      if constexpr (F8 && !ROPE) {
        const u32x2 w8 = *reinterpret_cast<const u32x2*>(krow + 32 * s + 8 * g);
        const u32x2 a = e4m3x4_to_16<QBF16>(w8.x), b = e4m3x4_to_16<QBF16>(w8.y);
        hi_part = u32x4{a.x, a.y, b.x, b.y};
      } else {
        hi_part = *reinterpret_cast<const u32x4*>(krow + 64 * s + 16 * g);
        if constexpr (ROPE)
          lo_part = *reinterpret_cast<const u32x4*>(krow + kPStep * S::KS + 64 * s + 16 * g);
      }
    };
    if constexpr (KUP) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < D / 32; ++s) read_k(tt, s, kop[tt][s], kol[ROPE ? tt : 0][s]);
    }
    // ---- V^T operands: contraction element kk of lane group g is token
    // 4 g + (kk & 3) + 16 (kk >> 2); two transpose reads per dim block b
    // (read up front, or -- RoPE at D = 256 -- right before their P.V)
    u32x4 vop[KUP ? D / 16 : 1];
    const uint8_t* vsrc = vt + (4 * g + (n >> 2)) * S::VS + 8 * (n & 3);
    auto read_v = [&](int b) {
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 32 * b));
      const s16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 16 * S::VS + 32 * b));
      const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      return u32x4{w0.x, w0.y, w1.x, w1.y};
    };
    if constexpr (KUP) {
#pragma unroll
      for (int b = 0; b < D / 16; ++b) vop[b] = read_v(b);
    }
    // ---- scores: S[tt][rt] = K(tokens 16 tt ..) . Q^T(rows of tile rt);
    // the accumulators are independent, so consecutive MFMAs never wait
    f32x4 sc[2][RT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if constexpr (!KUP)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) read_k(tt, s, kop[tt][0], kol[ROPE ? tt : 0][0]);
      const int ks = KUP ? s : 0;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          sc[tt][rt] = mma16x16x32<QBF16>(kop[tt][ks], qop[rt][s], sc[tt][rt]);
          if constexpr (ROPE) {
            sc[tt][rt] = mma16x16x32<QBF16>(kop[tt][ks], qlo[rt][s], sc[tt][rt]);
            sc[tt][rt] = mma16x16x32<QBF16>(kol[tt][ks], qop[rt][s], sc[tt][rt]);
          }
        }
    }
    // ---- softmax per row tile: lane (g, n) holds tokens 4 g + i and
    // 16 + 4 g + i (i < 4) of row n
    u32x4 pop[RT], plo[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = sc[0][rt][i];
        x[4 + i] = sc[1][rt][i];
      }
      if (__builtin_expect(tail, 0)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (tb + 4 * g + i >= lim[rt]) x[i] = -INFINITY;
          if (tb + 16 + 4 * g + i >= lim[rt]) x[4 + i] = -INFINITY;
        }
      }
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(__builtin_fmaf(x[i], c, -m[rt]));
      float sum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      if (__builtin_expect(__any(!(sum <= kPrefixLazySum)), 0)) {
        // exact row max of this step, rescale, recompute (a row with no key
        // so far -- all masked -- keeps m = -inf and gets p = 0)
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, x[i] * c);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m[rt], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m[rt] - m_use);
        l[rt] *= alpha;
#pragma unroll
        for (int b = 0; b < D / 16; ++b) oacc[rt][b] *= alpha;
        m[rt] = m_new;
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(__builtin_fmaf(x[i], c, -m_use));
        sum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      }
      l[rt] += sum;
      pop[rt] = u32x4{pack2<QBF16>(pr[0], pr[1]), pack2<QBF16>(pr[2], pr[3]),
                      pack2<QBF16>(pr[4], pr[5]), pack2<QBF16>(pr[6], pr[7])};
      if constexpr (SPLITP) {
        // bf16 keeps 8 bits of p: the residual p - bf16(p) goes through a
        // second P.V product
#pragma unroll
        for (int k = 0; k < 4; ++k)
          plo[rt][k] = pack2<true>(pr[2 * k] - lo16<true>(pop[rt][k]),
                                   pr[2 * k + 1] - hi16<true>(pop[rt][k]));
      }
    }
    // ---- P.V on MFMA 16x16x32
#pragma unroll
    for (int b = 0; b < D / 16; ++b) {
      const u32x4 vb = KUP ? vop[KUP ? b : 0] : read_v(b);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        oacc[rt][b] = mma16x16x32<QBF16>(vb, pop[rt], oacc[rt][b]);
      if constexpr (SPLITP) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          oacc[rt][b] = mma16x16x32<QBF16>(vb, plo[rt], oacc[rt][b]);
      }
    }
  };

  // two register sets: the one for step s + 1 is in flight while step s is
  // computed, the one for step s + 2 is issued at the start of step s
  using Set = typename std::conditional<ROPE, RopeSet, u32x4[NL]>::type;
  Set va, vb;
  auto load_set = [&](int tb, Set& st) {
    if constexpr (ROPE) load_rope(tb, st);
    else load(tb, st);
  };
  auto store_set = [&](int buf, const Set& st) {
    if constexpr (ROPE) store_rope(buf, st);
    else store(buf, st);
  };
  // The loads and stores run unconditionally, past the last step too: the
  // loader clamps every token to the tile's last key (in bounds, already
  // cached), the store goes to the buffer the step does not read, and
  // steps past the tile compute nothing (tb >= wave_hi).  Conditional loads
  // would make the compiler's wait counts merge over the branch and wait
  // for every load in flight -- including the ones just issued for two
  // steps ahead -- before each LDS store.
  __syncthreads();   // page table
  load_set(t0, va);
  store_set(0, va);
  if constexpr (ONE_SET) {
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
      const int tb = t0 + kPStep * step;
      load_set(tb + kPStep, va);
      if (tb < wave_hi) compute(tb, step & 1, tb + kPStep > wave_lo);
      store_set((step + 1) & 1, va);
      __syncthreads();
    }
  } else {
    load_set(t0 + kPStep, vb);
    // (plain instances) offsets of the loads two steps ahead, looked up one
    // step before they are issued
    uint64_t on[NL];
    if constexpr (!ROPE) offs(t0 + 2 * kPStep, on);
    __syncthreads();
    auto step_body = [&](int step, Set& nxt, Set& aft) {
      const int tb = t0 + kPStep * step;
      if constexpr (ROPE) {
        load_set(tb + 2 * kPStep, aft);
      } else {
        load_at(tb + 2 * kPStep, on, aft);
        offs(tb + 3 * kPStep, on);
      }
      if (tb < wave_hi) compute(tb, step & 1, tb + kPStep > wave_lo);
      store_set((step + 1) & 1, nxt);
      __syncthreads();
    };
    // (an odd step count runs one empty step at the end)
    for (int step = 0; step < nsteps; step += 2) {
      step_body(step, vb, va);
      step_body(step + 1, va, vb);
    }
  }

  // ---- finalize each row tile
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float lt = l[rt] + __shfl_xor(l[rt], 16);
    lt += __shfl_xor(lt, 32);
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (KV == kKvE4M3 && p.v_scale) inv *= p.v_scale[h];
    const float lse2 = lt > 0.f ? m[rt] + fast_log2(lt) : -INFINITY;
    if (!rok[rt]) continue;
    const int r = rreq[rt], j = rj[rt];
    const ReqInfo ri = p.req_info[r];
    if (ri.n_states <= 1) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)r * p.Hq + j) * D;
#pragma unroll
      for (int b = 0; b < D / 16; ++b) {
        u32x2 w = {pack2<QBF16>(oacc[rt][b][0] * inv, oacc[rt][b][1] * inv),
                   pack2<QBF16>(oacc[rt][b][2] * inv, oacc[rt][b][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * b + 4 * g) = w;
      }
      if (g == 0 && p.lse) p.lse[(int64_t)r * p.Hq + j] = lse2 * kLn2;
    } else {
      // state index: this level's chunk after the request's earlier levels
      const int c = tile.slot + (p.state_off ? p.state_off[r] : 0);
      const int64_t slot = ri.slot_base + (int64_t)c * p.Hkv + h;
      float* po = p.partial_o + (slot * G + (j - h * G)) * D;
#pragma unroll
      for (int b = 0; b < D / 16; ++b)
        *reinterpret_cast<f32x4*>(po + 16 * b + 4 * g) = oacc[rt][b] * inv;
      if (g == 0) p.partial_lse[slot * G + (j - h * G)] = lse2;
    }
  }
}

// Launches the multi-row kernel (RoPE instances: prefix_rope.hip).
hipError_t launch_prefix_rope(const DecodeParams& p, int num_tiles, int waves, bool append,
                              bool split, bool q_bf16, int kv, int head_dim, hipStream_t s);

}  // namespace fi
