// decode.hip -- gfx950 paged decode attention and cascade prefix kernels.
//
// Computes, for one query token per head, exact attention over the keys a
// request reaches through its page table (FlashInfer README "core features"
// item 1: paged / vector-sparse KV; item 3: head-query fusion for GQA,
// low-precision KV, cascade attention; flash-attention summary "How it
// works": exact attention that streams K/V once).  Softmax is the online
// form: a running max m and sum l per query row, with the accumulator
// rescaled by exp2(m_old - m_new) whenever the max grows; exponentials are
// taken base 2 with log2(e) folded into the score scale.
//
// MI355X mapping (one wave = 64 lanes, lane = 16 g + n):
//  * A decode workgroup is 4 waves; wave w owns kv head kv_head0 + w of one
//    request over a token chunk, so the G query heads that share the kv head
//    read each K/V row once.
//  * Scores: per 32-token block, S^T[token][head] = K . Q^T on MFMA
//    16x16x32 -- K rows go straight from HBM into the A operand (lane n
//    loads token n, 16 contiguous bytes per lane, 64 contiguous bytes per row
//    per instruction), q sits in the B operand for the whole tile
//    (columns n >= G are zero).  The D layout leaves lane (g, n) with
//    tokens 4g..4g+3 (+16) of head n, so the row max needs only two
//    cross-lane exchanges and P^T is already in B-operand layout.
//  * P.V: O^T[d][head] += V^T[d][token] . P^T[token][head] on MFMA.  V rows
//    are loaded coalesced (4 rows x 256 B per instruction), written to a
//    per-wave LDS tile and read back transposed (8 u16 per operand) in the
//    token order the P operand uses; the LDS row stride of 288 B keeps the 4
//    lane groups on disjoint banks.
//  * E4M3 K/V are converted to the q dtype in registers (exact) with the
//    per-kv-head scales folded into the score scale and the output.
//  * A tile whose (request, kv head) is split over several chunks writes an
//    fp32 partial state (o, log2-domain lse) that merge.hip combines.
#include "fi_device.h"

namespace fi {

constexpr int kVStride = 288;                      // bytes per LDS V row
constexpr int kVTileBytes = kBlockTokens * kVStride;  // 9216 per wave
constexpr int kKStride = 272;                      // bytes per LDS K row (prefix)

// LDS slot of block-relative token t: the P.V contraction index of lane
// group g, element kk is token 4g + (kk & 3) + 16 (kk >> 2); its V row is
// stored at slot 4 kk + g.
__device__ __forceinline__ int v_slot(int t) {
  const int g = (t & 15) >> 2, i = t & 3, hh = t >> 4;
  return 4 * (i + 4 * hh) + g;
}

// Reads the transposed V operand for d-block b: lane (g, n) gets
// V[token(g, kk)][16 b + n] for kk = 0..7.
__device__ __forceinline__ u32x4 read_vt(const uint8_t* vt, int g, int n, int b) {
  const uint8_t* base = vt + g * kVStride + (16 * b + n) * 2;
  uint32_t e[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    e[kk] = *reinterpret_cast<const uint16_t*>(base + 4 * kk * kVStride);
  u32x4 r;
  r.x = e[0] | (e[1] << 16);
  r.y = e[2] | (e[3] << 16);
  r.z = e[4] | (e[5] << 16);
  r.w = e[6] | (e[7] << 16);
  return r;
}

// Loads the q row pieces of one lane as the B operand of the 4 score steps.
// Step s holds d = dmap(s, g) .. +7; zero for columns past the group.
template <int KV>
__device__ __forceinline__ int q_dim(int s, int g) {
  if constexpr (KV == kKvE4M3) return 64 * (s >> 1) + 16 * g + 8 * (s & 1);
  else return 32 * s + 8 * g;
}

// K operand for score step s from the raw 16-byte loads of one token row.
// f16/bf16: load s is step s.  e4m3: load j covers steps 2j (low 8 codes) and
// 2j+1 (high 8 codes).
template <int KV, bool QBF16>
__device__ __forceinline__ u32x4 k_operand(const u32x4* raw, int s) {
  if constexpr (KV == kKvE4M3) {
    const u32x4 w = raw[s >> 1];
    const uint32_t lo = (s & 1) ? w.z : w.x, hi = (s & 1) ? w.w : w.y;
    const u32x2 a = e4m3x4_to_16<QBF16>(lo), b = e4m3x4_to_16<QBF16>(hi);
    return u32x4{a.x, a.y, b.x, b.y};
  } else {
    return raw[s];
  }
}

// ============================================================================
// decode tiles
// ============================================================================
template <int KV, bool QBF16>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int ES = KV == kKvE4M3 ? 1 : 2;          // bytes per K/V element
  constexpr int ROWB = kHeadDim * ES;                // bytes per K/V row
  constexpr int KLOADS = KV == kKvE4M3 ? 2 : 4;      // 16-B K loads per token row
  constexpr int VLOADS = KV == kKvE4M3 ? 4 : 8;      // 16-B V loads per lane per block
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWavesPerTile * kVTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Tile tile = p.tiles[blockIdx.x];
  const int h = tile.kv_head0 + wave;
  if (h >= p.Hkv) return;
  const int g = lane >> 4, n = lane & 15;
  const int r = tile.req, t0 = tile.t0, t1 = tile.t1;
  const int G = p.G;
  const int page_base = p.kv_indptr[r];
  uint8_t* vt = lds + wave * kVTileBytes;

  // q as the B operand of the score MFMAs
  u32x4 qop[4];
  {
    const bool ok = n < G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)r * p.Hq + h * G + (ok ? n : 0)) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + q_dim<KV>(s, g));
      qop[s] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  float c = p.sm_scale_log2;
  if (KV == kKvE4M3 && p.k_scale) c *= p.k_scale[h];

  const char* kbase = reinterpret_cast<const char*>(p.k_pages);
  const char* vbase = reinterpret_cast<const char*>(p.v_pages);
  auto row_off = [&](int t) -> int64_t {
    const int64_t slot = page_slot(p.kv_indices, page_base, t, p.page_size, p.ps_shift);
    return (slot * p.Hkv + h) * (int64_t)ROWB;
  };

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int tb = t0; tb < t1; tb += kBlockTokens) {
    const int last = t1 - 1;
    // ---- issue K and V loads (tokens past t1 re-read the last valid token)
    u32x4 kA[KLOADS], kB[KLOADS];
    {
      const int64_t oA = row_off(min(tb + n, last)), oB = row_off(min(tb + 16 + n, last));
#pragma unroll
      for (int j = 0; j < KLOADS; ++j) {
        kA[j] = ld_global<u32x4>(kbase, oA + 64 * j + 16 * g);
        kB[j] = ld_global<u32x4>(kbase, oB + 64 * j + 16 * g);
      }
    }
    u32x4 vr[VLOADS];
    int vslot[VLOADS];
    int vcol;
    if constexpr (KV == kKvE4M3) {
      // lane (q8 = lane / 8, c8 = lane % 8): instruction u loads token 8u + q8
      const int q8 = lane >> 3;
      vcol = (lane & 7) * 32;  // 16 codes -> 32 bytes of 16-bit values
#pragma unroll
      for (int u = 0; u < VLOADS; ++u) {
        const int t = 8 * u + q8;
        vslot[u] = v_slot(t);
        vr[u] = ld_global<u32x4>(vbase, row_off(min(tb + t, last)) + 16 * (lane & 7));
      }
    } else {
      vcol = 16 * n;
#pragma unroll
      for (int kk = 0; kk < VLOADS; ++kk) {
        const int t = 4 * g + (kk & 3) + 16 * (kk >> 2);
        vslot[kk] = 4 * kk + g;
        vr[kk] = ld_global<u32x4>(vbase, row_off(min(tb + t, last)) + 16 * n);
      }
    }

    // ---- scores S^T[token][head]
    f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sA = mma16x16x32<QBF16>(k_operand<KV, QBF16>(kA, s), qop[s], sA);
      sB = mma16x16x32<QBF16>(k_operand<KV, QBF16>(kB, s), qop[s], sB);
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (tb + 4 * g + i < t1) ? sA[i] * c : -INFINITY;
      x[4 + i] = (tb + 16 + 4 * g + i < t1) ? sB[i] * c : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float pr[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = fast_exp2(x[i] - m_use);
      psum += pr[i];
    }
    l = l * alpha + psum;
    m = m_new;
#pragma unroll
    for (int b = 0; b < 8; ++b) oacc[b] *= alpha;
    const u32x4 pop = {pack2<QBF16>(pr[0], pr[1]), pack2<QBF16>(pr[2], pr[3]),
                       pack2<QBF16>(pr[4], pr[5]), pack2<QBF16>(pr[6], pr[7])};

    // ---- V rows -> LDS (as q-dtype values), then transposed operands
    if constexpr (KV == kKvE4M3) {
#pragma unroll
      for (int u = 0; u < VLOADS; ++u) {
        const u32x2 a = e4m3x4_to_16<QBF16>(vr[u].x), b2 = e4m3x4_to_16<QBF16>(vr[u].y);
        const u32x2 c2 = e4m3x4_to_16<QBF16>(vr[u].z), d2 = e4m3x4_to_16<QBF16>(vr[u].w);
        uint8_t* dst = vt + vslot[u] * kVStride + vcol;
        *reinterpret_cast<u32x4*>(dst) = u32x4{a.x, a.y, b2.x, b2.y};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{c2.x, c2.y, d2.x, d2.y};
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < VLOADS; ++kk)
        *reinterpret_cast<u32x4*>(vt + vslot[kk] * kVStride + vcol) = vr[kk];
    }
#pragma unroll
    for (int b = 0; b < 8; ++b)
      oacc[b] = mma16x16x32<QBF16>(read_vt(vt, g, n, b), pop, oacc[b]);
  }

  // ---- finalize
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (KV == kKvE4M3 && p.v_scale) inv *= p.v_scale[h];
  const float lse2 = lt > 0.f ? m + fast_log2(lt) : -INFINITY;
  if (n >= G) return;
  const int j = h * G + n;
  if (tile.slot < 0) {
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)r * p.Hq + j) * kHeadDim;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      u32x2 w = {pack2<QBF16>(oacc[b][0] * inv, oacc[b][1] * inv),
                 pack2<QBF16>(oacc[b][2] * inv, oacc[b][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * b + 4 * g) = w;
    }
    if (g == 0 && p.lse) p.lse[(int64_t)r * p.Hq + j] = lse2 * kLn2;
  } else {
    const int64_t slot = tile.slot + wave;
    float* po = p.partial_o + (slot * G + n) * kHeadDim;
#pragma unroll
    for (int b = 0; b < 8; ++b)
      *reinterpret_cast<f32x4*>(po + 16 * b + 4 * g) = oacc[b] * inv;
    if (g == 0) p.partial_lse[slot * G + n] = lse2;
  }
}

// ============================================================================
// cascade prefix tiles: many query rows x one prefix chunk of one kv head.
// The 4 waves share each 32-token K/V block through LDS; wave w owns query
// rows row0 + 32 w + 16 ct + n (ct = 0, 1) as the N columns of its MFMAs.
// ============================================================================
template <int KV, bool QBF16>
__global__ __launch_bounds__(256) void prefix_kernel(DecodeParams p) {
  constexpr int ES = KV == kKvE4M3 ? 1 : 2;
  constexpr int ROWB = kHeadDim * ES;
  constexpr int KT = kBlockTokens * kKStride;  // K tile bytes
  constexpr int VT = kVTileBytes;              // V tile bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const Tile tile = p.tiles[p.num_tiles + blockIdx.x];
  const int grp = tile.req, h = tile.kv_head0, t0 = tile.t0, t1 = tile.t1;
  const int G = p.G;
  const int qo0 = p.qo_indptr[grp];
  const int page_base = p.kv_indptr[grp];

  // query rows of this lane's two column tiles
  u32x4 qop[2][4];
  int rrow[2], rreq[2], rj[2];
  bool rok[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = tile.row0 + 32 * wave + 16 * ct + n;
    rok[ct] = row < tile.row1;
    rrow[ct] = row;
    rreq[ct] = qo0 + (rok[ct] ? row : tile.row0) / G;
    rj[ct] = h * G + (rok[ct] ? row : tile.row0) % G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)rreq[ct] * p.Hq + rj[ct]) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + q_dim<kKvF16>(s, g));
      qop[ct][s] = rok[ct] ? v : u32x4{0, 0, 0, 0};
    }
  }
  float c = p.sm_scale_log2;
  if (KV == kKvE4M3 && p.k_scale) c *= p.k_scale[h];

  const char* kbase = reinterpret_cast<const char*>(p.k_pages);
  const char* vbase = reinterpret_cast<const char*>(p.v_pages);
  // cooperative loader: thread -> (token tl = tid / 16 + 16 u, chunk cc = tid % 16)
  // f16/bf16: 16 chunks of 16 B per row; e4m3: 8 chunks of 16 B, threads with
  // cc >= 8 idle for V/K staging.
  const int cc = tid & 15;
  auto load_block = [&](int tb, u32x4* kr, u32x4* vr) {
    const int last = t1 - 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = min(tb + (tid >> 4) + 16 * u, last);
      const int64_t slot = page_slot(p.kv_indices, page_base, t, p.page_size, p.ps_shift);
      const int64_t off = (slot * p.Hkv + h) * (int64_t)ROWB;
      if (KV != kKvE4M3 || cc < 8) {
        kr[u] = ld_global<u32x4>(kbase, off + 16 * cc);
        vr[u] = ld_global<u32x4>(vbase, off + 16 * cc);
      }
    }
  };
  auto store_block = [&](int buf, const u32x4* kr, const u32x4* vr) {
    uint8_t* kt = lds + buf * (KT + VT);
    uint8_t* vtile = kt + KT;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = (tid >> 4) + 16 * u;
      if constexpr (KV == kKvE4M3) {
        if (cc < 8) {
          const u32x2 a = e4m3x4_to_16<QBF16>(kr[u].x), b = e4m3x4_to_16<QBF16>(kr[u].y);
          const u32x2 c2 = e4m3x4_to_16<QBF16>(kr[u].z), d = e4m3x4_to_16<QBF16>(kr[u].w);
          uint8_t* dk = kt + t * kKStride + 32 * cc;
          *reinterpret_cast<u32x4*>(dk) = u32x4{a.x, a.y, b.x, b.y};
          *reinterpret_cast<u32x4*>(dk + 16) = u32x4{c2.x, c2.y, d.x, d.y};
          const u32x2 va = e4m3x4_to_16<QBF16>(vr[u].x), vb = e4m3x4_to_16<QBF16>(vr[u].y);
          const u32x2 vc = e4m3x4_to_16<QBF16>(vr[u].z), vd = e4m3x4_to_16<QBF16>(vr[u].w);
          uint8_t* dv = vtile + v_slot(t) * kVStride + 32 * cc;
          *reinterpret_cast<u32x4*>(dv) = u32x4{va.x, va.y, vb.x, vb.y};
          *reinterpret_cast<u32x4*>(dv + 16) = u32x4{vc.x, vc.y, vd.x, vd.y};
        }
      } else {
        *reinterpret_cast<u32x4*>(kt + t * kKStride + 16 * cc) = kr[u];
        *reinterpret_cast<u32x4*>(vtile + v_slot(t) * kVStride + 16 * cc) = vr[u];
      }
    }
  };

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 oacc[2][8];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int b = 0; b < 8; ++b) oacc[ct][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kr[2], vr[2];
  if (t0 < t1) {
    load_block(t0, kr, vr);
    store_block(0, kr, vr);
  }
  __syncthreads();
  int buf = 0;
  for (int tb = t0; tb < t1; tb += kBlockTokens) {
    const bool more = tb + kBlockTokens < t1;
    if (more) load_block(tb + kBlockTokens, kr, vr);   // prefetch next block
    const uint8_t* kt = lds + buf * (KT + VT);
    const uint8_t* vtile = kt + KT;
    // K operands (shared by both column tiles); K stored in q dtype layout
    u32x4 kop[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kop[tt][s] = *reinterpret_cast<const u32x4*>(kt + (16 * tt + n) * kKStride +
                                                     (32 * s + 8 * g) * 2);
    u32x4 pop[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sA = mma16x16x32<QBF16>(kop[0][s], qop[ct][s], sA);
        sB = mma16x16x32<QBF16>(kop[1][s], qop[ct][s], sB);
      }
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (tb + 4 * g + i < t1) ? sA[i] * c : -INFINITY;
        x[4 + i] = (tb + 16 + 4 * g + i < t1) ? sB[i] * c : -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[ct], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m[ct] - m_use);
      float pr[8], psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = fast_exp2(x[i] - m_use);
        psum += pr[i];
      }
      l[ct] = l[ct] * alpha + psum;
      m[ct] = m_new;
#pragma unroll
      for (int b = 0; b < 8; ++b) oacc[ct][b] *= alpha;
      pop[ct] = u32x4{pack2<QBF16>(pr[0], pr[1]), pack2<QBF16>(pr[2], pr[3]),
                      pack2<QBF16>(pr[4], pr[5]), pack2<QBF16>(pr[6], pr[7])};
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const u32x4 vop = read_vt(vtile, g, n, b);
      oacc[0][b] = mma16x16x32<QBF16>(vop, pop[0], oacc[0][b]);
      oacc[1][b] = mma16x16x32<QBF16>(vop, pop[1], oacc[1][b]);
    }
    if (more) {
      __syncthreads();              // everyone is done reading buffer buf^1's old block
      store_block(buf ^ 1, kr, vr);
      __syncthreads();
      buf ^= 1;
    }
  }

  // ---- finalize each column tile
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float lt = l[ct] + __shfl_xor(l[ct], 16);
    lt += __shfl_xor(lt, 32);
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (KV == kKvE4M3 && p.v_scale) inv *= p.v_scale[h];
    const float lse2 = lt > 0.f ? m[ct] + fast_log2(lt) : -INFINITY;
    if (!rok[ct]) continue;
    const int r = rreq[ct], j = rj[ct];
    const ReqInfo ri = p.req_info[r];
    if (ri.n_states <= 1) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)r * p.Hq + j) * kHeadDim;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        u32x2 w = {pack2<QBF16>(oacc[ct][b][0] * inv, oacc[ct][b][1] * inv),
                   pack2<QBF16>(oacc[ct][b][2] * inv, oacc[ct][b][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * b + 4 * g) = w;
      }
      if (g == 0 && p.lse) p.lse[(int64_t)r * p.Hq + j] = lse2 * kLn2;
    } else {
      const int64_t slot = ri.slot_base + (int64_t)tile.slot * p.Hkv + h;
      float* po = p.partial_o + (slot * G + (j - h * G)) * kHeadDim;
#pragma unroll
      for (int b = 0; b < 8; ++b)
        *reinterpret_cast<f32x4*>(po + 16 * b + 4 * g) = oacc[ct][b] * inv;
      if (g == 0) p.partial_lse[slot * G + (j - h * G)] = lse2;
    }
  }
}

// ---- launchers ----------------------------------------------------------------
template <int KV, bool QBF16>
static hipError_t launch_decode_t(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<KV, QBF16>), dim3(num_tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int KV, bool QBF16>
static hipError_t launch_prefix_t(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefix_kernel<KV, QBF16>), dim3(num_tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

// q_bf16: q (and o) are bf16, else fp16.  kv: KvKind.
hipError_t launch_decode(const DecodeParams& p, int num_tiles, bool q_bf16, int kv,
                         hipStream_t s) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_decode_t<kKvE4M3, true>(p, num_tiles, s)
                  : launch_decode_t<kKvE4M3, false>(p, num_tiles, s);
  return q_bf16 ? launch_decode_t<kKvBF16, true>(p, num_tiles, s)
                : launch_decode_t<kKvF16, false>(p, num_tiles, s);
}

hipError_t launch_prefix(const DecodeParams& p, int num_tiles, bool q_bf16, int kv,
                         hipStream_t s) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_prefix_t<kKvE4M3, true>(p, num_tiles, s)
                  : launch_prefix_t<kKvE4M3, false>(p, num_tiles, s);
  return q_bf16 ? launch_prefix_t<kKvBF16, true>(p, num_tiles, s)
                : launch_prefix_t<kKvF16, false>(p, num_tiles, s);
}

}  // namespace fi
