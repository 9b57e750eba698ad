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
// V[token(g, kk)][16 b + n] for kk = 0..7, with two gfx950 transpose reads.
// ds_read_b64_tr_b16 works per 16-lane group: lane i's element k is element
// i % 4 of the 4 x 16-bit row addressed by lane i / 4 + 4 k of its group.  So
// lane n addresses the d-quad n % 4 (columns 16 b + 4 (n % 4) ..) of the row
// of contraction element kk = n / 4 (first read) or 4 + n / 4 (second).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x4 read_vt(const uint8_t* vt, int g, int n, int b) {
  const int kk = n >> 2, col = (16 * b + 4 * (n & 3)) * 2;
  const uint8_t* a0 = vt + (4 * kk + g) * kVStride + col;
  const uint8_t* a1 = vt + (4 * (kk + 4) + g) * kVStride + col;
  const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
  const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
  const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
  return u32x4{w0.x, w0.y, w1.x, w1.y};
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
// decode tiles (page-staged)
// ============================================================================
// A workgroup of W waves owns W consecutive kv heads h0 .. h0+W-1 of one
// request over a token chunk.  Per 16-token step it loads the K and V rows
// of those heads for the 16 tokens -- W * row bytes contiguous per token, a
// whole 32 KiB page when W = Hkv = 8 and page_size = 16 -- with 16-byte
// non-temporal loads, 1 KiB contiguous per wave instruction, into padded LDS
// tiles; then wave w computes kv head h0 + w from LDS:
//   scores  S^T[token][head] = K . Q^T, MFMA 16x16x32 (K rows from LDS in A
//           layout, q in B layout, columns past the group zero)
//   softmax online, base 2, lazy running max (see kLazyMax)
//   P.V     O^T[d][head] += V^T[d][token] . P^T[token][head], MFMA 16x16x16
//           with V^T read by ds_read_b64_tr_b16 and P^T straight from the
//           score accumulator layout.
// Page indices run two steps ahead; the next step's K/V loads are in flight
// in registers while the current step computes.  fp8 K stays fp8 in LDS
// (converted after the read); fp8 V is converted to 16-bit on the LDS write.
constexpr float kLazyMax = 8.f;
constexpr int kStep = 16;

template <int KV>
struct Stage {
  static constexpr int ROWB = KV == kKvE4M3 ? 128 : 256;  // K/V row bytes in HBM
  static constexpr int VR = ROWB / 16;                    // 16-B vectors per row
  static constexpr int LOADS = ROWB / 64;                 // vectors per thread per pool per step
  static constexpr int TOK_PER_U = 64 / VR;               // token advance per load index u
  static __host__ __device__ constexpr int k_stride(int W) { return W * ROWB + 16; }
  static __host__ __device__ constexpr int v_stride(int W) { return W * 256 + 32; }
  static __host__ __device__ constexpr int lds_bytes(int W) {
    return kStep * (k_stride(W) + v_stride(W));
  }
};

template <bool QBF16>
__device__ __forceinline__ f32x4 mma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  if constexpr (QBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

template <int KV, bool QBF16, bool PS_POW2>
__global__ __launch_bounds__(64 * kWavesPerTile) void decode_kernel(DecodeParams p) {
  using S = Stage<KV>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int W = blockDim.x >> 6;                  // waves = kv heads of the tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Tile tile = p.tiles[blockIdx.x];
  const int h0 = tile.kv_head0;
  const int h = h0 + wave;
  const int g = lane >> 4, n = lane & 15;
  const int r = tile.req, t0 = tile.t0, t1 = tile.t1;
  const int G = p.G;
  const int ps = p.page_size, ps_shift = p.ps_shift;
  const int page_base = p.kv_indptr[r];
  const int KS = S::k_stride(W), VS = S::v_stride(W);
  uint8_t* klds = lds;
  uint8_t* vlds = lds + kStep * KS;

  // q of this wave's head group as the B operand of the score MFMAs
  u32x4 qop[4];
  {
    const bool ok = n < G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)r * p.Hq + h * G + (ok ? n : 0)) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
      qop[s] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  float c = p.sm_scale_log2;
  if (KV == kKvE4M3 && p.k_scale) c *= p.k_scale[h];

  // cooperative loader: load u of thread tid covers token tk0 + u * TOK_PER_U
  // of the step and 16-byte vector vin of that token's W-head run
  const int tk0 = tid / (S::VR * W);
  const int vin = tid - tk0 * (S::VR * W);
  const char* kbase = reinterpret_cast<const char*>(p.k_pages) + (int64_t)h0 * S::ROWB + 16 * vin;
  const char* vbase = reinterpret_cast<const char*>(p.v_pages) + (int64_t)h0 * S::ROWB + 16 * vin;
  const uint32_t slot_bytes = (uint32_t)p.Hkv * S::ROWB;
  const int last = t1 - 1;
  const int nsteps = (t1 - t0 + kStep - 1) / kStep;

  // page of token t0 + 16 step + (lane & 15), clamped to the tile
  auto load_page = [&](int step) -> int {
    const int t = min(t0 + kStep * step + (lane & 15), last);
    const int pi = PS_POW2 ? (t >> ps_shift) : (t / ps);
    return p.kv_indices[page_base + pi];
  };
  u32x4 kr[S::LOADS], vr[S::LOADS];
  auto issue = [&](int step, int pg) {
    const int tb = t0 + kStep * step;
#pragma unroll
    for (int u = 0; u < S::LOADS; ++u) {
      const int tk = tk0 + u * S::TOK_PER_U;
      const int t = min(tb + tk, last);
      const uint32_t page = (uint32_t)__shfl(pg, t - tb);
      const uint32_t slot = PS_POW2 ? ((page << ps_shift) | (uint32_t)(t & (ps - 1)))
                                    : (page * (uint32_t)ps + (uint32_t)(t % ps));
      const uint64_t off = (uint64_t)slot * slot_bytes;
      kr[u] = ld_stream<u32x4>(kbase, off);
      vr[u] = ld_stream<u32x4>(vbase, off);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < S::LOADS; ++u) {
      const int tk = tk0 + u * S::TOK_PER_U;
      *reinterpret_cast<u32x4*>(klds + tk * KS + 16 * vin) = kr[u];
      if constexpr (KV == kKvE4M3) {
        const u32x2 a = e4m3x4_to_16<QBF16>(vr[u].x), b = e4m3x4_to_16<QBF16>(vr[u].y);
        const u32x2 c2 = e4m3x4_to_16<QBF16>(vr[u].z), d = e4m3x4_to_16<QBF16>(vr[u].w);
        uint8_t* dst = vlds + tk * VS + 32 * vin;
        *reinterpret_cast<u32x4*>(dst) = u32x4{a.x, a.y, b.x, b.y};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{c2.x, c2.y, d.x, d.y};
      } else {
        *reinterpret_cast<u32x4*>(vlds + tk * VS + 16 * vin) = vr[u];
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this lane's LDS addresses: K row of token n; V^T source row 4g + n/4 at
  // d-quad n % 4 (transpose-read layout)
  const uint8_t* krow = klds + n * KS + wave * S::ROWB;
  const uint8_t* vsrc = vlds + (4 * g + (n >> 2)) * VS + wave * 256 + 8 * (n & 3);

  auto compute = [&](int step) {
    const int tb = t0 + kStep * step;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 kop;
      if constexpr (KV == kKvE4M3) {
        const u32x2 w8 = *reinterpret_cast<const u32x2*>(krow + 32 * s + 8 * g);
        const u32x2 a = e4m3x4_to_16<QBF16>(w8.x), b = e4m3x4_to_16<QBF16>(w8.y);
        kop = u32x4{a.x, a.y, b.x, b.y};
      } else {
        kop = *reinterpret_cast<const u32x4*>(krow + 64 * s + 16 * g);
      }
      sc = mma16x16x32<QBF16>(kop, qop[s], sc);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sc[i] * c;
    if (tb + kStep > t1) {                       // tail step: mask tokens past t1
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tb + 4 * g + i >= t1) x[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m + kLazyMax;
    if (__any(move)) {
      const float m_new = move ? mx : m;
      const float alpha = fast_exp2(m - m_new);   // m = -inf first: 0
      l *= alpha;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) oacc[bb] *= alpha;
      m = m_new;
    }
    // every step has a valid token, so m is finite here
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[i] - m);
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const u32x2 pop = {pack2<QBF16>(pr[0], pr[1]), pack2<QBF16>(pr[2], pr[3])};
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 32 * bb));
      oacc[bb] = mma16x16x16<QBF16>(__builtin_bit_cast(u32x2, vt), pop, oacc[bb]);
    }
  };

  // ---- pipelined step loop
  if (nsteps > 0) {
    int pg1 = nsteps > 1 ? load_page(1) : 0;
    issue(0, load_page(0));
    for (int step = 0; step < nsteps; ++step) {
      const int pg2 = step + 2 < nsteps ? load_page(step + 2) : 0;
      stage();
      __syncthreads();
      if (step + 1 < nsteps) issue(step + 1, pg1);
      compute(step);
      __syncthreads();
      pg1 = pg2;
    }
  }

  // ---- finalize
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (KV == kKvE4M3 && p.v_scale) inv *= p.v_scale[h];
  const float lse2 = lt > 0.f ? m + fast_log2(lt) : -INFINITY;
  const int j = h * G + n;
  if (tile.slot < 0) {
    if (n < G) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)r * p.Hq + j) * kHeadDim;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        u32x2 w = {pack2<QBF16>(oacc[b][0] * inv, oacc[b][1] * inv),
                   pack2<QBF16>(oacc[b][2] * inv, oacc[b][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * b + 4 * g) = w;
      }
      if (g == 0 && p.lse) p.lse[(int64_t)r * p.Hq + j] = lse2 * kLn2;
    }
    return;
  }
  const int64_t slot = tile.slot + wave;
  if (n < G) {
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
        kr[u] = ld_stream<u32x4>(kbase, off + 16 * cc);
        vr[u] = ld_stream<u32x4>(vbase, off + 16 * cc);
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
static hipError_t launch_decode_t(const DecodeParams& p, int num_tiles, int waves,
                                  hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  const size_t lds = (size_t)Stage<KV>::lds_bytes(waves);
  // dynamic LDS above 64 KiB must be allowed per kernel (once per process)
  static const hipError_t attr = [] {
    const int max_lds = Stage<KV>::lds_bytes(kWavesPerTile);
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, true>), dim3(num_tiles), dim3(64 * waves), lds,
                       s, p);
  else
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, false>), dim3(num_tiles), dim3(64 * waves), lds,
                       s, p);
  return hipGetLastError();
}

template <int KV, bool QBF16>
static hipError_t launch_prefix_t(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefix_kernel<KV, QBF16>), dim3(num_tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

// q_bf16: q (and o) are bf16, else fp16.  kv: KvKind.
hipError_t launch_decode(const DecodeParams& p, int num_tiles, int waves, bool q_bf16,
                         int kv, hipStream_t s) {
  if (waves < 1 || waves > kWavesPerTile) return hipErrorInvalidValue;
  if (kv == kKvE4M3)
    return q_bf16 ? launch_decode_t<kKvE4M3, true>(p, num_tiles, waves, s)
                  : launch_decode_t<kKvE4M3, false>(p, num_tiles, waves, s);
  return q_bf16 ? launch_decode_t<kKvBF16, true>(p, num_tiles, waves, s)
                : launch_decode_t<kKvF16, false>(p, num_tiles, waves, s);
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
