// decode.hip -- gfx950 paged decode attention, cascade prefix and append
// kernels.
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
//  * decode_kernel: a workgroup is W waves (W = kv heads per tile, 1..8) of
//    one request over a token chunk; wave w computes kv head kv_head0 + w,
//    so the G query heads that share it read each K/V row once.  Per
//    16-token step the workgroup streams the step's K and V rows of its W
//    heads (W x row bytes contiguous per token: a whole 32 KiB page at
//    W = Hkv = 8, page_size 16, D 128 fp16) with 16-byte non-temporal loads
//    into padded LDS tiles; the next step's loads are in flight while a
//    step computes.
//  * Scores S^T[token][head] = K . Q^T on MFMA 16x16x32 (K from LDS in the A
//    operand, q in the B operand for the whole tile, columns n >= G zero).
//    The D layout leaves lane (g, n) with tokens 4g..4g+3 of head n, so the
//    row max needs two cross-lane exchanges and P^T is already in B-operand
//    layout.
//  * P.V: O^T[d][head] += V^T[d][token] . P^T[token][head] on MFMA 16x16x16,
//    V^T read from LDS with gfx950's ds_read_b64_tr_b16 transpose read.
//  * E4M3 K/V are converted to the q dtype (exact) with the per-kv-head
//    scales folded into the score scale and the output.
//  * A tile whose (request, kv head) is split over several chunks writes an
//    fp32 partial state (o, log2-domain lse) that merge.hip combines; a
//    cascade suffix tile folds its request's prefix states in instead.
//  * LLaMA-style RoPE (README decode example, pos_encoding_mode): the
//    decode kernel turns each key by its distance from the query before the
//    score MFMAs (described above rope_key8).
//  * prefix_kernel: many query rows against one chunk of one key list, K/V
//    staged in LDS and shared by 8 waves x 32 rows (16 at head_dim 256) --
//    the G heads of every request of a cascade group against the shared
//    prefix, or the query tokens of an append request (README append
//    example, causal mask) against its own keys; described above the kernel.
//  * K/V rows are addressed by page, slot and head strides: NHD or HND
//    pages, or the ragged layout (page size 1, no page table).
//  * head_dim D (64, 128, 256) is a template parameter: D / 32 q operands
//    and D / 16 output blocks per lane; at 256 prefix_kernel gives each wave
//    one 16-row column tile instead of two (registers).
#include <algorithm>
#include <type_traits>

#include "fi_device.h"

namespace fi {

// gfx950 transpose read of 16-bit LDS data (ds_read_b64_tr_b16), used for
// the V^T operand of P.V.  It works per 16-lane group: lane i's element k is
// element i % 4 of the 4 x 16-bit row addressed by lane i / 4 + 4 k of its
// group (layout measured with a probe).  So a lane that addresses the d-quad
// n % 4 of the row holding contraction element kk = n / 4 receives, over its
// four elements, that d column for four consecutive contraction elements.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ============================================================================
// decode tiles (page-staged)
// ============================================================================
// A workgroup of W waves owns W consecutive kv heads h0 .. h0+W-1 of one
// request over a token chunk.  Per 16-token step it loads the K and V rows
// of those heads for the 16 tokens -- W * row bytes contiguous per token, a
// whole 32 KiB page when W = Hkv = 8, page_size = 16 and D = 128 in fp16 --
// with 16-byte non-temporal loads, 1 KiB contiguous per wave instruction,
// into padded LDS tiles; then wave w computes kv head h0 + w from LDS:
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

template <int KV, int D>
struct Stage {
  static constexpr int ROWB = KV == kKvE4M3 ? D : 2 * D;  // K/V row bytes in HBM
  static constexpr int VR = ROWB / 16;                    // 16-B vectors per row
  static constexpr int LOADS = ROWB / 64;                 // vectors per thread per pool per step
  static constexpr int TOK_PER_U = 64 / VR;               // token advance per load index u
  static __host__ __device__ constexpr int k_stride(int W) { return W * ROWB + 16; }
  static __host__ __device__ constexpr int v_stride(int W) { return W * 2 * D + 32; }
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

// Folds nst earlier attention states of this wave's query rows into its own
// unnormalised state.  Lane (g, n) holds, for q head n of the group, the
// running reference M (log2 units), the mass S = sum 2^(x - M) and
// A[b][i] = sum 2^(x - M) v[16 b + 4 g + i].  State c (fp32 normalised o_c
// and log2-lse s_c, at partial row (slot_base + c Hkv + h) G + n) has mass
// 2^(s_c - M) and contributes that times o_c; the reference moves up to s_c
// when s_c is larger, so every weight stays <= 1.  One state per round trip
// (the fold runs once per tile; its registers stay within the main loop's).
template <int D>
__device__ __forceinline__ void fold_states(const float* __restrict__ partial_o,
                                            const float* __restrict__ partial_lse,
                                            int slot_base, int nst, int Hkv, int h, int G, int n,
                                            int g, f32x4 (&A)[D / 16], float& M, float& S) {
  const int nn = n < G ? n : 0, col = 4 * g;
  for (int c = 0; c < nst; ++c) {
    const int64_t row = ((int64_t)slot_base + (int64_t)c * Hkv + h) * G + nn;
    const float s = partial_lse[row];
    const float* po = partial_o + row * D + col;
    f32x4 o[D / 16];
#pragma unroll
    for (int b = 0; b < D / 16; ++b) o[b] = *reinterpret_cast<const f32x4*>(po + 16 * b);
    // branch-free (selects keep one copy of A live): new reference
    // M' = max(M, s), old mass scaled by 2^(M - M'), state weight 2^(s - M')
    const float Mn = fmaxf(M, s);
    const float f = M == Mn ? 1.f : fast_exp2(M - Mn);     // M = -inf < s: 0
    const float w = s == -INFINITY ? 0.f : fast_exp2(s - Mn);
    S = S * f + w;
#pragma unroll
    for (int b = 0; b < D / 16; ++b) A[b] = A[b] * f + w * o[b];
    M = Mn;
  }
}

// ---- RoPE ---------------------------------------------------------------------
// The rotation is applied in its relative form: turning q by the angle of
// its position p and key t by that of t is, for the dot product, the same as
// turning the key alone by the angle of t - p (rotations compose and are
// orthogonal).  So q enters the score MFMAs as stored, and each key is turned
// back by its distance d = p - t >= 0 from the query.
//
// Table (fp32, built on the device in fp64): row d, frequency i holds
// (cos, sin) of d / scale * theta^(-2 i / D).  A step needs the rows of
// distances d0 - n, n < 16 (d0 = p - first token of the step); the
// workgroup builds them in LDS from row d0 and rows 0..15 by the
// angle-difference identities, each (n, i) once.
template <bool BF16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (BF16) return __builtin_bit_cast(float, w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffff));
}
template <bool BF16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (BF16) return __builtin_bit_cast(float, w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// (x0 - h.lo, x1 - h.hi) rounded to the 16-bit type, h = the pair (x0, x1)
// already rounded.  f16: one mixed-precision FMA per half (the f16 operand
// is widened inside the instruction, the result rounded to f16 in place).
template <bool BF16>
__device__ __forceinline__ uint32_t residual2(uint32_t h, float x0, float x1) {
  if constexpr (BF16) {
    return pack2<true>(x0 - lo16<true>(h), x1 - hi16<true>(h));
  } else {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(r)
        : "v"(h), "v"(x0), "v"(x1));
    return r;
  }
}

// Turns 8 + 8 partner elements of one key (a: dims f..f+7, b: dims
// f+64..f+71, 16-bit) back by its distance, (cos, sin) of frequencies
// f..f+7 in cs, in fp32; writes the result as a 16-bit high part plus a
// 16-bit residual, so that two MFMAs against the same q carry the rotated
// key to about fp32 accuracy.
template <bool BF16>
__device__ __forceinline__ void rope_key8(u32x4 a, u32x4 b, const float4* cs, u32x4& ahi,
                                          u32x4& alo, u32x4& bhi, u32x4& blo) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 t = cs[k];   // frequencies f + 2k, f + 2k + 1
    float ra[2], rb[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float c = e ? t.z : t.x, sn = e ? t.w : t.y;
      const float x = e ? hi16<BF16>(a[k]) : lo16<BF16>(a[k]);
      const float y = e ? hi16<BF16>(b[k]) : lo16<BF16>(b[k]);
      ra[e] = __builtin_fmaf(x, c, __builtin_fmaf(y, sn, 0.f));
      rb[e] = __builtin_fmaf(y, c, __builtin_fmaf(-x, sn, 0.f));
    }
    ahi[k] = pack2<BF16>(ra[0], ra[1]);
    bhi[k] = pack2<BF16>(rb[0], rb[1]);
    alo[k] = residual2<BF16>(ahi[k], ra[0], ra[1]);
    blo[k] = residual2<BF16>(bhi[k], rb[0], rb[1]);
  }
}

// (cos, sin) table of the plan: one thread per (distance, frequency), angle
// in fp64 from the definition, stored as two fp32.
__global__ void rope_table_kernel(float2* table, int rows, int D, double theta, double scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * (D / 2)) return;
  const int d = (int)(i / (D / 2)), f = (int)(i % (D / 2));
  const double ang = (d / scale) * pow(theta, -2.0 * f / D);
  table[i] = float2{(float)cos(ang), (float)sin(ang)};
}

hipError_t launch_rope_table(void* table, int rows, int head_dim, float theta, float scale,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = (int64_t)rows * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<float2*>(table), rows, head_dim, (double)theta,
                     (double)scale);
  return hipGetLastError();
}

// FOLD: the plan has tiles that fold earlier states into their output (a
// separate instance: the fold costs registers the plain kernel keeps free).
// DEPTH: steps of K/V loads in flight per workgroup.  ROPE: every key is
// turned by its distance from the query (LLaMA-style RoPE, relative form)
// before the score MFMAs; the LDS after K and V holds the step's 16 rows
// (padded: conflict-free reads of one row per lane) and table rows 0..15.
template <int D>
struct RopeLds {
  static constexpr int FREQ = D / 2;                 // frequencies (table row entries)
  static constexpr int ROW = rope_row_bytes(D);      // table row bytes
  static constexpr int STRIDE = ROW + 16;            // the step's rows in LDS (padded)
  static constexpr int BYTES = kStep * STRIDE + kStep * ROW;
  static constexpr int FPL = (FREQ + 63) / 64;       // frequencies per lane
};
template <int KV, bool QBF16, bool PS_POW2, bool FOLD, int DEPTH, bool ROPE, int D>
__global__ __launch_bounds__(64 * kWavesPerTile) void decode_kernel(DecodeParams p) {
  static_assert(!ROPE || !FOLD, "RoPE plans have no cascade level to fold");
  using S = Stage<KV, D>;
  using RL = RopeLds<D>;
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
  const int page_base = tile.row0;   // kv_indptr[r], copied by the plan
  // slots of the states a final tile folds in (read now, used at the end)
  const int fold_base = FOLD && tile.slot < 0 && tile.row1 > 0 ? p.req_info[r].slot_base : 0;
  const int KS = S::k_stride(W), VS = S::v_stride(W);
  uint8_t* klds = lds;
  uint8_t* vlds = lds + kStep * KS;
  uint8_t* rlds = lds + kStep * (KS + VS);   // RoPE: the step's rows
  const float2* r16 = reinterpret_cast<const float2*>(rlds + kStep * RL::STRIDE);

  // q of this wave's head group as the B operand of the score MFMAs
  u32x4 qop[D / 32];
  {
    const bool ok = n < G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)r * p.Hq + h * G + (ok ? n : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
      qop[s] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  // RoPE: the query sits at position kv_len - 1
  const int qpos = ROPE ? p.req_info[r].kv_len - 1 : 0;
  float c = p.sm_scale_log2;
  if (KV == kKvE4M3 && p.k_scale) c *= p.k_scale[h];

  // cooperative loader: load u of thread tid covers token tk0 + u * TOK_PER_U
  // of the step and 16-byte vector vin of that token's W-head run
  const int tk0 = tid / (S::VR * W);
  const int vin = tid - tk0 * (S::VR * W);
  // vector vin = head vin / VR of the tile's run, 16-byte chunk vin % VR
  const int vh = vin / S::VR, vc = vin - vh * S::VR;
  const int64_t hoff = (int64_t)(h0 + vh) * p.head_stride + 16 * vc;
  const char* kbase = reinterpret_cast<const char*>(p.k_pages) + hoff;
  const char* vbase = reinterpret_cast<const char*>(p.v_pages) + hoff;
  const int last = t1 - 1;
  const int nsteps = (t1 - t0 + kStep - 1) / kStep;

  // page of token t0 + 16 step + (lane & 15), clamped to the tile
  auto load_page = [&](int step) -> int {
    const int t = min(t0 + kStep * step + (lane & 15), last);
    const int pi = PS_POW2 ? (t >> ps_shift) : (t / ps);
    return p.ragged ? page_base + pi : p.kv_indices[page_base + pi];
  };
  // DEPTH register sets of step loads (kr/vr[d]); set d holds steps d, d +
  // DEPTH, ...
  u32x4 kr[DEPTH][S::LOADS], vr[DEPTH][S::LOADS];
  // RoPE: thread (wave w, lane i) builds entries (n, f) of the step's rows
  // for n = w, w + W, ... and frequencies f = i + 64 k < D / 2: it holds
  // (cos, sin) at distance d0 for those frequencies (2 registers each per
  // step in flight) and reads rows n from LDS
  struct RopeRow {
    float2 v[RL::FPL];
  };
  const float2* rtab = reinterpret_cast<const float2*>(p.rope_table);
  RopeRow rr[DEPTH];
  auto issue_rope = [&](int step, RopeRow& rq) {
    if constexpr (ROPE) {
#pragma unroll
      for (int k = 0; k < RL::FPL; ++k) {
        const int f = lane + 64 * k;
        if (RL::FREQ % 64 == 0 || f < RL::FREQ)
          rq.v[k] = rtab[(int64_t)(qpos - t0 - kStep * step) * RL::FREQ + f];
      }
    }
  };
  auto stage_rope = [&](const RopeRow& rq) {
    if constexpr (ROPE) {
      for (int nn = wave; nn < kStep; nn += W) {
#pragma unroll
        for (int k = 0; k < RL::FPL; ++k) {
          const int f = lane + 64 * k;
          if (RL::FREQ % 64 == 0 || f < RL::FREQ) {
            const float2 o = r16[nn * RL::FREQ + f];
            const float2 q = rq.v[k];
            const float c = __builtin_fmaf(q.x, o.x, q.y * o.y);    // cos((d0 - n) w)
            const float sn = __builtin_fmaf(q.y, o.x, -q.x * o.y);  // sin((d0 - n) w)
            *reinterpret_cast<float2*>(rlds + nn * RL::STRIDE + 8 * f) = float2{c, sn};
          }
        }
      }
    }
  };
  if constexpr (ROPE) {
    constexpr int kVec = kStep * RL::ROW / 16;   // rows 0..15 in 16-byte vectors
    constexpr int kPer = (kVec + 63) / 64;       // per thread at W = 1
    const u32x4* src = reinterpret_cast<const u32x4*>(p.rope_table);
    u32x4* dst = reinterpret_cast<u32x4*>(rlds + kStep * RL::STRIDE);
    u32x4 o16[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (tid + u * 64 * W < kVec) o16[u] = src[tid + u * 64 * W];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (tid + u * 64 * W < kVec) dst[tid + u * 64 * W] = o16[u];
    __syncthreads();   // rows 0..15 are read across waves by the first stage
  }
  auto issue = [&](int step, int pg, u32x4 (&kq)[S::LOADS], u32x4 (&vq)[S::LOADS]) {
    const int tb = t0 + kStep * step;
#pragma unroll
    for (int u = 0; u < S::LOADS; ++u) {
      const int tk = tk0 + u * S::TOK_PER_U;
      const int t = min(tb + tk, last);
      const uint32_t page = (uint32_t)__shfl(pg, t - tb);
      const uint32_t sl = PS_POW2 ? (uint32_t)(t & (ps - 1)) : (uint32_t)(t % ps);
      const uint64_t off = (uint64_t)page * p.page_bytes + sl * p.slot_stride;
      kq[u] = ld_stream<u32x4>(kbase, off);
      vq[u] = ld_stream<u32x4>(vbase, off);
    }
  };
  auto stage = [&](const u32x4 (&kq)[S::LOADS], const u32x4 (&vq)[S::LOADS]) {
#pragma unroll
    for (int u = 0; u < S::LOADS; ++u) {
      const int tk = tk0 + u * S::TOK_PER_U;
      *reinterpret_cast<u32x4*>(klds + tk * KS + 16 * vin) = kq[u];
      if constexpr (KV == kKvE4M3) {
        const u32x2 a = e4m3x4_to_16<QBF16>(vq[u].x), b = e4m3x4_to_16<QBF16>(vq[u].y);
        const u32x2 c2 = e4m3x4_to_16<QBF16>(vq[u].z), d = e4m3x4_to_16<QBF16>(vq[u].w);
        uint8_t* dst = vlds + tk * VS + 32 * vin;
        *reinterpret_cast<u32x4*>(dst) = u32x4{a.x, a.y, b.x, b.y};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{c2.x, c2.y, d.x, d.y};
      } else {
        *reinterpret_cast<u32x4*>(vlds + tk * VS + 16 * vin) = vq[u];
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int b = 0; b < D / 16; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this lane's LDS addresses: K row of token n; V^T source row 4g + n/4 at
  // d-quad n % 4 (transpose-read layout)
  const uint8_t* krow = klds + n * KS + wave * S::ROWB;
  const uint8_t* vsrc = vlds + (4 * g + (n >> 2)) * VS + wave * (2 * D) + 8 * (n & 3);

  auto compute = [&](int step) {
    const int tb = t0 + kStep * step;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    // lane (g, n): dims 32 s + 8 g .. +7 of key n of the step
    auto kop_of = [&](int s) -> u32x4 {
      if constexpr (KV == kKvE4M3) {
        const u32x2 w8 = *reinterpret_cast<const u32x2*>(krow + 32 * s + 8 * g);
        const u32x2 a = e4m3x4_to_16<QBF16>(w8.x), b = e4m3x4_to_16<QBF16>(w8.y);
        return u32x4{a.x, a.y, b.x, b.y};
      } else {
        return *reinterpret_cast<const u32x4*>(krow + 64 * s + 16 * g);
      }
    };
    if constexpr (ROPE) {
      // dims of kop(j) (frequencies 32 j + 8 g ..) pair with kop(j + D / 64)
      constexpr int HALF = D / 64;
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const float4* cs =
            reinterpret_cast<const float4*>(rlds + n * RL::STRIDE + 256 * j + 64 * g);
        u32x4 ahi, alo, bhi, blo;
        rope_key8<QBF16>(kop_of(j), kop_of(j + HALF), cs, ahi, alo, bhi, blo);
        sc = mma16x16x32<QBF16>(ahi, qop[j], sc);
        sc = mma16x16x32<QBF16>(alo, qop[j], sc);
        sc = mma16x16x32<QBF16>(bhi, qop[j + HALF], sc);
        sc = mma16x16x32<QBF16>(blo, qop[j + HALF], sc);
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) sc = mma16x16x32<QBF16>(kop_of(s), qop[s], sc);
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
      for (int bb = 0; bb < D / 16; ++bb) oacc[bb] *= alpha;
      m = m_new;
    }
    // every step has a valid token, so m is finite here
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[i] - m);
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    const u32x2 pop = {pack2<QBF16>(pr[0], pr[1]), pack2<QBF16>(pr[2], pr[3])};
    // bf16 V: p also as a bf16 residual (bf16 keeps 8 bits of p; with a few
    // comparable keys that alone moves o past the accuracy bar)
    u32x2 plo;
    if constexpr (KV == kKvBF16)
      plo = u32x2{pack2<true>(pr[0] - lo16<true>(pop.x), pr[1] - hi16<true>(pop.x)),
                  pack2<true>(pr[2] - lo16<true>(pop.y), pr[3] - hi16<true>(pop.y))};
#pragma unroll
    for (int bb = 0; bb < D / 16; ++bb) {
      const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 32 * bb));
      oacc[bb] = mma16x16x16<QBF16>(__builtin_bit_cast(u32x2, vt), pop, oacc[bb]);
      if constexpr (KV == kKvBF16)
        oacc[bb] = mma16x16x16<QBF16>(__builtin_bit_cast(u32x2, vt), plo, oacc[bb]);
    }
  };

  // ---- pipelined step loop: the loads of the next DEPTH steps are in
  // flight while a step computes; page indices are read DEPTH + 1 steps
  // ahead of their loads
  if constexpr (DEPTH == 1) {
    if (nsteps > 0) {
      int pg1 = nsteps > 1 ? load_page(1) : 0;
      issue(0, load_page(0), kr[0], vr[0]);
      issue_rope(0, rr[0]);
      for (int step = 0; step < nsteps; ++step) {
        const int pg2 = step + 2 < nsteps ? load_page(step + 2) : 0;
        stage(kr[0], vr[0]);
        stage_rope(rr[0]);
        __syncthreads();
        if (step + 1 < nsteps) {
          issue(step + 1, pg1, kr[0], vr[0]);
          issue_rope(step + 1, rr[0]);
        }
        compute(step);
        __syncthreads();
        pg1 = pg2;
      }
    }
  } else {
    if (nsteps > 0) {
      issue(0, load_page(0), kr[0], vr[0]);
      issue_rope(0, rr[0]);
      if (nsteps > 1) {
        issue(1, load_page(1), kr[1], vr[1]);
        issue_rope(1, rr[DEPTH - 1]);
      }
      int pga = nsteps > 2 ? load_page(2) : 0;   // page of the next even step to issue
      int pgb = nsteps > 3 ? load_page(3) : 0;   // ... odd step
      // one body per register set: set d stages step s and refills with s + 2
      auto body = [&](int step, int& pgn, u32x4 (&kq)[S::LOADS], u32x4 (&vq)[S::LOADS],
                      RopeRow& rq) {
        stage(kq, vq);
        stage_rope(rq);
        __syncthreads();
        if (step + 2 < nsteps) {
          issue(step + 2, pgn, kq, vq);
          issue_rope(step + 2, rq);
        }
        pgn = step + 4 < nsteps ? load_page(step + 4) : 0;
        compute(step);
        __syncthreads();
      };
      for (int step = 0; step < nsteps; step += 2) {
        body(step, pga, kr[0], vr[0], rr[0]);
        if (step + 1 < nsteps) body(step + 1, pgb, kr[1], vr[1], rr[DEPTH - 1]);
      }
    }
  }

  // ---- finalize
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  const float vs = (KV == kKvE4M3 && p.v_scale) ? p.v_scale[h] : 1.f;
  const int j = h * G + n;
  if (tile.slot < 0) {
    // final output; a cascade request whose suffix is this one tile first
    // folds in the states its prefix tiles left (tile.row1 of them)
    float M = m, S = lt, osc = vs;
    if (FOLD && tile.row1 > 0) {
      if (KV == kKvE4M3) {
#pragma unroll
        for (int b = 0; b < D / 16; ++b) oacc[b] *= vs;
        osc = 1.f;
      }
      fold_states<D>(p.partial_o, p.partial_lse, fold_base, tile.row1, p.Hkv, h, G, n, g, oacc,
                  M, S);
    }
    const float inv = (S > 0.f ? 1.f / S : 0.f) * osc;
    const float lse2 = S > 0.f ? M + fast_log2(S) : -INFINITY;
    if (n < G) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)r * p.Hq + j) * D;
#pragma unroll
      for (int b = 0; b < D / 16; ++b) {
        u32x2 w = {pack2<QBF16>(oacc[b][0] * inv, oacc[b][1] * inv),
                   pack2<QBF16>(oacc[b][2] * inv, oacc[b][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * b + 4 * g) = w;
      }
      if (g == 0 && p.lse) p.lse[(int64_t)r * p.Hq + j] = lse2 * kLn2;
    }
    return;
  }
  const float inv = (lt > 0.f ? 1.f / lt : 0.f) * vs;
  const float lse2 = lt > 0.f ? m + fast_log2(lt) : -INFINITY;
  const int64_t slot = tile.slot + wave;
  if (n < G) {
    float* po = p.partial_o + (slot * G + n) * D;
#pragma unroll
    for (int b = 0; b < D / 16; ++b)
      *reinterpret_cast<f32x4*>(po + 16 * b + 4 * g) = oacc[b] * inv;
    if (g == 0) p.partial_lse[slot * G + n] = lse2;
  }
}

// ============================================================================
// cascade prefix tiles: many query rows x one prefix chunk of one kv head.
// ============================================================================
// Workgroup = WAVES waves; wave w owns query rows row0 + 16 RT w + 16 rt + n
// (rt < RT: 2 row tiles, 1 at head_dim 256) as the N columns of its MFMAs,
// so each K/V element staged in LDS serves 16 RT WAVES rows.  The tile's slice of the page table is copied to LDS
// once.  Per 32-token step the workgroup loads the step's K and V rows of the
// tile's kv head (NL 16-byte vectors per thread) two steps ahead into
// registers, stores them to one of two LDS buffers after computing from the
// other, one barrier per step.  Scores: MFMA 16x16x32 with every K operand of
// the step read from LDS up front; the V^T operands (transpose reads) are
// issued before the softmax so their latency hides under it.  Softmax: the
// probabilities are formed against the running max m; only when a lane's sum
// of them exceeds kPrefixLazySum (or is not finite: the first step, where m =
// -inf) does the wave take the exact row max, rescale and recompute, so the
// common step carries no max reduction.  P.V: MFMA 16x16x32.  The prefix is
// reused across row tiles, so its loads use the default (cached) policy, and
// the block -> tile map puts all row tiles of one (head, chunk) on the same
// XCD (workgroups are dispatched to the 8 XCDs round-robin) so they share
// that XCD's L2.
//
// The same kernel runs append tiles (APPEND): the rows are the query tokens
// of one request (token-major, G heads each) over that request's own pages;
// row i may attend keys below its limit (ReqInfo.kv_len of its token: its
// causal limit, or all keys without the mask), so a step that reaches past
// the smallest limit of the wave's rows masks per row, and a wave skips
// steps past the largest limit of its rows.
constexpr int kPStep = 32;
constexpr float kPrefixLazySum = 256.f;

template <int KV, int D>
struct PStage {
  static constexpr int ROWB = KV == kKvE4M3 ? D : 2 * D;    // K row bytes kept in LDS
  static constexpr int KS = ROWB + 16;                      // K LDS row stride
  static constexpr int VS = 2 * D + 32;                     // V LDS row stride (16-bit values)
  static constexpr int BUF = kPStep * (KS + VS);
  static constexpr int PTAB = kPrefixMaxChunk + 2;          // page-table slots (page_size 1)
  static constexpr int LDS = 2 * BUF + 4 * PTAB;
};

// XCD-aware map: block b runs on XCD b % 8; give each XCD a contiguous range
// of the (chunk, head, row tile)-ordered tile list.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int x = b & 7, k = b >> 3, per = n >> 3, rem = n & 7;
  return x * per + min(x, rem) + k;
}

template <int KV, bool QBF16, int WAVES, bool PS_POW2, bool APPEND, int D>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 && D != 256 ? 2 : 1) void prefix_kernel(
    DecodeParams p) {
  // row tiles (16 query rows each) per wave: two, one at D = 256
  constexpr int RT = prefix_rows_per_wave(D) / 16;
  using S = PStage<KV, D>;
  // bf16 append tiles: P.V takes p as a bf16 high part plus a bf16
  // residual -- bf16 keeps 8 bits of p, and when a few keys carry
  // comparable weight (the first rows of a prefill see a handful of keys)
  // that rounding alone moves o past the accuracy bar.  Cascade prefix tiles
  // keep one bf16 p: their rows see a long shared prefix, and both the
  // residual products and a per-tile choice (both paths' registers: 256
  // VGPRs with spills) cost the MFMA-bound prefix kernel more than a tenth.
  constexpr bool SPLITP = APPEND && KV == kKvBF16;
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

  // query rows of this lane's two column tiles (B operands of the scores)
  u32x4 qop[RT][D / 32];
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
  // token (idx % (32 VR)) / VR, chunk idx % VR.
  constexpr bool F8 = KV == kKvE4M3;
  constexpr int VR = S::ROWB / 16;
  constexpr int T = 64 * WAVES;
  constexpr int PV = 32 * VR;                       // vectors per pool per step
  constexpr int NL = (2 * PV + T - 1) / T;
  const char* kbase = reinterpret_cast<const char*>(p.k_pages) + (int64_t)h * p.head_stride;
  const char* vbase = reinterpret_cast<const char*>(p.v_pages) + (int64_t)h * p.head_stride;
  const int last = t1 - 1;
  auto load = [&](int tb, u32x4 (&vec)[NL]) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + u * T;
      if (2 * PV % T != 0 && idx >= 2 * PV) continue;
      const int q = idx % PV;
      const int t = min(tb + q / VR, last);
      const int pi = page_idx(t);
      const uint32_t sl = PS_POW2 ? (uint32_t)(t & (ps - 1)) : (uint32_t)(t - pi * ps);
      const uint32_t page = (uint32_t)ptab[pi - pfirst];
      const uint64_t off =
          (uint64_t)page * p.page_bytes + sl * p.slot_stride + 16 * (q % VR);
      vec[u] = ld_global<u32x4>(idx < PV ? kbase : vbase, off);
    }
  };
  auto store = [&](int buf, const u32x4 (&vec)[NL]) {
    uint8_t* kt = lds + buf * S::BUF;
    uint8_t* vt = kt + kPStep * S::KS;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + u * T;
      if (2 * PV % T != 0 && idx >= 2 * PV) continue;
      const int q = idx % PV;
      const int tok = q / VR, chk = q % VR;
      if (idx < PV) {
        *reinterpret_cast<u32x4*>(kt + tok * S::KS + 16 * chk) = vec[u];
      } else if constexpr (F8) {
        const u32x2 a = e4m3x4_to_16<QBF16>(vec[u].x), b = e4m3x4_to_16<QBF16>(vec[u].y);
        const u32x2 c2 = e4m3x4_to_16<QBF16>(vec[u].z), d = e4m3x4_to_16<QBF16>(vec[u].w);
        uint8_t* dv = vt + tok * S::VS + 32 * chk;
        *reinterpret_cast<u32x4*>(dv) = u32x4{a.x, a.y, b.x, b.y};
        *reinterpret_cast<u32x4*>(dv + 16) = u32x4{c2.x, c2.y, d.x, d.y};
      } else {
        *reinterpret_cast<u32x4*>(vt + tok * S::VS + 16 * chk) = vec[u];
      }
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
    const uint8_t* vt = kt + kPStep * S::KS;
    // ---- K operands of both token tiles (tokens 16 tt + n), all k slices
    u32x4 kop[2][D / 32];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint8_t* krow = kt + (16 * tt + n) * S::KS;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        if constexpr (F8) {
          const u32x2 w8 = *reinterpret_cast<const u32x2*>(krow + 32 * s + 8 * g);
          const u32x2 a = e4m3x4_to_16<QBF16>(w8.x), b = e4m3x4_to_16<QBF16>(w8.y);
          kop[tt][s] = u32x4{a.x, a.y, b.x, b.y};
        } else {
          kop[tt][s] = *reinterpret_cast<const u32x4*>(krow + 64 * s + 16 * g);
        }
      }
    }
    // ---- V^T operands: contraction element kk of lane group g is token
    // 4 g + (kk & 3) + 16 (kk >> 2); two transpose reads per dim block b
    u32x4 vop[D / 16];
    const uint8_t* vsrc = vt + (4 * g + (n >> 2)) * S::VS + 8 * (n & 3);
#pragma unroll
    for (int b = 0; b < D / 16; ++b) {
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 32 * b));
      const s16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vsrc + 16 * S::VS + 32 * b));
      const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
      vop[b] = u32x4{w0.x, w0.y, w1.x, w1.y};
    }
    // ---- scores: S[tt][rt] = K(tokens 16 tt ..) . Q^T(rows of tile rt);
    // the four accumulators are independent, so consecutive MFMAs never wait
    f32x4 sc[2][RT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) sc[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          sc[tt][rt] = mma16x16x32<QBF16>(kop[tt][s], qop[rt][s], sc[tt][rt]);
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
    if constexpr (SPLITP) {
#pragma unroll
      for (int b = 0; b < D / 16; ++b) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          oacc[rt][b] = mma16x16x32<QBF16>(vop[b], pop[rt], oacc[rt][b]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          oacc[rt][b] = mma16x16x32<QBF16>(vop[b], plo[rt], oacc[rt][b]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < D / 16; ++b)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          oacc[rt][b] = mma16x16x32<QBF16>(vop[b], pop[rt], oacc[rt][b]);
    }
  };

  // two register sets: the one for step s + 1 is in flight while step s is
  // computed, the one for step s + 2 is issued at the start of step s
  u32x4 va[NL], vb[NL];
  __syncthreads();   // page table
  load(t0, va);
  store(0, va);
  if (nsteps > 1) load(t0 + kPStep, vb);
  __syncthreads();
  auto step_body = [&](int step, u32x4 (&nxt)[NL], u32x4 (&aft)[NL]) {
    const int tb = t0 + kPStep * step;
    if (step + 2 < nsteps) load(tb + 2 * kPStep, aft);
    if (tb < wave_hi) compute(tb, step & 1, tb + kPStep > wave_lo);
    if (step + 1 < nsteps) store((step + 1) & 1, nxt);
    __syncthreads();
  };
  for (int step = 0; step < nsteps; step += 2) {
    step_body(step, vb, va);
    if (step + 1 < nsteps) step_body(step + 1, va, vb);
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

// ---- launchers ----------------------------------------------------------------
// FI_DECODE_DEPTH=1 keeps one step in flight for every workgroup size (for
// measurement); read once.
static int getenv_depth() {
  static const int d = [] {
    const char* v = getenv("FI_DECODE_DEPTH");
    return v && *v ? atoi(v) : 0;
  }();
  return d;
}

constexpr int kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950

template <int KV, bool QBF16, bool FOLD, int DEPTH, bool ROPE, int D>
static hipError_t launch_decode_t(const DecodeParams& p, int num_tiles, int waves,
                                  hipStream_t s) {
  constexpr int rope_lds = ROPE ? RopeLds<D>::BYTES : 0;
  const size_t lds = (size_t)Stage<KV, D>::lds_bytes(waves) + rope_lds;
  // (head_dim 256 with RoPE: at most 4 kv heads per tile fit)
  if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
  // dynamic LDS above 64 KiB must be allowed per kernel (once per process)
  static const hipError_t attr = [] {
    const int max_lds = std::min(Stage<KV, D>::lds_bytes(kWavesPerTile) + rope_lds, kMaxLds);
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, true, FOLD, DEPTH, ROPE, D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, false, FOLD, DEPTH, ROPE, D>),
          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, true, FOLD, DEPTH, ROPE, D>), dim3(num_tiles),
                       dim3(64 * waves), lds, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, false, FOLD, DEPTH, ROPE, D>), dim3(num_tiles),
                       dim3(64 * waves), lds, s, p);
  return hipGetLastError();
}

// The fold instance (cascade suffix tiles, planned as few long 2-head
// tiles) keeps two steps of loads in flight; the plain instance keeps one,
// so that two 8-wave workgroups fit on a compute unit (two steps measured
// no faster for the plain workloads).  head_dim 256 keeps one step in
// flight in both instances (its K/V registers of one step already take 64
// VGPRs) and has no RoPE table.
template <int KV, bool QBF16, int D>
static hipError_t launch_decode_f(const DecodeParams& p, int num_tiles, int waves, bool fold,
                                  hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  if constexpr (D == 256) {
    if (p.rope_table) return launch_decode_t<KV, QBF16, false, 1, true, D>(p, num_tiles, waves, s);
    return fold ? launch_decode_t<KV, QBF16, true, 1, false, D>(p, num_tiles, waves, s)
                : launch_decode_t<KV, QBF16, false, 1, false, D>(p, num_tiles, waves, s);
  } else {
    if (p.rope_table) {
      // (RoPE at head_dim 64: one step in flight measured 8 % faster)
      if constexpr (D == 64)
        return launch_decode_t<KV, QBF16, false, 1, true, D>(p, num_tiles, waves, s);
      else
        return getenv_depth() == 1
                   ? launch_decode_t<KV, QBF16, false, 1, true, D>(p, num_tiles, waves, s)
                   : launch_decode_t<KV, QBF16, false, 2, true, D>(p, num_tiles, waves, s);
    }
    const bool deep = fold && waves <= 4 && getenv_depth() != 1;
    if (fold)
      return deep ? launch_decode_t<KV, QBF16, true, 2, false, D>(p, num_tiles, waves, s)
                  : launch_decode_t<KV, QBF16, true, 1, false, D>(p, num_tiles, waves, s);
    return deep ? launch_decode_t<KV, QBF16, false, 2, false, D>(p, num_tiles, waves, s)
                : launch_decode_t<KV, QBF16, false, 1, false, D>(p, num_tiles, waves, s);
  }
}

template <int KV, bool QBF16, int W, bool APPEND, int D>
static void launch_prefix_w(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, W, true, APPEND, D>), dim3(num_tiles),
                       dim3(64 * W), 0, s, p);
  else
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, W, false, APPEND, D>), dim3(num_tiles),
                       dim3(64 * W), 0, s, p);
}

template <int KV, bool QBF16, int D>
static hipError_t launch_prefix_t(const DecodeParams& p, int num_tiles, int waves, bool append,
                                  hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  if (waves == 4)
    append ? launch_prefix_w<KV, QBF16, 4, true, D>(p, num_tiles, s)
           : launch_prefix_w<KV, QBF16, 4, false, D>(p, num_tiles, s);
  else
    append ? launch_prefix_w<KV, QBF16, 8, true, D>(p, num_tiles, s)
           : launch_prefix_w<KV, QBF16, 8, false, D>(p, num_tiles, s);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams& p, int num_tiles, int waves, bool q_bf16,
                                  int kv, bool fold, hipStream_t s) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_decode_f<kKvE4M3, true, D>(p, num_tiles, waves, fold, s)
                  : launch_decode_f<kKvE4M3, false, D>(p, num_tiles, waves, fold, s);
  return q_bf16 ? launch_decode_f<kKvBF16, true, D>(p, num_tiles, waves, fold, s)
                : launch_decode_f<kKvF16, false, D>(p, num_tiles, waves, fold, s);
}

template <int D>
static hipError_t launch_prefix_d(const DecodeParams& p, int num_tiles, int waves, bool append,
                                  bool q_bf16, int kv, hipStream_t s) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_prefix_t<kKvE4M3, true, D>(p, num_tiles, waves, append, s)
                  : launch_prefix_t<kKvE4M3, false, D>(p, num_tiles, waves, append, s);
  return q_bf16 ? launch_prefix_t<kKvBF16, true, D>(p, num_tiles, waves, append, s)
                : launch_prefix_t<kKvF16, false, D>(p, num_tiles, waves, append, s);
}

// q_bf16: q (and o) are bf16, else fp16.  kv: KvKind.  fold: the work list
// has tiles that fold earlier states into their output.  head_dim: 64, 128
// or 256.
hipError_t launch_decode(const DecodeParams& p, int num_tiles, int waves, bool q_bf16,
                         int kv, bool fold, int head_dim, hipStream_t s) {
  if (waves < 1 || waves > kWavesPerTile) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return launch_decode_d<64>(p, num_tiles, waves, q_bf16, kv, fold, s);
    case 128: return launch_decode_d<128>(p, num_tiles, waves, q_bf16, kv, fold, s);
    case 256: return launch_decode_d<256>(p, num_tiles, waves, q_bf16, kv, fold, s);
    default: return hipErrorInvalidValue;
  }
}

// append: append tiles (rows limited by ReqInfo.kv_len), else cascade
// prefix.  head_dim: 64, 128 or 256.
hipError_t launch_prefix(const DecodeParams& p, int num_tiles, int waves, bool append,
                         bool q_bf16, int kv, int head_dim, hipStream_t s) {
  if (waves != 4 && waves != 8) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return launch_prefix_d<64>(p, num_tiles, waves, append, q_bf16, kv, s);
    case 128: return launch_prefix_d<128>(p, num_tiles, waves, append, q_bf16, kv, s);
    case 256: return launch_prefix_d<256>(p, num_tiles, waves, append, q_bf16, kv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fi
