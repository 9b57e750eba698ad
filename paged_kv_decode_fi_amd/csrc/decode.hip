// decode.hip -- gfx950 paged decode attention kernel (the multi-row kernel of
// cascade prefix and append tiles is in fi_prefix.h, launched from
// prefix.hip and prefix_rope.hip).
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
//  * K/V rows are addressed by page, slot and head strides: NHD or HND
//    pages, or the ragged layout (page size 1, no page table).
//  * head_dim D (64, 128, 256) is a template parameter: D / 32 q operands
//    and D / 16 output blocks per lane.
#include <algorithm>
#include <type_traits>

#include "fi_device.h"

namespace fi {


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
  // K row stride in LDS: a 16-bit K row run padded by 32 bytes (SQ_LDS_BANK_CONFLICT
  // reads 0 for the score operand reads at this stride, 12 % of LDS-active
  // cycles at 16 bytes); e4m3 rows by 16 (32 measured more conflicts there)
  static __host__ __device__ constexpr int k_stride(int W) {
    return W * ROWB + (KV == kKvE4M3 ? 16 : 32);
  }
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
// Turns 8 + 8 partner elements of one key (a: dims f..f+7, b: dims
// f+64..f+71, 16-bit) back by its distance, (cos, sin) of frequencies
// f..f+7 in cs, in fp32; writes the result as a 16-bit high part plus a
// 16-bit residual, so that two MFMAs against the same q carry the rotated
// key to about fp32 accuracy.
template <bool BF16, bool SPLIT>
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
    if constexpr (SPLIT) {
      alo[k] = residual2<BF16>(ahi[k], ra[0], ra[1]);
      blo[k] = residual2<BF16>(bhi[k], rb[0], rb[1]);
    }
  }
}

// Two fp16 pairs (x, y) = (a.lo, b.lo), (a.hi, b.hi) turned back by fp16
// (cos, sin) in packed fp16: x' = x c + f16(y s), y' = y c - f16(x s), each
// a fused multiply-add of a rounded product.  With every request at least
// kRopeSingleKeys long this moves lse by no more than the single-rounded
// fp32 turn does (CPU simulation: 2.7e-4 against 2.4e-4 at 64 keys).
__device__ __forceinline__ void rope_pair_f16(uint32_t a, uint32_t b, uint32_t c, uint32_t s,
                                              uint32_t& ra, uint32_t& rb) {
  const f16x2 x = __builtin_bit_cast(f16x2, a), y = __builtin_bit_cast(f16x2, b);
  const f16x2 cc = __builtin_bit_cast(f16x2, c), ss = __builtin_bit_cast(f16x2, s);
  const f16x2 ys = y * ss, xs = x * ss;
  ra = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(x, cc, ys));
  rb = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(y, cc, -xs));
}

// (cos, sin) table of the plan: one thread per (distance, frequency), angle
// in fp64 from the definition, stored as two fp32 (row d: D/2 pairs), or --
// f16 -- rounded once to fp16, row d = D/2 cosines then D/2 sines.
__global__ void rope_table_kernel(void* table, int rows, int D, double theta, double scale,
                                  int f16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * (D / 2)) return;
  const int d = (int)(i / (D / 2)), f = (int)(i % (D / 2));
  const double ang = (d / scale) * pow(theta, -2.0 * f / D);
  if (f16) {
    _Float16* row = reinterpret_cast<_Float16*>(table) + (int64_t)d * D;
    row[f] = (_Float16)cos(ang);
    row[D / 2 + f] = (_Float16)sin(ang);
  } else {
    reinterpret_cast<float2*>(table)[i] = float2{(float)cos(ang), (float)sin(ang)};
  }
}

hipError_t launch_rope_table(void* table, int rows, int head_dim, float theta, float scale,
                             bool f16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = (int64_t)rows * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     table, rows, head_dim, (double)theta, (double)scale, f16 ? 1 : 0);
  return hipGetLastError();
}

// Packed 16-bit dot product with fp32 accumulation: c + a.lo * b.lo +
// a.hi * b.hi (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
}

// FOLD: the plan has tiles that fold earlier states into their output (a
// separate instance: the fold costs registers the plain kernel keeps free).
// DEPTH: steps of K/V loads in flight per workgroup.  ROPE (1, 2): every key
// is turned by its distance from the query (LLaMA-style RoPE, relative form)
// before the score MFMAs; the LDS after K and V holds the step's 16 rows
// (padded: conflict-free reads of one row per lane) and table rows 0..15.
template <int D>
struct RopeLds {
  static constexpr int FREQ = D / 2;                 // frequencies (table row entries)
  static constexpr int ROW = rope_row_bytes(D);      // table row bytes
  static constexpr int STRIDE = ROW + 16;            // the step's rows in LDS (padded)
  static constexpr int BYTES = kStep * STRIDE + kStep * ROW;
  static constexpr int FPL = (FREQ + 63) / 64;       // frequencies per lane
  // fp16 table (ROPE == 2): a row is D/2 fp16 cosines then D/2 fp16 sines
  // (2 D bytes), copied per step straight from the table into LDS rows
  // padded to 2 D + 32 bytes (conflict-free for the reads of the turn)
  static constexpr int ROW16 = 2 * D;
  static constexpr int STRIDE16 = ROW16 + 32;
  static constexpr int BYTES16 = kStep * STRIDE16;
  static constexpr int VEC16 = kStep * ROW16 / 16;   // 16-byte vectors per step
};
// REC (a test instance): every K vector load also writes its byte offset in
// the K pool to p.rec at ((rec_base[request] + token) * Hkv + kv head) * VR +
// 16-byte chunk -- the page walk exactly as the loads take it.
//
// VG > 0 (the VALU instance, for up to VG q heads per kv head, plain plans):
// no MFMA.  Lane (g, n) takes key n of the step and dims 32 s + 8 g .. +7
// (the same LDS reads as the MFMA path); per q head j it accumulates packed
// 16-bit dot products (v_dot2 with fp32 accumulation) and two cross-lane
// sums give every lane the score of key n.  The softmax keeps the lazy
// running max (the exact step max, over the 16 keys, only when some score
// passes it by more than kLazyMax), and P.V runs as fp32 FMAs: lane i
// accumulates dims D/64 i .. of each head, reading each key's p with
// readlane and its V values from LDS.
//
// QCVT (bf16 q over e4m3 K/V, RoPE plans with the turned key as one value):
// the tile computes in fp16 -- e4m3 K/V convert to fp16 as exactly as to
// bf16, and fp16 carries the turned key and p to 11 bits -- with q read as
// bf16 and scaled into fp16 by a power of two per wave (below); o is
// written as bf16.
template <int KV, bool QBF16, bool PS_POW2, bool FOLD, int DEPTH, int ROPE, int D,
          bool REC = false, int VG = 0, bool QCVT = false>
__global__ __launch_bounds__(64 * kWavesPerTile) void decode_kernel(DecodeParams p) {
  static_assert(!ROPE || !FOLD, "RoPE plans have no cascade level to fold");
  static_assert(VG == 0 || (!ROPE && !FOLD), "the VALU instance serves plain plans");
  static_assert(!QCVT || (!QBF16 && KV == kKvE4M3 && VG == 0 && !FOLD && !REC),
                "the converted-q instance computes in fp16 over e4m3 K/V, plain or RoPE");
  constexpr bool OBF16 = QBF16 || QCVT;   // o's type: q's type in memory
  constexpr int VGX = VG > 0 ? VG : 1;
  constexpr int NV = D / 64;   // VALU instance: output dims per lane
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
  // VALU instance: q head j, dims 32 s + 8 g .. +7 (every lane of group g)
  u32x4 qv[VGX][D / 32];
  if constexpr (VG > 0) {
#pragma unroll
    for (int jj = 0; jj < VG; ++jj) {
      const bool ok = jj < G;
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                             ((int64_t)r * p.Hq + h * G + (ok ? jj : 0)) * D;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
        qv[jj][s] = ok ? v : u32x4{0, 0, 0, 0};
      }
    }
  } else {
    const bool ok = n < G;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)r * p.Hq + h * G + (ok ? n : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
      qop[s] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }
  // QCVT: the wave's bf16 q times 2^qexp, chosen so that its largest
  // magnitude lands in [2^14, 2^15): every bf16 value (8 significant bits)
  // is then an exact fp16 value unless it lies more than 2^28 below that
  // maximum (an fp16 subnormal, off by < 2^-39 of the maximum); qexp is at
  // most 64 (so the score scale stays a normal fp32 number): a wave whose
  // q is all below 2^-49 lands in fp16 subnormals, each off by < 2^-89.
  // The score scale takes the 2^-qexp back exactly
  int qexp = 0;
  if constexpr (QCVT) {
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        mx = fmaxf(mx, fmaxf(fabsf(lo16<true>(qop[s][k])), fabsf(hi16<true>(qop[s][k]))));
    mx = wave_max(mx);
    qexp = __builtin_amdgcn_readfirstlane(
        mx > 0.f ? min(15 - __builtin_amdgcn_frexp_expf(mx), 64) : 0);
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qop[s][k] = pack2<false>(__builtin_ldexpf(lo16<true>(qop[s][k]), qexp),
                                 __builtin_ldexpf(hi16<true>(qop[s][k]), qexp));
  }
  // RoPE: the query sits at position kv_len - 1
  const int qpos = ROPE ? p.req_info[r].kv_len - 1 : 0;
  float c = p.sm_scale_log2;
  if (KV == kKvE4M3 && p.k_scale) c *= p.k_scale[h];
  if constexpr (QCVT) c = __builtin_ldexpf(c, -qexp);

  // cooperative loader: load u of thread tid covers token tk0 + u * TOK_PER_U
  // of the step and 16-byte vector vin of that token's W-head run
  const int tk0 = tid / (S::VR * W);
  const int vin = tid - tk0 * (S::VR * W);
  // vector vin = head vin / VR of the tile's run, 16-byte chunk vin % VR
  const int vh = vin / S::VR, vc = vin - vh * S::VR;
  const int64_t hoff = (int64_t)(h0 + vh) * p.head_stride + 16 * vc;
  const int64_t rec_tok = REC ? p.rec_base[r] : 0;
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
  // fp16 table (ROPE == 2): thread tid < VEC16 copies 16-byte vector tid
  // of the step's 16 rows (row n = distance d0 - n, clamped at 0 for the
  // masked tokens past the tile) from the table to LDS
  struct RopeRow16 {
    u32x4 v;
  };
  RopeRow16 rr16[DEPTH];
  auto issue_rope16 = [&](int step, RopeRow16& rq) {
    if constexpr (ROPE == 2) {
      constexpr int VPR = RL::ROW16 / 16;   // vectors per row
      if (tid < RL::VEC16) {
        const int nn = tid / VPR, vv = tid - nn * VPR;
        const int dist = max(qpos - t0 - kStep * step - nn, 0);
        rq.v = reinterpret_cast<const u32x4*>(p.rope_table)[(int64_t)dist * VPR + vv];
      }
    }
  };
  auto stage_rope16 = [&](const RopeRow16& rq) {
    if constexpr (ROPE == 2) {
      constexpr int VPR = RL::ROW16 / 16;
      if (tid < RL::VEC16) {
        const int nn = tid / VPR, vv = tid - nn * VPR;
        *reinterpret_cast<u32x4*>(rlds + nn * RL::STRIDE16 + 16 * vv) = rq.v;
      }
    }
  };
  auto issue_rope = [&](int step, RopeRow& rq) {
    if constexpr (ROPE == 1) {
#pragma unroll
      for (int k = 0; k < RL::FPL; ++k) {
        const int f = lane + 64 * k;
        if (RL::FREQ % 64 == 0 || f < RL::FREQ)
          rq.v[k] = rtab[(int64_t)(qpos - t0 - kStep * step) * RL::FREQ + f];
      }
    }
  };
  auto stage_rope = [&](const RopeRow& rq) {
    if constexpr (ROPE == 1) {
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
  if constexpr (ROPE == 1) {
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
      if constexpr (REC)
        p.rec[((rec_tok + t) * p.Hkv + h0 + vh) * S::VR + vc] = (int64_t)(off + hoff);
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
  // VALU instance: running max (the same in every lane), this lane's key's
  // share of the sum, and dims NV lane .. of each head's output
  float mv[VGX], lv[VGX], ov[VGX][NV];
#pragma unroll
  for (int jj = 0; jj < VGX; ++jj) {
    mv[jj] = -INFINITY;
    lv[jj] = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) ov[jj][i] = 0.f;
  }
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
        if constexpr (ROPE == 2) {
          // fp16 q: the pairs turned in packed fp16 (product rounded, then
          // the fused add) against fp16 (cos, sin), the key rounded once
          const uint8_t* row = rlds + n * RL::STRIDE16 + 2 * (32 * j + 8 * g);
          const u32x4 c8 = *reinterpret_cast<const u32x4*>(row);
          const u32x4 s8 = *reinterpret_cast<const u32x4*>(row + 2 * RL::FREQ);
          const u32x4 a = kop_of(j), b = kop_of(j + HALF);
          u32x4 ra, rb;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t x, y;
            rope_pair_f16(a[k], b[k], c8[k], s8[k], x, y);
            ra[k] = x;
            rb[k] = y;
          }
          sc = mma16x16x32<QBF16>(ra, qop[j], sc);
          sc = mma16x16x32<QBF16>(rb, qop[j + HALF], sc);
        } else {
          const float4* cs =
              reinterpret_cast<const float4*>(rlds + n * RL::STRIDE + 256 * j + 64 * g);
          u32x4 ahi, alo, bhi, blo;
          rope_key8<QBF16, true>(kop_of(j), kop_of(j + HALF), cs, ahi, alo, bhi, blo);
          sc = mma16x16x32<QBF16>(ahi, qop[j], sc);
          sc = mma16x16x32<QBF16>(alo, qop[j], sc);
          sc = mma16x16x32<QBF16>(bhi, qop[j + HALF], sc);
          sc = mma16x16x32<QBF16>(blo, qop[j + HALF], sc);
        }
      }
    } else if constexpr (VG > 0) {
      // ---- VALU instance: scores, softmax and P.V without MFMA
      float acc[VG];
#pragma unroll
      for (int jj = 0; jj < VG; ++jj) acc[jj] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const u32x4 k = kop_of(s);
#pragma unroll
        for (int jj = 0; jj < VG; ++jj)
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[jj] = dot2<QBF16>(k[w], qv[jj][s][w], acc[jj]);
      }
      const bool valid = tb + n < t1;
      float pv[VG];
#pragma unroll
      for (int jj = 0; jj < VG; ++jj) {
        acc[jj] += __shfl_xor(acc[jj], 16);
        acc[jj] += __shfl_xor(acc[jj], 32);
        const float xj = valid ? acc[jj] * c : -INFINITY;
        if (__any(xj > mv[jj] + kLazyMax)) {
          float mx = xj;
#pragma unroll
          for (int o2 = 1; o2 < 16; o2 <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
          const float alpha = fast_exp2(mv[jj] - mx);   // mv = -inf first: 0
          lv[jj] *= alpha;
#pragma unroll
          for (int i = 0; i < NV; ++i) ov[jj][i] *= alpha;
          mv[jj] = mx;
        }
        pv[jj] = fast_exp2(xj - mv[jj]);
        lv[jj] += pv[jj];
      }
      // P.V: key t's p sits in lane t; V row t of this wave's head in LDS
      const uint8_t* vrow = vlds + wave * (2 * D) + 2 * NV * lane;
#pragma unroll
      for (int t = 0; t < kStep; ++t) {
        float v[NV];
        if constexpr (NV == 1) {
          v[0] = lo16<QBF16>(*reinterpret_cast<const uint16_t*>(vrow + t * VS));
        } else if constexpr (NV == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(vrow + t * VS);
          v[0] = lo16<QBF16>(w);
          v[1] = hi16<QBF16>(w);
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(vrow + t * VS);
          v[0] = lo16<QBF16>(w.x);
          v[1] = hi16<QBF16>(w.x);
          v[2] = lo16<QBF16>(w.y);
          v[3] = hi16<QBF16>(w.y);
        }
#pragma unroll
        for (int jj = 0; jj < VG; ++jj) {
          const float pt = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv[jj]), t));
#pragma unroll
          for (int i = 0; i < NV; ++i) ov[jj][i] = __builtin_fmaf(pt, v[i], ov[jj][i]);
        }
      }
      return;
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
      issue_rope16(0, rr16[0]);
      for (int step = 0; step < nsteps; ++step) {
        const int pg2 = step + 2 < nsteps ? load_page(step + 2) : 0;
        stage(kr[0], vr[0]);
        stage_rope(rr[0]);
        stage_rope16(rr16[0]);
        __syncthreads();
        if (step + 1 < nsteps) {
          issue(step + 1, pg1, kr[0], vr[0]);
          issue_rope(step + 1, rr[0]);
          issue_rope16(step + 1, rr16[0]);
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
      issue_rope16(0, rr16[0]);
      if (nsteps > 1) {
        issue(1, load_page(1), kr[1], vr[1]);
        issue_rope(1, rr[DEPTH - 1]);
        issue_rope16(1, rr16[DEPTH - 1]);
      }
      int pga = nsteps > 2 ? load_page(2) : 0;   // page of the next even step to issue
      int pgb = nsteps > 3 ? load_page(3) : 0;   // ... odd step
      // one body per register set: set d stages step s and refills with s + 2
      auto body = [&](int step, int& pgn, u32x4 (&kq)[S::LOADS], u32x4 (&vq)[S::LOADS],
                      RopeRow& rq, RopeRow16& rq16) {
        stage(kq, vq);
        stage_rope(rq);
        stage_rope16(rq16);
        __syncthreads();
        if (step + 2 < nsteps) {
          issue(step + 2, pgn, kq, vq);
          issue_rope(step + 2, rq);
          issue_rope16(step + 2, rq16);
        }
        pgn = step + 4 < nsteps ? load_page(step + 4) : 0;
        compute(step);
        __syncthreads();
      };
      for (int step = 0; step < nsteps; step += 2) {
        body(step, pga, kr[0], vr[0], rr[0], rr16[0]);
        if (step + 1 < nsteps) body(step + 1, pgb, kr[1], vr[1], rr[DEPTH - 1], rr16[DEPTH - 1]);
      }
    }
  }

  // ---- finalize
  const float vs = (KV == kKvE4M3 && p.v_scale) ? p.v_scale[h] : 1.f;
  if constexpr (VG > 0) {
    // VALU instance: head j's sum over the 16 keys of the lane group, then
    // dims NV lane .. of its output (final, or an fp32 partial state)
#pragma unroll
    for (int jj = 0; jj < VG; ++jj) {
      if (jj >= G) break;
      float lt = lv[jj];
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) lt += __shfl_xor(lt, o2);
      const float inv = (lt > 0.f ? 1.f / lt : 0.f) * vs;
      const float lse2 = lt > 0.f ? mv[jj] + fast_log2(lt) : -INFINITY;
      const int jq = h * G + jj;
      if (tile.slot < 0) {
        uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)r * p.Hq + jq) * D;
        if constexpr (NV == 1) {
          orow[lane] = (uint16_t)(pack2<QBF16>(ov[jj][0] * inv, 0.f) & 0xffffu);
        } else if constexpr (NV == 2) {
          reinterpret_cast<uint32_t*>(orow)[lane] = pack2<QBF16>(ov[jj][0] * inv, ov[jj][1] * inv);
        } else {
          reinterpret_cast<u32x2*>(orow)[lane] =
              u32x2{pack2<QBF16>(ov[jj][0] * inv, ov[jj][1] * inv),
                    pack2<QBF16>(ov[jj][2] * inv, ov[jj][3] * inv)};
        }
        if (lane == 0 && p.lse) p.lse[(int64_t)r * p.Hq + jq] = lse2 * kLn2;
      } else {
        const int64_t slot = tile.slot + wave;
        float* po = p.partial_o + (slot * G + jj) * D + NV * lane;
#pragma unroll
        for (int i = 0; i < NV; ++i) po[i] = ov[jj][i] * inv;
        if (lane == 0) p.partial_lse[slot * G + jj] = lse2;
      }
    }
    return;
  }
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
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
        u32x2 w = {pack2<OBF16>(oacc[b][0] * inv, oacc[b][1] * inv),
                   pack2<OBF16>(oacc[b][2] * inv, oacc[b][3] * inv)};
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

// ---- launchers ----------------------------------------------------------------
// depth (from the plan's tuning): 0 = each instance's own choice below, 1 =
// one step of loads in flight everywhere, 2 = two where the instance has a
// two-step form.

constexpr int kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950

// occ != NULL: nothing is launched; *occ receives the workgroups of this
// instance that one compute unit holds at once (the same kernel, block size
// and dynamic LDS as the launch).
template <int KV, bool QBF16, bool FOLD, int DEPTH, int ROPE, int D, bool QCVT = false>
static hipError_t launch_decode_t(const DecodeParams& p, int num_tiles, int waves,
                                  hipStream_t s, int* occ = nullptr) {
  constexpr int rope_lds = ROPE == 2 ? RopeLds<D>::BYTES16 : ROPE ? RopeLds<D>::BYTES : 0;
  const size_t lds = (size_t)Stage<KV, D>::lds_bytes(waves) + rope_lds;
  // (head_dim 256 with RoPE: at most 4 kv heads per tile fit)
  if (lds > (size_t)kMaxLds) return hipErrorInvalidValue;
  // dynamic LDS above 64 KiB must be allowed per kernel (once per process)
  static const hipError_t attr = [] {
    const int max_lds = std::min(Stage<KV, D>::lds_bytes(kWavesPerTile) + rope_lds, kMaxLds);
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, true, FOLD, DEPTH, ROPE, D, false, 0, QCVT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, false, FOLD, DEPTH, ROPE, D, false, 0, QCVT>),
          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (occ)
    return p.ps_shift >= 0
               ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                     occ, decode_kernel<KV, QBF16, true, FOLD, DEPTH, ROPE, D, false, 0, QCVT>, 64 * waves, lds)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                     occ, decode_kernel<KV, QBF16, false, FOLD, DEPTH, ROPE, D, false, 0, QCVT>, 64 * waves, lds);
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, true, FOLD, DEPTH, ROPE, D, false, 0, QCVT>), dim3(num_tiles),
                       dim3(64 * waves), lds, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, false, FOLD, DEPTH, ROPE, D, false, 0, QCVT>), dim3(num_tiles),
                       dim3(64 * waves), lds, s, p);
  return hipGetLastError();
}

// The fold instance (cascade suffix tiles, planned as few long 2-head
// tiles) keeps two steps of loads in flight; the plain instance keeps one,
// so that two 8-wave workgroups fit on a compute unit (two steps measured
// no faster for the plain workloads).  head_dim 256 keeps one step in
// flight in both instances (its K/V registers of one step already take 64
// VGPRs) and has no RoPE table.
// RoPE plans: two steps of loads in flight at head_dim 128 unless the plan
// forces one; one step at head_dim 64 (measured 8 % faster) and 256
// (registers).
template <int KV, bool QBF16, int ROPE, int D, bool QCVT = false>
static hipError_t launch_decode_rope(const DecodeParams& p, int num_tiles, int waves, int depth,
                                     hipStream_t s, int* occ) {
  if constexpr (D == 128) {
    if (depth != 1)
      return launch_decode_t<KV, QBF16, false, 2, ROPE, D, QCVT>(p, num_tiles, waves, s, occ);
  }
  return launch_decode_t<KV, QBF16, false, 1, ROPE, D, QCVT>(p, num_tiles, waves, s, occ);
}

// VALU instances (plain plans, head_dim 128, one step of loads in flight):
// vg = 1, 2 or 4 q heads per kv head at most.
template <int KV, bool QBF16, int VG>
static hipError_t launch_decode_valu_t(const DecodeParams& p, int num_tiles, int waves,
                                       hipStream_t s, int* occ) {
  const size_t lds = (size_t)Stage<KV, 128>::lds_bytes(waves);
  static const hipError_t attr = [] {
    const int max_lds = Stage<KV, 128>::lds_bytes(kWavesPerTile);
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, true, false, 1, 0, 128, false, VG>),
        hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(
              &decode_kernel<KV, QBF16, false, false, 1, 0, 128, false, VG>),
          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (occ)
    return p.ps_shift >= 0
               ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                     occ, decode_kernel<KV, QBF16, true, false, 1, 0, 128, false, VG>,
                     64 * waves, lds)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                     occ, decode_kernel<KV, QBF16, false, false, 1, 0, 128, false, VG>,
                     64 * waves, lds);
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, true, false, 1, 0, 128, false, VG>),
                       dim3(num_tiles), dim3(64 * waves), lds, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, false, false, 1, 0, 128, false, VG>),
                       dim3(num_tiles), dim3(64 * waves), lds, s, p);
  return hipGetLastError();
}

template <int KV, bool QBF16>
static hipError_t launch_decode_valu(const DecodeParams& p, int num_tiles, int waves,
                                     hipStream_t s, int* occ) {
  switch (p.valu_heads) {
    case 1: return launch_decode_valu_t<KV, QBF16, 1>(p, num_tiles, waves, s, occ);
    case 2: return launch_decode_valu_t<KV, QBF16, 2>(p, num_tiles, waves, s, occ);
    case 4: return launch_decode_valu_t<KV, QBF16, 4>(p, num_tiles, waves, s, occ);
    default: return hipErrorInvalidValue;
  }
}

template <int KV, bool QBF16, int D>
static hipError_t launch_decode_f(const DecodeParams& p, int num_tiles, int waves, bool fold,
                                  int depth, hipStream_t s, int* occ) {
  if (num_tiles <= 0 && !occ) return hipSuccess;
  if (p.valu_heads > 0) {
    if constexpr (D == 128) {
      if (!fold && !p.rope_table)
        return launch_decode_valu<KV, QBF16>(p, num_tiles, waves, s, occ);
    }
    return hipErrorInvalidValue;
  }
  if (p.rope_table) {
    // the rotated key as one fp16 value (fp16 q; bf16 q over e4m3 K/V on
    // the converted-q fp16 instance) or a high part plus a residual
    if constexpr (!QBF16) {
      if (p.rope_single)
        return launch_decode_rope<KV, QBF16, 2, D>(p, num_tiles, waves, depth, s, occ);
    } else if constexpr (KV == kKvE4M3) {
      if (p.rope_single)
        return launch_decode_rope<KV, false, 2, D, true>(p, num_tiles, waves, depth, s, occ);
    }
    return launch_decode_rope<KV, QBF16, 1, D>(p, num_tiles, waves, depth, s, occ);
  }
  if constexpr (D == 256) {
    return fold ? launch_decode_t<KV, QBF16, true, 1, 0, D>(p, num_tiles, waves, s, occ)
                : launch_decode_t<KV, QBF16, false, 1, 0, D>(p, num_tiles, waves, s, occ);
  } else {
    const bool deep = depth == 2 || (depth == 0 && fold && waves <= 4);
    if (fold)
      return deep ? launch_decode_t<KV, QBF16, true, 2, 0, D>(p, num_tiles, waves, s, occ)
                  : launch_decode_t<KV, QBF16, true, 1, 0, D>(p, num_tiles, waves, s, occ);
    return deep ? launch_decode_t<KV, QBF16, false, 2, 0, D>(p, num_tiles, waves, s, occ)
                : launch_decode_t<KV, QBF16, false, 1, 0, D>(p, num_tiles, waves, s, occ);
  }
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams& p, int num_tiles, int waves, bool q_bf16,
                                  int kv, bool fold, int depth, hipStream_t s, int* occ) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_decode_f<kKvE4M3, true, D>(p, num_tiles, waves, fold, depth, s, occ)
                  : launch_decode_f<kKvE4M3, false, D>(p, num_tiles, waves, fold, depth, s, occ);
  return q_bf16 ? launch_decode_f<kKvBF16, true, D>(p, num_tiles, waves, fold, depth, s, occ)
                : launch_decode_f<kKvF16, false, D>(p, num_tiles, waves, fold, depth, s, occ);
}

// ---- record instances (test hook): head_dim 128, fp16 q + fp16 K/V or bf16
// q + e4m3 K/V; the loop shapes of one and two steps in flight (fp16), no
// fold and no RoPE (neither changes the loads' addresses)
template <int KV, bool QBF16, int DEPTH>
static hipError_t launch_decode_rec_t(const DecodeParams& p, int num_tiles, int waves,
                                      hipStream_t s) {
  const size_t lds = (size_t)Stage<KV, 128>::lds_bytes(waves);
  static const hipError_t attr = [] {
    const int max_lds = Stage<KV, 128>::lds_bytes(kWavesPerTile);
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<KV, QBF16, true, false, DEPTH, 0, 128, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(
              &decode_kernel<KV, QBF16, false, false, DEPTH, 0, 128, true>),
          hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, true, false, DEPTH, 0, 128, true>),
                       dim3(num_tiles), dim3(64 * waves), lds, s, p);
  else
    hipLaunchKernelGGL((decode_kernel<KV, QBF16, false, false, DEPTH, 0, 128, true>),
                       dim3(num_tiles), dim3(64 * waves), lds, s, p);
  return hipGetLastError();
}

static hipError_t launch_decode_rec(const DecodeParams& p, int num_tiles, int waves,
                                    bool q_bf16, int kv, int depth, int head_dim,
                                    hipStream_t s) {
  if (head_dim != 128 || p.rope_table) return hipErrorInvalidValue;
  if (kv == kKvF16 && !q_bf16)
    return depth == 2 ? launch_decode_rec_t<kKvF16, false, 2>(p, num_tiles, waves, s)
                      : launch_decode_rec_t<kKvF16, false, 1>(p, num_tiles, waves, s);
  if (kv == kKvE4M3 && q_bf16 && depth != 2)
    return launch_decode_rec_t<kKvE4M3, true, 1>(p, num_tiles, waves, s);
  return hipErrorInvalidValue;
}

// q_bf16: q (and o) are bf16, else fp16.  kv: KvKind.  fold: the work list
// has tiles that fold earlier states into their output.  depth: 0, 1 or 2
// (above).  head_dim: 64, 128 or 256.  p.rec != NULL selects the record
// instances (hipErrorInvalidValue for a configuration they do not cover).
hipError_t launch_decode(const DecodeParams& p, int num_tiles, int waves, bool q_bf16,
                         int kv, bool fold, int depth, int head_dim, hipStream_t s) {
  if (waves < 1 || waves > kWavesPerTile) return hipErrorInvalidValue;
  if (p.rec) {
    if (num_tiles <= 0) return hipSuccess;
    return launch_decode_rec(p, num_tiles, waves, q_bf16, kv,
                             depth ? depth : (fold && waves <= 4 ? 2 : 1), head_dim, s);
  }
  switch (head_dim) {
    case 64: return launch_decode_d<64>(p, num_tiles, waves, q_bf16, kv, fold, depth, s, nullptr);
    case 128: return launch_decode_d<128>(p, num_tiles, waves, q_bf16, kv, fold, depth, s, nullptr);
    case 256: return launch_decode_d<256>(p, num_tiles, waves, q_bf16, kv, fold, depth, s, nullptr);
    default: return hipErrorInvalidValue;
  }
}

// Workgroups of `waves` waves per compute unit that the instance
// launch_decode picks for the same arguments holds at once (its registers,
// LDS and block size, as the device reports them); nothing is launched.
hipError_t decode_occupancy(const DecodeParams& p, int waves, bool q_bf16, int kv, bool fold,
                            int depth, int head_dim, int* blocks) {
  *blocks = 0;
  if (waves < 1 || waves > kWavesPerTile) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return launch_decode_d<64>(p, 0, waves, q_bf16, kv, fold, depth, nullptr, blocks);
    case 128: return launch_decode_d<128>(p, 0, waves, q_bf16, kv, fold, depth, nullptr, blocks);
    case 256: return launch_decode_d<256>(p, 0, waves, q_bf16, kv, fold, depth, nullptr, blocks);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fi
