// fi_device.h -- gfx950 device primitives shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fi_internal.h"

namespace fi {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum KvKind { kKvF16 = 0, kKvBF16 = 1, kKvE4M3 = 2 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- MFMA 16x16x32 (fp32 accumulate) ----------------------------------------
// Operand layout (64 lanes, lane = 16 * g + n, g in 0..3, n in 0..15):
//   A (16 x 32): lane holds A[n][8g .. 8g+7]
//   B (32 x 16): lane holds B[8g .. 8g+7][n]
//   D (16 x 16): lane holds D[4g .. 4g+3][n]
template <bool BF16>
__device__ __forceinline__ f32x4 mma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---- page walk ----------------------------------------------------------------
// Physical token slot (page * page_size + slot) of logical token t of the
// table row starting at kv_indices[page_base].  ps_shift = log2(page_size)
// when page_size is a power of two, else -1.
__device__ __forceinline__ int64_t page_slot(const int32_t* __restrict__ kv_indices,
                                             int page_base, int t, int page_size,
                                             int ps_shift) {
  int pi, sl;
  if (ps_shift >= 0) {
    pi = t >> ps_shift;
    sl = t & (page_size - 1);
  } else {
    pi = t / page_size;
    sl = t - pi * page_size;
  }
  const int64_t page = kv_indices[page_base + pi];
  return page * page_size + sl;
}

// ---- conversions ----------------------------------------------------------------
// Two fp32 -> two packed 16-bit floats (round to nearest even), one packed
// convert instruction on gfx950.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Four OCP e4m3fn codes (one dword) -> four 16-bit floats (two dwords), exact.
// gfx950's scaled converts take the OCP encoding; scale 1.0 keeps the value.
template <bool BF16>
__device__ __forceinline__ u32x2 e4m3x4_to_16(uint32_t w) {
  u32x2 r;
  if constexpr (BF16) {
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  } else {
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  return r;
}

// gfx950 transpose read of 16-bit LDS data (ds_read_b64_tr_b16), used for
// the V^T operand of P.V.  It works per 16-lane group: lane i's element k is
// element i % 4 of the 4 x 16-bit row addressed by lane i / 4 + 4 k of its
// group (layout measured with a probe).  So a lane that addresses the d-quad
// n % 4 of the row holding contraction element kk = n / 4 receives, over its
// four elements, that d column for four consecutive contraction elements.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ T ld_global(const void* base, int64_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Streaming load: data read exactly once (K/V rows), marked non-temporal so
// it does not displace reusable lines; measurably closer to the HBM read
// ceiling on MI355X than default-policy loads.
template <typename T>
__device__ __forceinline__ T ld_stream(const void* base, int64_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Merge of n attention states over disjoint key sets for one query row,
// by one wave (D / 64 dims per lane).  State c lives at row row0 + c * stride
// of partial_o [.][D] / partial_lse [.] (lse in log2 units):
//   M = max_c s_c, S = sum_c 2^(s_c - M), o = sum_c 2^(s_c - M) o_c / S,
//   lse = (M + log2 S) ln 2; all states empty -> o = 0, lse = -inf.
// Lanes read 64 lse values at a time; partial rows are read BATCH at a time
// (half of it at head_dim 256, for registers) with independent loads issued
// together (BATCH 64 for rows with many states).  The first batch of partial
// rows is issued before the lse pass: its addresses do not depend on the lse
// values, so both are one round trip.
template <int NV> struct LaneVec;
template <> struct LaneVec<1> { using T = float; };
template <> struct LaneVec<2> { using T = f32x2; };
template <> struct LaneVec<4> { using T = f32x4; };

template <bool OBF16, int BATCH, int D>
__device__ __forceinline__ void merge_state_row(const float* __restrict__ partial_o,
                                                const float* __restrict__ partial_lse,
                                                int64_t row0, int64_t stride, int n,
                                                uint16_t* orow, float* lse_out, int lane) {
  constexpr int NV = D / 64;                          // dims per lane
  constexpr int EB = NV == 4 ? BATCH / 2 : BATCH;     // rows per batch
  using V = typename LaneVec<NV>::T;
  auto elem = [](const V& x, int i) -> float {
    if constexpr (NV == 1) return x;
    else return x[i];
  };
  const float* po = partial_o + row0 * D + NV * lane;
  auto load_rows = [&](int c, int cnt, V (&v)[EB]) {
#pragma unroll
    for (int k = 0; k < EB; ++k)
      v[k] = k < cnt ? *reinterpret_cast<const V*>(po + (int64_t)(c + k) * stride * D) : V{};
  };
  V v[EB];
  load_rows(0, min(n, EB), v);
  const float s0 = lane < n ? partial_lse[row0 + lane * stride] : -INFINITY;
  float M = s0;
  for (int c0 = 64; c0 < n; c0 += 64) {
    const int c = c0 + lane;
    M = fmaxf(M, c < n ? partial_lse[row0 + c * stride] : -INFINITY);
  }
  M = wave_max(M);
  float a[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) a[i] = 0.f;
  float S = 0.f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int c = c0 + lane;
      const float sc = c0 == 0 ? s0 : (c < n ? partial_lse[row0 + c * stride] : -INFINITY);
      const float w = c < n ? fast_exp2(sc - M) : 0.f;
      S += w;
      const int cn = min(64, n - c0);
      for (int k0 = 0; k0 < cn; k0 += EB) {
        if (c0 + k0 > 0) load_rows(c0 + k0, min(EB, cn - k0), v);
#pragma unroll
        for (int k = 0; k < EB; ++k) {
          // uniform lane index: a scalar read of lane k0 + k's weight
          const float wk = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (k0 + k) & 63));
#pragma unroll
          for (int i = 0; i < NV; ++i) a[i] += wk * elem(v[k], i);
        }
      }
    }
    S = wave_sum(S);
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  if constexpr (NV == 1) {
    orow[lane] = (uint16_t)(pack2<OBF16>(a[0] * inv, 0.f) & 0xffffu);
  } else if constexpr (NV == 2) {
    reinterpret_cast<uint32_t*>(orow)[lane] = pack2<OBF16>(a[0] * inv, a[1] * inv);
  } else {
    reinterpret_cast<u32x2*>(orow)[lane] =
        u32x2{pack2<OBF16>(a[0] * inv, a[1] * inv), pack2<OBF16>(a[2] * inv, a[3] * inv)};
  }
  if (lane == 0 && lse_out) *lse_out = S > 0.f ? (M + fast_log2(S)) * kLn2 : -INFINITY;
}

}  // namespace fi
