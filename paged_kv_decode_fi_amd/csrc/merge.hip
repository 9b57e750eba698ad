// merge.hip -- recombination of attention states over disjoint key sets.
//
// Splitting one request's keys over several workgroups (the load-balanced
// plan of the FlashInfer README, "core features" item 2) and cascade
// attention (item 3: shared prefix + own suffix) both need the union of
// attention states: with s_i the log-sum-exp of key set i and v_i its
// softmax-weighted value,
//     s = M + ln sum_i exp(s_i - M),   M = max_i s_i,
//     v = sum_i exp(s_i - s) v_i,
// and an all-empty union gives v = 0, s = -inf.  Internal partial states
// carry s in log2 units (the decode kernel's exp2 domain).
#include "fi_device.h"

namespace fi {

// One wave per (merged request, q head); the arithmetic is merge_state_row.
template <bool OBF16, int D>
__global__ __launch_bounds__(256) void merge_partials_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (j >= p.Hq) return;
  const MergeUnit u = p.units[blockIdx.x];
  const int h = j / p.G, jj = j - h * p.G;
  const int64_t stride = (int64_t)p.Hkv * p.G;                  // rows between states
  const int64_t row0 = ((int64_t)u.slot_base + h) * p.G + jj;   // state 0's row
  uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + ((int64_t)u.req * p.Hq + j) * D;
  float* lse_out = p.lse ? p.lse + (int64_t)u.req * p.Hq + j : nullptr;
  if (u.n_states > 16)
    merge_state_row<OBF16, 64, D>(p.partial_o, p.partial_lse, row0, stride, u.n_states, orow,
                                  lse_out, lane);
  else
    merge_state_row<OBF16, 16, D>(p.partial_o, p.partial_lse, row0, stride, u.n_states, orow,
                                  lse_out, lane);
}

// Many units with few states each (append plans: one unit per query
// token): one workgroup per (unit,
// 256 / (D / 16) q heads), D / 16 threads per head with 16 dims each, every
// state's rows loaded by all threads at once.  One wave per (unit, head)
// would spend most of its short life waiting on two dependent round trips.
template <bool OBF16, int D>
__global__ __launch_bounds__(256) void merge_units_wide_kernel(MergeParams p) {
  constexpr int TPH = D / 16;   // threads per head
  const int t = threadIdx.x;
  const int j = blockIdx.y * (256 / TPH) + t / TPH;
  if (j >= p.Hq) return;
  const int d0 = 16 * (t % TPH);
  const MergeUnit u = p.units[blockIdx.x];
  const int h = j / p.G, jj = j - h * p.G;
  const int64_t stride = (int64_t)p.Hkv * p.G;                  // rows between states
  const int64_t row0 = ((int64_t)u.slot_base + h) * p.G + jj;   // state 0's row
  const int n = u.n_states;
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, p.partial_lse[row0 + c * stride]);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float S = 0.f;
  if (M != -INFINITY) {
#pragma unroll 4
    for (int c = 0; c < n; ++c) {
      const float w = fast_exp2(p.partial_lse[row0 + c * stride] - M);
      S += w;
      const f32x4* src =
          reinterpret_cast<const f32x4*>(p.partial_o + (row0 + c * stride) * D + d0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v = src[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[4 * k + i] += w * v[i];
      }
    }
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.o) +
                                        ((int64_t)u.req * p.Hq + j) * D + d0);
#pragma unroll
  for (int k = 0; k < 2; ++k)
    dst[k] = u32x4{pack2<OBF16>(acc[8 * k] * inv, acc[8 * k + 1] * inv),
                   pack2<OBF16>(acc[8 * k + 2] * inv, acc[8 * k + 3] * inv),
                   pack2<OBF16>(acc[8 * k + 4] * inv, acc[8 * k + 5] * inv),
                   pack2<OBF16>(acc[8 * k + 6] * inv, acc[8 * k + 7] * inv)};
  if (t % TPH == 0 && p.lse)
    p.lse[(int64_t)u.req * p.Hq + j] = S > 0.f ? (M + fast_log2(S)) * kLn2 : -INFINITY;
}

template <int D>
static void launch_merge_d(const MergeParams& p, int num_units, bool o_bf16, bool wide,
                           hipStream_t s) {
  if (wide) {
    constexpr int HPB = 256 / (D / 16);   // heads per workgroup
    dim3 grid(num_units, (p.Hq + HPB - 1) / HPB);
    if (o_bf16)
      hipLaunchKernelGGL((merge_units_wide_kernel<true, D>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((merge_units_wide_kernel<false, D>), grid, dim3(256), 0, s, p);
    return;
  }
  dim3 grid(num_units, (p.Hq + 3) / 4);
  if (o_bf16)
    hipLaunchKernelGGL((merge_partials_kernel<true, D>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((merge_partials_kernel<false, D>), grid, dim3(256), 0, s, p);
}

// wide: the workgroup-per-unit kernel (many units, few states each), else
// one wave per (unit, q head).
hipError_t launch_merge_partials(const MergeParams& p, int num_units, bool o_bf16, bool wide,
                                 int head_dim, hipStream_t s) {
  if (num_units <= 0) return hipSuccess;
  switch (head_dim) {
    case 64: launch_merge_d<64>(p, num_units, o_bf16, wide, s); break;
    case 128: launch_merge_d<128>(p, num_units, o_bf16, wide, s); break;
    case 256: launch_merge_d<256>(p, num_units, o_bf16, wide, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- public K-way merge: one wave per row, natural-log lse ----------------
__device__ __forceinline__ float load_val(const void* base, int dt, int64_t i) {
  if (dt == 3) return reinterpret_cast<const float*>(base)[i];
  const uint16_t u = reinterpret_cast<const uint16_t*>(base)[i];
  if (dt == 1) return __builtin_bit_cast(float, (uint32_t)u << 16);
  return (float)__builtin_bit_cast(_Float16, u);
}

__device__ __forceinline__ void store_val(void* base, int dt, int64_t i, float v) {
  if (dt == 3) {
    reinterpret_cast<float*>(base)[i] = v;
  } else if (dt == 1) {
    __bf16 b = (__bf16)v;
    reinterpret_cast<uint16_t*>(base)[i] = __builtin_bit_cast(uint16_t, b);
  } else {
    _Float16 hv = (_Float16)v;
    reinterpret_cast<uint16_t*>(base)[i] = __builtin_bit_cast(uint16_t, hv);
  }
}

__global__ __launch_bounds__(256) void merge_states_kernel(MergeStatesParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.num_rows) return;
  float M = -INFINITY;
  for (int i = 0; i < p.num_states; ++i) M = fmaxf(M, p.s[i][row]);
  float S = 0.f;
  if (M != -INFINITY)
    for (int i = 0; i < p.num_states; ++i) S += __expf(p.s[i][row] - M);
  const float lse = S > 0.f ? M + __logf(S) : -INFINITY;
  for (int d = lane; d < p.head_dim; d += 64) {
    float acc = 0.f;
    if (S > 0.f)
      for (int i = 0; i < p.num_states; ++i)
        acc += __expf(p.s[i][row] - lse) *
               load_val(p.v[i], p.v_dtype, row * p.head_dim + d);
    store_val(p.v_out, p.out_dtype, row * p.head_dim + d, acc);
  }
  if (lane == 0 && p.s_out) p.s_out[row] = lse;
}

hipError_t launch_merge_states(const MergeStatesParams& p, hipStream_t s) {
  if (p.num_rows <= 0) return hipSuccess;
  const int64_t blocks = (p.num_rows + 3) / 4;
  hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---- test hook: the decode kernel's page walk, token by token --------------
__global__ void gather_kernel(const int32_t* kv_indptr, const int32_t* kv_indices,
                              const int64_t* token_indptr, int page_size, int ps_shift,
                              int64_t* out) {
  const int r = blockIdx.x;
  const int page_base = kv_indptr[r];
  const int64_t t_begin = token_indptr[r], L = token_indptr[r + 1] - t_begin;
  for (int64_t t = threadIdx.x; t < L; t += blockDim.x)
    out[t_begin + t] = page_slot(kv_indices, page_base, (int)t, page_size, ps_shift);
}

hipError_t launch_gather(const int32_t* kv_indptr, const int32_t* kv_indices,
                         const int64_t* token_indptr, int batch, int page_size,
                         int ps_shift, int64_t* out, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(batch), dim3(256), 0, s, kv_indptr, kv_indices,
                     token_indptr, page_size, ps_shift, out);
  return hipGetLastError();
}

// ---- test hook: plain streaming read of a buffer (bandwidth ceiling and
// counter calibration).  Each workgroup reads contiguous 64 KiB chunks with
// 16-byte non-temporal loads (the fastest plain-read pattern measured on
// MI355X) and folds them into one word per thread so the loads stay live.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          int64_t n16, uint32_t* sink) {
  constexpr int64_t kChunk = 4096;  // 16-byte vectors per workgroup step
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * kChunk; base < n16;
       base += (int64_t)gridDim.x * kChunk) {
    u32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t k = base + u * 256 + threadIdx.x;
      v[u] = k < n16 ? __builtin_nontemporal_load(src + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                              hipStream_t s) {
  if (bytes < 16 || blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s,
                     reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace fi
