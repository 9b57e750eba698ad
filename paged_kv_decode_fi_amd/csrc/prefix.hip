// prefix.hip -- launchers of the multi-row kernel (fi_prefix.h): cascade
// prefix tiles and batch-append tiles without RoPE, and the record
// instances of the page-walk test hook.  The RoPE instances are built in
// prefix_rope.hip (a separate translation unit, compiled in parallel).
#include <type_traits>

#include "fi_prefix.h"

namespace fi {

template <int KV, bool QBF16, int W, int MODE, int D>
static void launch_prefix_w(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, W, true, MODE, D>), dim3(num_tiles),
                       dim3(64 * W), 0, s, p);
  else
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, W, false, MODE, D>), dim3(num_tiles),
                       dim3(64 * W), 0, s, p);
}

template <int KV, bool QBF16, int W, int D>
static void launch_prefix_m(const DecodeParams& p, int num_tiles, bool append, bool split,
                            hipStream_t s) {
  if (append) {
    launch_prefix_w<KV, QBF16, W, kPrefixAppend, D>(p, num_tiles, s);
    return;
  }
  if constexpr (KV == kKvBF16) {   // the split instance exists for bf16 K/V only
    if (split) {
      launch_prefix_w<KV, QBF16, W, kPrefixSplitP, D>(p, num_tiles, s);
      return;
    }
  }
  launch_prefix_w<KV, QBF16, W, kPrefixPlain, D>(p, num_tiles, s);
}

template <int KV, bool QBF16, int D>
static hipError_t launch_prefix_t(const DecodeParams& p, int num_tiles, int waves, bool append,
                                  bool split, hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  if (waves == 4)
    launch_prefix_m<KV, QBF16, 4, D>(p, num_tiles, append, split, s);
  else
    launch_prefix_m<KV, QBF16, 8, D>(p, num_tiles, append, split, s);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefix_d(const DecodeParams& p, int num_tiles, int waves, bool append,
                                  bool split, bool q_bf16, int kv, hipStream_t s) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_prefix_t<kKvE4M3, true, D>(p, num_tiles, waves, append, split, s)
                  : launch_prefix_t<kKvE4M3, false, D>(p, num_tiles, waves, append, split, s);
  return q_bf16 ? launch_prefix_t<kKvBF16, true, D>(p, num_tiles, waves, append, split, s)
                : launch_prefix_t<kKvF16, false, D>(p, num_tiles, waves, append, split, s);
}

// ---- record instances (test hook): head_dim 128, 8 waves, fp16 q + fp16 K/V
// (cascade and append) or bf16 q + e4m3 K/V (cascade)
template <int KV, bool QBF16, int MODE>
static hipError_t launch_prefix_rec_t(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, 8, true, MODE, 128, false, true>), dim3(num_tiles),
                       dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, 8, false, MODE, 128, false, true>), dim3(num_tiles),
                       dim3(512), 0, s, p);
  return hipGetLastError();
}

static hipError_t launch_prefix_rec(const DecodeParams& p, int num_tiles, int waves,
                                    bool append, bool q_bf16, int kv, int head_dim,
                                    hipStream_t s) {
  if (head_dim != 128 || waves != 8) return hipErrorInvalidValue;
  if (kv == kKvF16 && !q_bf16)
    return append ? launch_prefix_rec_t<kKvF16, false, kPrefixAppend>(p, num_tiles, s)
                  : launch_prefix_rec_t<kKvF16, false, kPrefixPlain>(p, num_tiles, s);
  if (kv == kKvE4M3 && q_bf16 && !append)
    return launch_prefix_rec_t<kKvE4M3, true, kPrefixPlain>(p, num_tiles, s);
  return hipErrorInvalidValue;
}

// append: append tiles (rows limited by ReqInfo.kv_len), else cascade
// prefix; split: bf16 cascade prefix tiles pass p with a residual.
// head_dim: 64, 128 or 256.  p.rope_table != NULL selects the RoPE
// instances (prefix_rope.hip).
hipError_t launch_prefix(const DecodeParams& p, int num_tiles, int waves, bool append,
                         bool split, bool q_bf16, int kv, int head_dim, hipStream_t s) {
  if (waves != 4 && waves != 8) return hipErrorInvalidValue;
  if (p.rec) {
    if (num_tiles <= 0) return hipSuccess;
    return launch_prefix_rec(p, num_tiles, waves, append, q_bf16, kv, head_dim, s);
  }
  if (p.rope_table)
    return launch_prefix_rope(p, num_tiles, waves, append, split, q_bf16, kv, head_dim, s);
  switch (head_dim) {
    case 64: return launch_prefix_d<64>(p, num_tiles, waves, append, split, q_bf16, kv, s);
    case 128: return launch_prefix_d<128>(p, num_tiles, waves, append, split, q_bf16, kv, s);
    case 256: return launch_prefix_d<256>(p, num_tiles, waves, append, split, q_bf16, kv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fi
