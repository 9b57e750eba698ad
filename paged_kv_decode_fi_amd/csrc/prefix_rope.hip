// prefix_rope.hip -- the RoPE instances of the multi-row kernel
// (fi_prefix.h): cascade prefix tiles and batch-append tiles whose query
// rows and keys are turned by their positions (absolute form, described
// above the kernel).  8 waves, 16 query rows per wave.
#include "fi_prefix.h"

namespace fi {

template <int KV, bool QBF16, int MODE, int D>
static void launch_prefix_rope_m(const DecodeParams& p, int num_tiles, hipStream_t s) {
  if (p.ps_shift >= 0)
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, 8, true, MODE, D, true>), dim3(num_tiles),
                       dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((prefix_kernel<KV, QBF16, 8, false, MODE, D, true>), dim3(num_tiles),
                       dim3(512), 0, s, p);
}

template <int KV, bool QBF16, int D>
static hipError_t launch_prefix_rope_t(const DecodeParams& p, int num_tiles, bool append,
                                       bool split, hipStream_t s) {
  if (num_tiles <= 0) return hipSuccess;
  if (append) {
    launch_prefix_rope_m<KV, QBF16, kPrefixAppend, D>(p, num_tiles, s);
  } else {
    bool done = false;
    if constexpr (KV == kKvBF16) {   // the split instance exists for bf16 K/V only
      if (split) {
        launch_prefix_rope_m<KV, QBF16, kPrefixSplitP, D>(p, num_tiles, s);
        done = true;
      }
    }
    if (!done) launch_prefix_rope_m<KV, QBF16, kPrefixPlain, D>(p, num_tiles, s);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefix_rope_d(const DecodeParams& p, int num_tiles, bool append,
                                       bool split, bool q_bf16, int kv, hipStream_t s) {
  if (kv == kKvE4M3)
    return q_bf16 ? launch_prefix_rope_t<kKvE4M3, true, D>(p, num_tiles, append, split, s)
                  : launch_prefix_rope_t<kKvE4M3, false, D>(p, num_tiles, append, split, s);
  return q_bf16 ? launch_prefix_rope_t<kKvBF16, true, D>(p, num_tiles, append, split, s)
                : launch_prefix_rope_t<kKvF16, false, D>(p, num_tiles, append, split, s);
}

// p.rope_table: the plan's fp32 (cos, sin) table; p.rope_qpos: the
// positions of the query rows (cascade: this level's row of the plan's
// table, append: one per query token).  waves must be 8.
hipError_t launch_prefix_rope(const DecodeParams& p, int num_tiles, int waves, bool append,
                              bool split, bool q_bf16, int kv, int head_dim, hipStream_t s) {
  if (waves != 8 || !p.rope_qpos) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return launch_prefix_rope_d<64>(p, num_tiles, append, split, q_bf16, kv, s);
    case 128: return launch_prefix_rope_d<128>(p, num_tiles, append, split, q_bf16, kv, s);
    case 256: return launch_prefix_rope_d<256>(p, num_tiles, append, split, q_bf16, kv, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fi
