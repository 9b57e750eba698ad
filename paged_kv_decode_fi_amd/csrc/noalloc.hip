// noalloc.hip -- the device scratch of the allocation-free decode entry
// point (fi_decode_noalloc) and the planner that writes its work list on the
// device.
//
// Callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc) pass only inputs and
// outputs.  The work list, request info, merge units and fp32 partial states
// of a plain decode then live in one file-scope device array, `scratch`, of
// kScratchBytes per GPU, held until the process ends.  Every call on a GPU
// uses that GPU's copy: calls that overlap on one GPU (two streams, two host
// threads) race on it.  Nothing in it has to start at zero: the planner
// kernel rewrites the work list each call and every partial state is written
// before the merge reads it.
//
// The work list is the planned decode's (README "core features" item 2:
// plan, then run), cut the same way: the host picks the chunk length from
// the host copies of the page table, and device_plan_kernel derives every
// tile from the device copies -- so no host-to-device copy is needed and the
// call can be captured into a graph.  Tiles come out request by request
// instead of longest first; each tile computes the same thing either way.
#include <mutex>

#include "fi_device.h"

namespace fi {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per GPU
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

size_t scratch_capacity() { return kScratchBytes; }

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; host code uses only this
// address, never the array's name.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

struct DevicePlanArgs {
  const int32_t* kv_indptr;       // device [B+1]
  const int32_t* last_page_len;   // device [B] (NULL: ragged, lengths from indptr)
  int32_t batch, page_size, chunk, heads_per_tile, Hkv;
  Tile* tiles;                    // capacity tile_cap
  ReqInfo* req_info;              // [B]
  MergeUnit* units;               // capacity unit_cap
  int64_t tile_cap, unit_cap;
};

// Inclusive scan of three counts over a 1024-thread workgroup; returns the
// workgroup totals.
__device__ __forceinline__ void block_scan3(int64_t (&v)[3], int64_t (&total)[3],
                                            int64_t* lds /* [16][3] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t t = __shfl_up(v[k], o);
      if (lane >= o) v[k] += t;
    }
  if (lane == 63)
#pragma unroll
    for (int k = 0; k < 3; ++k) lds[wave * 3 + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    int64_t before = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
      const int64_t x = lds[w * 3 + k];
      if (w < wave) before += x;
      all += x;
    }
    v[k] += before;
    total[k] = all;
  }
  __syncthreads();
}

// One workgroup of 1024 threads: request r's length from its table row,
// its chunk count nc = ceil(len / chunk), then by exclusive scans over the
// batch its tile, partial-slot and merge-unit offsets; writes max(nc, 1) x
// (Hkv / heads_per_tile) tiles (an empty request gets one empty tile per
// head group, which writes o = 0, lse = -inf), its request info and, when
// split (nc >= 2), a merge unit.  Writes stay within the capacities the host
// computed from its copy of the tables.
__global__ __launch_bounds__(1024) void device_plan_kernel(DevicePlanArgs a) {
  __shared__ int64_t lds[16 * 3];
  const int HG = a.Hkv / a.heads_per_tile;
  int64_t carry[3] = {0, 0, 0};   // tiles, slots, units before this round
  for (int r0 = 0; r0 < a.batch; r0 += 1024) {
    const int r = r0 + (int)threadIdx.x;
    int64_t len = 0, nc = 0, page_base = 0;
    if (r < a.batch) {
      page_base = a.kv_indptr[r];
      const int64_t n = (int64_t)a.kv_indptr[r + 1] - page_base;
      len = a.last_page_len ? (n == 0 ? 0 : (n - 1) * a.page_size + a.last_page_len[r]) : n;
      nc = len > 0 ? (len + a.chunk - 1) / a.chunk : 0;
    }
    const bool split = nc >= 2;
    int64_t v[3] = {r < a.batch ? (nc > 1 ? nc : 1) * HG : 0, split ? nc * a.Hkv : 0,
                    split ? 1 : 0};
    const int64_t own[3] = {v[0], v[1], v[2]};
    int64_t total[3];
    block_scan3(v, total, lds);
    if (r < a.batch) {
      const int64_t tb = carry[0] + v[0] - own[0];
      const int64_t sb = carry[1] + v[1] - own[1];
      const int64_t ub = carry[2] + v[2] - own[2];
      a.req_info[r] = ReqInfo{split ? (int32_t)sb : -1, (int32_t)nc, (int32_t)len, 0};
      if (split && ub < a.unit_cap) a.units[ub] = MergeUnit{r, (int32_t)sb, (int32_t)nc, 0};
      const int64_t ncx = nc > 1 ? nc : 1;
      // the request's 16-token steps shared out evenly over its chunks (the
      // first ones one step longer), as the host plan does
      const int64_t nst = (len + kChunkAlign - 1) / kChunkAlign;
      const int64_t per = nst / ncx, extra = nst % ncx;
      auto bound = [&](int64_t c) {
        return (int32_t)min((int64_t)kChunkAlign * (c * per + min(c, extra)), len);
      };
      for (int64_t c = 0; c < ncx; ++c)
        for (int hg = 0; hg < HG; ++hg) {
          const int64_t ti = tb + c * HG + hg;
          if (ti >= a.tile_cap) continue;
          Tile t;
          t.req = r;
          t.kv_head0 = hg * a.heads_per_tile;
          t.t0 = bound(c);
          t.t1 = bound(c + 1);
          t.slot = split ? (int32_t)(sb + c * a.Hkv + t.kv_head0) : -1;
          t.kind = kDecodeTile;
          t.row0 = (int32_t)page_base;   // the request's first page-table entry
          t.row1 = 0;
          a.tiles[ti] = t;
        }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) carry[k] += total[k];
  }
}

hipError_t launch_device_plan(const int32_t* kv_indptr, const int32_t* last_page_len,
                              int batch, int page_size, int chunk, int heads_per_tile, int Hkv,
                              void* tiles, void* req_info, void* units, int64_t tile_cap,
                              int64_t unit_cap, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  DevicePlanArgs a;
  a.kv_indptr = kv_indptr;
  a.last_page_len = last_page_len;
  a.batch = batch;
  a.page_size = page_size;
  a.chunk = chunk;
  a.heads_per_tile = heads_per_tile;
  a.Hkv = Hkv;
  a.tiles = reinterpret_cast<Tile*>(tiles);
  a.req_info = reinterpret_cast<ReqInfo*>(req_info);
  a.units = reinterpret_cast<MergeUnit*>(units);
  a.tile_cap = tile_cap;
  a.unit_cap = unit_cap;
  hipLaunchKernelGGL(device_plan_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace fi
