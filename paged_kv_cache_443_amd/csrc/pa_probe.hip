// HBM read probe: the achievable read rate of this GPU for the access
// patterns paged decode makes, and the cache flush of the benchmark.
//
// Decode is bound by reading the KV cache (page "vLLM框架是怎么做推理加速的",
// section 3), so its speed follows HBM bandwidth (page "字节跳动 AI Infra
// (2)", third question, layer-4 table).  The probe measures what a kernel can
// actually pull from HBM here: a plain sequential pass, and whole tiles of
// tile_bytes read in a scattered order (the shape of a block-table gather:
// every (block, kv head) tile is contiguous, the tiles are not).  Loads are
// ordinary (they allocate in L2 and the Infinity Cache; a pass over a buffer
// larger than both is the benchmark's flush) or non-temporal.
//
// Every 32-bit word read is folded into a per-thread XOR; a thread writes its
// fold to sink[0] only if it equals a fixed constant, so the loads cannot be
// removed and the sink is practically never written.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;  // loads in flight per thread
constexpr uint32_t kNeverFold = 0x9e3779b9u;

template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4 *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// A work-group reads one contiguous range of the pass, [beg, end) of
// `items`; its threads take kProbeInFlight neighbouring 4 KiB runs at a time
// (measured: about 7.0 TB/s for a sequential non-temporal pass, against 5.2-6.2
// for the same loads strided over the whole grid).
template <bool NT>
__device__ __forceinline__ uint32_t probe_range(const u32x4 *buf, int64_t items, int64_t per_wg, int vpt,
                                                int64_t ntiles) {
  const int64_t beg = static_cast<int64_t>(blockIdx.x) * per_wg;
  const int64_t end = beg + per_wg < items ? beg + per_wg : items;
  const uint64_t mask = static_cast<uint64_t>(ntiles) - 1;
  uint32_t acc = 0;
  for (int64_t i0 = beg + threadIdx.x; i0 < end; i0 += kProbeInFlight * kProbeThreads) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int64_t i = i0 + u * kProbeThreads;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (i < end) {
        int64_t at = i;  // sequential pass: item i is vector i
        if (ntiles > 0) {
          // tile pass: item i is vector i % vpt of tile t = i / vpt of the pass,
          // physical tile perm(t) = (t * odd + offset) mod ntiles (a bijection:
          // ntiles is a power of two), so neighbours in the pass lie far apart
          const uint64_t t = static_cast<uint64_t>(i / vpt);
          const uint64_t pt = (t * 0x9E3779B97F4A7C15ull + 0x632BE59BD9B4E019ull) & mask;
          at = static_cast<int64_t>(pt) * vpt + (i % vpt);
        }
        v[u] = probe_load<NT>(buf + at);
      }
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= fold(v[u]);
  }
  return acc;
}

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_kernel(const u32x4 *buf, int64_t items, int64_t per_wg, int vpt,
                                                              int64_t ntiles, uint32_t *sink) {
  const uint32_t acc = probe_range<NT>(buf, items, per_wg, vpt, ntiles);
  if (acc == kNeverFold) sink[0] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void *buf, size_t bytes, int mode, int tile_bytes, uint32_t *sink, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const u32x4 *b = static_cast<const u32x4 *>(buf);
  int64_t items = static_cast<int64_t>(bytes / 16), ntiles = 0;
  int vpt = 1;
  if (mode >= 2) {  // the largest power-of-two count of whole tiles that fits
    ntiles = 1;
    while (ntiles * 2 * static_cast<int64_t>(tile_bytes) <= static_cast<int64_t>(bytes)) ntiles *= 2;
    vpt = tile_bytes / 16;
    items = ntiles * vpt;
  }
  // eight work-groups per CU, each a contiguous range of whole in-flight rounds
  constexpr int64_t kRound = static_cast<int64_t>(kProbeThreads) * kProbeInFlight;
  const int64_t want = 8LL * std::max(cus, 1);
  const int64_t per_wg = std::max<int64_t>(kRound, (items + want * kRound - 1) / (want * kRound) * kRound);
  const uint32_t grid = static_cast<uint32_t>((items + per_wg - 1) / per_wg);
  if (mode & 1)
    hipLaunchKernelGGL(probe_kernel<true>, dim3(grid), dim3(kProbeThreads), 0, s, b, items, per_wg, vpt, ntiles, sink);
  else
    hipLaunchKernelGGL(probe_kernel<false>, dim3(grid), dim3(kProbeThreads), 0, s, b, items, per_wg, vpt, ntiles, sink);
  return hipGetLastError();
}

}  // namespace pa
