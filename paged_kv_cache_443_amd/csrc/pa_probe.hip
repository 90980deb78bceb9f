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

// Sequential: vector i of the buffer, grid-stride, kProbeInFlight loads at a time.
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_seq_kernel(const u32x4 *buf, int64_t nvec, uint32_t *sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  uint32_t acc = 0;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i0 < nvec;
       i0 += kProbeInFlight * stride) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = i < nvec ? probe_load<NT>(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= fold(v[u]);
  }
  if (acc == kNeverFold) sink[0] = acc;
}

// Scattered tiles: tile t of the pass reads physical tile
// perm(t) = (t * odd + offset) mod ntiles (ntiles a power of two, so perm is a
// bijection): every tile once, neighbours in the pass far apart in memory.
// A work-group reads whole tiles; kProbeInFlight tiles per thread in flight.
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_tiles_kernel(const u32x4 *buf, int64_t ntiles, int vec_per_tile,
                                                                    uint32_t *sink) {
  const int64_t items = ntiles * vec_per_tile;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  const uint64_t mask = static_cast<uint64_t>(ntiles) - 1;
  uint32_t acc = 0;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i0 < items;
       i0 += kProbeInFlight * stride) {
    u32x4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (i < items) {
        const uint64_t t = static_cast<uint64_t>(i / vec_per_tile);
        const uint64_t pt = (t * 0x9E3779B97F4A7C15ull + 0x632BE59BD9B4E019ull) & mask;
        v[u] = probe_load<NT>(buf + pt * vec_per_tile + (i % vec_per_tile));
      }
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= fold(v[u]);
  }
  if (acc == kNeverFold) sink[0] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void *buf, size_t bytes, int mode, int tile_bytes, uint32_t *sink, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const u32x4 *b = static_cast<const u32x4 *>(buf);
  const bool nt = (mode & 1) != 0;
  if (mode < 2) {
    const int64_t nvec = static_cast<int64_t>(bytes / 16);
    const int64_t want = (nvec + kProbeThreads * kProbeInFlight - 1) / (kProbeThreads * kProbeInFlight);
    const uint32_t grid = static_cast<uint32_t>(std::max<int64_t>(1, std::min<int64_t>(want, 16LL * cus)));
    if (nt)
      hipLaunchKernelGGL(probe_seq_kernel<true>, dim3(grid), dim3(kProbeThreads), 0, s, b, nvec, sink);
    else
      hipLaunchKernelGGL(probe_seq_kernel<false>, dim3(grid), dim3(kProbeThreads), 0, s, b, nvec, sink);
    return hipGetLastError();
  }
  int64_t ntiles = 1;
  while (ntiles * 2 * static_cast<int64_t>(tile_bytes) <= static_cast<int64_t>(bytes)) ntiles *= 2;
  const int vpt = tile_bytes / 16;
  const int64_t items = ntiles * vpt;
  const int64_t want = (items + kProbeThreads * kProbeInFlight - 1) / (kProbeThreads * kProbeInFlight);
  const uint32_t grid = static_cast<uint32_t>(std::max<int64_t>(1, std::min<int64_t>(want, 16LL * cus)));
  if (nt)
    hipLaunchKernelGGL(probe_tiles_kernel<true>, dim3(grid), dim3(kProbeThreads), 0, s, b, ntiles, vpt, sink);
  else
    hipLaunchKernelGGL(probe_tiles_kernel<false>, dim3(grid), dim3(kProbeThreads), 0, s, b, ntiles, vpt, sink);
  return hipGetLastError();
}

}  // namespace pa
