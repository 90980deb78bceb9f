// Whole-block copies between pools of one layout.
//
// Copy-on-write copies inside one pool (page "字节跳动 AI Infra (2)",
// PagedAttention question, block-pool figure: the second beam writes into
// B6', a copy of the shared B6; page "LLM推理优化", section 3.2).  A swap
// copies between the GPU pool and a pinned host pool when a request is
// preempted or memory runs short, and back before it resumes (page
// "字节跳动 AI Infra (2)", PagedAttention question, scheduling list; page
// "vLLM框架是怎么做推理加速的", section 2); the GPU reaches the host pool
// directly over the bus, so one launch moves any number of blocks.
//
// One work-group per (pair, kv head): the (block, kv head) K tile and V tile
// are each block_size * head_dim contiguous elements in their pools (layout in
// pa.h), copied in 16-byte vectors, plus the tile's block_size fp16 scales for
// int8 caches.  Sources are read once: non-temporal loads.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;

template <bool SCALES>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyParams p) {
  const int pair = static_cast<int>(blockIdx.x / static_cast<uint32_t>(p.num_kv_heads));
  const int h = static_cast<int>(blockIdx.x % static_cast<uint32_t>(p.num_kv_heads));
  const int32_t src = p.pairs[2 * pair];
  const int32_t dst = p.pairs[2 * pair + 1];
  if (src < 0 || src >= p.src_blocks || dst < 0 || dst >= p.dst_blocks) return;  // skipped pair
  const size_t n16 = p.tile_bytes / 16;
  const size_t s_tile = static_cast<size_t>(src) * p.num_kv_heads + h;
  const size_t d_tile = static_cast<size_t>(dst) * p.num_kv_heads + h;
  const u32x4 *ks = static_cast<const u32x4 *>(p.src_k) + s_tile * n16;
  const u32x4 *vs = static_cast<const u32x4 *>(p.src_v) + s_tile * n16;
  u32x4 *kd = static_cast<u32x4 *>(p.dst_k) + d_tile * n16;
  u32x4 *vd = static_cast<u32x4 *>(p.dst_v) + d_tile * n16;
  for (size_t i = threadIdx.x; i < n16; i += kCopyThreads) {
    const u32x4 a = __builtin_nontemporal_load(ks + i);
    const u32x4 b = __builtin_nontemporal_load(vs + i);
    kd[i] = a;
    vd[i] = b;
  }
  if constexpr (SCALES) {
    const int s16 = p.block_size / 8;  // fp16 scales of one tile in 16-byte vectors
    if (static_cast<int>(threadIdx.x) < 2 * s16) {
      const int which = threadIdx.x / s16, i = threadIdx.x % s16;
      const u32x4 *ss = static_cast<const u32x4 *>(which ? p.src_v_scale : p.src_k_scale) + s_tile * s16;
      u32x4 *sd = static_cast<u32x4 *>(which ? p.dst_v_scale : p.dst_k_scale) + d_tile * s16;
      sd[i] = ss[i];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t s) {
  const uint32_t nwg = static_cast<uint32_t>(static_cast<int64_t>(p.num_pairs) * p.num_kv_heads);
  if (p.src_k_scale != nullptr)
    hipLaunchKernelGGL(copy_blocks_kernel<true>, dim3(nwg), dim3(kCopyThreads), 0, s, p);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<false>, dim3(nwg), dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
