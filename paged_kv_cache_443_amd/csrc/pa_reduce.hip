// Log-sum-exp merge of KV-split partials (second pass of FlashDecoding-style
// decode: page "字节跳动 AI Infra (2)", third question, layer-2 table).
//
// Partition p of a sequence carries its normalised output o_p and
// lse_p = log sum over its tokens of exp(score).  With M = max_p lse_p and
// w_p = exp(lse_p - M), the full-sequence output is sum_p w_p o_p / sum_p w_p
// (the online-softmax statistics of page "LLM推理优化", section 2.2, combined
// across ranges).  One wavefront per (sequence, query head); lane l owns
// channels l, l + 64.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

template <int D>
__global__ __launch_bounds__(64) void reduce_kernel(ReduceParams p) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;  // b * num_heads + h
  const int b = static_cast<int>(row / p.num_heads);
  const int L = max(p.context_lens[b], 0);
  const int n = min((L + p.partition_size - 1) / p.partition_size, p.max_num_partitions);
  const float *lse = p.part_lse + row * p.max_num_partitions;
  const float *po = p.part_out + row * p.max_num_partitions * D;

  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, lse[i]);
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int i = 0; i < n; ++i) {
      const float w = expf(lse[i] - M);
      wsum += w;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += w * po[static_cast<size_t>(i) * D + lane + 64 * k];
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float o = wsum > 0.f ? acc[k] / wsum : 0.f;
    const size_t idx = row * D + lane + 64 * k;
    if (p.out_bf16)
      static_cast<uint16_t *>(p.out)[idx] = float_to_bf16_bits(o);
    else
      static_cast<float *>(p.out)[idx] = o;
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceParams &p, hipStream_t s) {
  const uint32_t nwg = static_cast<uint32_t>(static_cast<int64_t>(p.num_seqs) * p.num_heads);
  if (p.head_dim == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, dim3(nwg), dim3(64), 0, s, p);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL(reduce_kernel<64>, dim3(nwg), dim3(64), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
