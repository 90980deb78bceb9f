// Log-sum-exp merge of KV-split partials (second pass of FlashDecoding-style
// decode: page "字节跳动 AI Infra (2)", third question, layer-2 table).
//
// Partition p of a sequence carries its normalised output o_p and
// lse_p = log sum over its tokens of exp(score).  With M = max_p lse_p and
// w_p = exp(lse_p - M), the full-sequence output is sum_p w_p o_p / sum_p w_p
// (the online-softmax statistics of page "LLM推理优化", section 2.2, combined
// across ranges).
//
// One work-group of 4 wavefronts per (sequence, query head).  Wavefront w
// folds partitions w, w + 4, ... (lanes cover head_dim, 8 bytes per lane at
// head_dim 128), loading four partitions ahead; the four wavefront sums are
// then added in wavefront order through LDS, so the summation order is fixed
// and the result bitwise reproducible.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kRw = 4;      // wavefronts per work-group
constexpr int kUnroll = 4;  // partitions in flight per wavefront

template <int VEC>
struct Vec;
template <>
struct Vec<1> {
  typedef float T;
};
template <>
struct Vec<2> {
  typedef float2 T;
};

template <int D>
__global__ __launch_bounds__(kRw * 64) void reduce_kernel(ReduceParams p) {
  constexpr int VEC = D / 64;  // floats per lane
  typedef typename Vec<VEC>::T VT;
  __shared__ float sm_max[kRw];
  __shared__ float sm_w[kRw];
  __shared__ float sm_acc[kRw][D];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const size_t row = blockIdx.x;  // b * num_heads + h
  const int b = static_cast<int>(row / p.num_heads);
  const int L = max(p.context_lens[b], 0);
  const int n = min((L + p.partition_size - 1) / p.partition_size, p.max_num_partitions);
  const float *lse = p.part_lse + row * p.max_num_partitions;
  const VT *po = reinterpret_cast<const VT *>(p.part_out + row * p.max_num_partitions * D);

  // M = max over the used partitions (max is exact in any order)
  float m = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kRw * 64) m = fmaxf(m, lse[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) sm_max[w] = m;
  __syncthreads();
  float M = sm_max[0];
#pragma unroll
  for (int v = 1; v < kRw; ++v) M = fmaxf(M, sm_max[v]);

  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    constexpr float kLog2e = 1.4426950408889634f;
    for (int i0 = w; i0 < n; i0 += kRw * kUnroll) {
      VT v[kUnroll];
      float l[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = min(i0 + u * kRw, n - 1);
        v[u] = po[static_cast<size_t>(i) * 64 + lane];
        l[u] = lse[i];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (i0 + u * kRw < n) {
          const float wt = __builtin_amdgcn_exp2f((l[u] - M) * kLog2e);
          wsum += wt;
          if constexpr (VEC == 1) {
            acc[0] += wt * v[u];
          } else {
            acc[0] += wt * v[u].x;
            acc[1] += wt * v[u].y;
          }
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < VEC; ++k) sm_acc[w][lane * VEC + k] = acc[k];
  if (lane == 0) sm_w[w] = wsum;
  __syncthreads();
  if (w == 0) {
    float tw = 0.f;
#pragma unroll
    for (int v = 0; v < kRw; ++v) tw += sm_w[v];
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
      const int d = lane * VEC + k;
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < kRw; ++v) s += sm_acc[v][d];
      const float o = tw > 0.f ? s / tw : 0.f;
      const size_t idx = row * D + d;
      if (p.out_bf16)
        static_cast<uint16_t *>(p.out)[idx] = float_to_bf16_bits(o);
      else
        static_cast<float *>(p.out)[idx] = o;
    }
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceParams &p, hipStream_t s) {
  const uint32_t nwg = static_cast<uint32_t>(static_cast<int64_t>(p.num_seqs) * p.num_heads);
  if (p.head_dim == 128)
    hipLaunchKernelGGL(reduce_kernel<128>, dim3(nwg), dim3(kRw * 64), 0, s, p);
  else if (p.head_dim == 64)
    hipLaunchKernelGGL(reduce_kernel<64>, dim3(nwg), dim3(kRw * 64), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pa
