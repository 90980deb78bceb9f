// Log-sum-exp merge of KV-split partials (second pass of FlashDecoding-style
// decode: page "字节跳动 AI Infra (2)", third question, layer-2 table).
//
// Partition p of a sequence carries its normalised output o_p and
// lse_p = log sum over its tokens of exp(score).  With M = max_p lse_p and
// w_p = exp(lse_p - M), the full-sequence output is sum_p w_p o_p / sum_p w_p
// (the online-softmax statistics of page "LLM推理优化", section 2.2, combined
// across ranges).
//
// A work-group of four wavefronts serves RPW (sequence, query head) rows;
// each row gets W = 4 / RPW wavefronts, and wavefront w of a row folds the
// row's partitions w, w + W, ... with kUnroll of them loaded at once (lanes
// cover head_dim, 8 bytes per lane at head_dim 128).  Each wavefront keeps
// its own maximum; the W partial sums are rescaled to the row maximum and
// added in wavefront order, so the result is bitwise reproducible.  The host
// picks RPW from max_num_partitions: many short rows pack four to a
// work-group, a few long rows get four wavefronts each.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;   // wavefronts per work-group
constexpr int kUnroll = 16;  // partitions in flight per wavefront

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

template <int D, int RPW>
__global__ __launch_bounds__(kWaves * 64) void reduce_kernel(ReduceParams p) {
  constexpr int VEC = D / 64;  // floats per lane
  constexpr int W = kWaves / RPW;  // wavefronts per row
  typedef typename Vec<VEC>::T VT;
  __shared__ float sm_m[kWaves];
  __shared__ float sm_l[kWaves];
  __shared__ float sm_acc[kWaves][D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = wave / W;  // row of this work-group
  const int w = wave % W;  // wavefront within the row
  const int64_t rows = static_cast<int64_t>(p.num_seqs) * p.num_heads;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPW + r;
  const bool live = row < rows;

  float m = -INFINITY, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
  if (live) {
    const int b = static_cast<int>(row / p.num_heads);
    const int L = max(p.context_lens[b], 0);
    const int n = min((L + p.partition_size - 1) / p.partition_size, p.max_num_partitions);
    const float *lse = p.part_lse + row * p.max_num_partitions;
    const VT *po = reinterpret_cast<const VT *>(p.part_out + row * p.max_num_partitions * D);
    constexpr float kLog2e = 1.4426950408889634f;
    for (int i0 = w; i0 < n; i0 += W * kUnroll) {
      VT v[kUnroll];
      float ls[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = min(i0 + u * W, n - 1);
        v[u] = po[static_cast<size_t>(i) * 64 + lane];
        ls[u] = lse[i];
      }
      float mn = m;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (i0 + u * W < n) mn = fmaxf(mn, ls[u]);
      if (mn != -INFINITY) {
        const float alpha = __builtin_amdgcn_exp2f((m - mn) * kLog2e);  // 0 when m is -inf
        l *= alpha;
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] *= alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (i0 + u * W < n) {
            const float wt = __builtin_amdgcn_exp2f((ls[u] - mn) * kLog2e);
            l += wt;
            if constexpr (VEC == 1) {
              acc[0] += wt * v[u];
            } else {
              acc[0] += wt * v[u].x;
              acc[1] += wt * v[u].y;
            }
          }
        }
        m = mn;
      }
    }
  }
  if constexpr (W == 1) {
    if (live) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float o = l > 0.f ? acc[k] / l : 0.f;
        const size_t idx = static_cast<size_t>(row) * D + lane * VEC + k;
        if (p.out_bf16)
          static_cast<uint16_t *>(p.out)[idx] = float_to_bf16_bits(o);
        else
          static_cast<float *>(p.out)[idx] = o;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < VEC; ++k) sm_acc[wave][lane * VEC + k] = acc[k];
    if (lane == 0) {
      sm_m[wave] = m;
      sm_l[wave] = l;
    }
    __syncthreads();
    if (w == 0 && live) {
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < W; ++v) M = fmaxf(M, sm_m[r * W + v]);
      float f[W];
      float tl = 0.f;
#pragma unroll
      for (int v = 0; v < W; ++v) {
        f[v] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sm_m[r * W + v] - M) * 1.4426950408889634f);
        tl += f[v] * sm_l[r * W + v];
      }
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const int d = lane * VEC + k;
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < W; ++v) s += f[v] * sm_acc[r * W + v][d];
        const float o = tl > 0.f ? s / tl : 0.f;
        const size_t idx = static_cast<size_t>(row) * D + d;
        if (p.out_bf16)
          static_cast<uint16_t *>(p.out)[idx] = float_to_bf16_bits(o);
        else
          static_cast<float *>(p.out)[idx] = o;
      }
    }
  }
}

template <int D, int RPW>
hipError_t launch_r(const ReduceParams &p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.num_seqs) * p.num_heads;
  const uint32_t nwg = static_cast<uint32_t>((rows + RPW - 1) / RPW);
  hipLaunchKernelGGL((reduce_kernel<D, RPW>), dim3(nwg), dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ReduceParams &p, hipStream_t s) {
  // one wavefront per row while it can hold every partition in flight at once
  if (p.max_num_partitions <= kUnroll) return launch_r<D, 4>(p, s);
  if (p.max_num_partitions <= 2 * kUnroll) return launch_r<D, 2>(p, s);
  return launch_r<D, 1>(p, s);
}

}  // namespace

hipError_t launch_reduce(const ReduceParams &p, hipStream_t s) {
  if (p.head_dim == 128) return launch_d<128>(p, s);
  if (p.head_dim == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
