// Paged decode attention for fp32 KV caches, on the vector ALUs.
//
// Same result as the matrix-core path (page "字节跳动 AI Infra (2)", KV-cache
// question, step-t equations; block-table walk from the same page's
// PagedAttention sketch), kept in fp32 end to end: products, online softmax
// (page "LLM推理优化", section 2.2) and accumulation.  One wavefront per
// (query head, sequence[, partition]), or per (query head, query row) for
// causal multi-query launches (query token i of a sequence's n new tokens
// sees the positions up to L - n + i: the step-t equations taken for each new
// token); lane l owns channels l, l + 64.  This path serves fp32 caches
// (exactness over speed); bf16, int8 and int4 caches use the matrix cores.
#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int D, int BS, bool CAUSAL>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeParams p) {
  constexpr int X = 4;
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int id = blockIdx.x;
  const int hq = id % p.num_heads;
  const int rest = id / p.num_heads;
  const int kvh = hq / p.group;
  int b, part = 0;
  size_t row;  // row of q and out (query row x heads + head)
  int nq = 1, i = 0;
  if constexpr (CAUSAL) {
    // query row `rest`: its sequence is the last b with q_start[b] <= rest
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.q_start[mid] <= rest) lo = mid; else hi = mid - 1;
    }
    b = lo;
    const int qb = p.q_start[b];
    nq = p.q_start[b + 1] - qb;
    i = rest - qb;
    // a sequence whose offsets leave [0, num_queries] or exceed max_q_len is
    // skipped, as are rows outside it (uniform over the wavefront)
    if (qb < 0 || nq < 1 || qb + nq > p.num_queries || nq > p.max_q_len || i < 0 || i >= nq) return;
    row = static_cast<size_t>(rest) * p.num_heads + hq;
  } else {
    b = rest % p.num_seqs;
    part = rest / p.num_seqs;
    row = static_cast<size_t>(b) * p.num_heads + hq;
  }

  const int L = min(max(p.context_lens[b], 0), p.max_blocks_per_seq * BS);
  int t0 = 0, t1 = L;
  if constexpr (CAUSAL) t1 = max(0, min(L, L - nq + i + 1));  // positions up to the row's own
  if (p.partition_size > 0) {
    t0 = part * p.partition_size;
    t1 = min(t0 + p.partition_size, L);
  }
  if (p.partition_size > 0 && t1 <= t0) return;  // partitions past the end are left untouched
  const int32_t *table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  const float *kpool = static_cast<const float *>(p.k_cache);
  const float *vpool = static_cast<const float *>(p.v_cache);

  float qv[PER], acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    qv[k] = static_cast<const float *>(p.q)[row * D + lane + 64 * k];
    acc[k] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int t = t0; t < t1; ++t) {
    const uint32_t pb = min(static_cast<uint32_t>(table[t / BS]), static_cast<uint32_t>(p.num_blocks - 1));
    const int o = t % BS;
    const size_t tile = static_cast<size_t>(pb) * p.num_kv_heads + kvh;
    float part_dot = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      part_dot += qv[k] * kpool[((tile * (D / X) + d / X) * BS + o) * X + d % X];
    }
    const float s = wave_sum(part_dot) * p.scale_log2;
    const float m_new = fmaxf(m_run, s);
    const float alpha = exp2f(m_run - m_new);
    const float pe = exp2f(s - m_new);
    m_run = m_new;
    l_run = l_run * alpha + pe;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      acc[k] = acc[k] * alpha + pe * vpool[((tile * (BS / X) + o / X) * D + d) * X + o % X];
    }
  }
  const bool empty = t1 <= t0;
  if (p.partition_size > 0) {
    const size_t prow = row * p.max_num_partitions + part;
#pragma unroll
    for (int k = 0; k < PER; ++k) p.part_out[prow * D + lane + 64 * k] = empty ? 0.f : acc[k] / l_run;
    if (lane == 0) p.part_lse[prow] = empty ? -INFINITY : (m_run + log2f(l_run)) * kLn2;
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) static_cast<float *>(p.out)[row * D + lane + 64 * k] = empty ? 0.f : acc[k] / l_run;
  }
}

template <int D, int BS>
hipError_t launch_t(const DecodeParams &p, hipStream_t s) {
  if (p.q_start != nullptr) {  // causal multi-query: one wavefront per (query row, head)
    const int64_t nwg = static_cast<int64_t>(p.num_heads) * p.num_queries;
    hipLaunchKernelGGL((decode_f32_kernel<D, BS, true>), dim3(static_cast<uint32_t>(nwg)), dim3(64), 0, s, p);
    return hipGetLastError();
  }
  const int64_t nparts = p.partition_size > 0 ? p.max_num_partitions : 1;
  const int64_t nwg = static_cast<int64_t>(p.num_heads) * p.num_seqs * nparts;
  hipLaunchKernelGGL((decode_f32_kernel<D, BS, false>), dim3(static_cast<uint32_t>(nwg)), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bs(const DecodeParams &p, int bs, hipStream_t s) {
  switch (bs) {
    case 16: return launch_t<D, 16>(p, s);
    case 32: return launch_t<D, 32>(p, s);
    case 64: return launch_t<D, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_f32(const DecodeParams &p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim == 128) return launch_bs<128>(p, block_size, s);
  if (head_dim == 64) return launch_bs<64>(p, block_size, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
