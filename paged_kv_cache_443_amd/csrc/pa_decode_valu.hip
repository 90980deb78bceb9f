// Paged decode attention for bf16 KV caches on the vector ALUs.
//
// The same computation as the matrix-core units (page "字节跳动 AI Infra (2)",
// KV-cache question, step-t equations; block-table walk from the same page's
// PagedAttention sketch; online softmax, page "LLM推理优化", section 2.2),
// with every product on v_dot2_f32_bf16 (two bf16 products summed into an
// fp32 accumulator) instead of MFMA.  It exists to measure which arithmetic
// unit a single-token decode should use: the matrix cores spend a 16-row
// product on G query heads per kv head (15 of 16 rows idle at G = 1), the
// vector ALUs spend one lane-instruction per two products and nothing on
// padding.  pa_decode takes this path when the environment variable
// PA_DECODE_VALU is "1" (bf16 cache, head_dim 128, G <= 16, whole-sequence
// pass); otherwise the matrix-core units run.
//
// Work: one work-group of NW wavefronts per (sequence, kv head), holding
// the G query heads of that kv head.  Wavefront w takes the 32-token chunks
// w, w + NW, ... of the sequence, one chunk in flight while the previous one
// is computed, and the wavefronts' states are merged through LDS at the end.
//   QK: lane (t = lane % 32, half = lane / 32) holds token t's channels
//       64 half .. 64 half + 63 (eight 16-byte K vectors) and forms their
//       partial dot product with each head's query (LDS, broadcast reads);
//       the halves are summed across lanes.
//   softmax: per head, the chunk maximum across the 32 tokens, an online
//       update against a lazily moved reference (the weights stay below
//       2^8 between rescales), and the weights written to LDS as bf16
//       pairs, a high part and the remainder (their sum is the fp32 weight
//       to about 2^-17).
//   PV: lane l holds channels l and l + 64 for the chunk's four 8-token V
//       vectors each and accumulates both parts of every weight pair.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kValuD = 128;     // head_dim the kernel is built for
constexpr int kValuChunk = 32;  // tokens per wavefront step
constexpr int kValuNW = 4;      // wavefronts per work-group
// Weight growth (log2 units) the online softmax absorbs before it rescales.
constexpr float kValuLazyLog2 = 8.f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// LDS of one work-group; GP = G rounded up to a power of two (<= 16).
//   int32 tbl[TW]              block-table window
//   u32   q[GP][64]            queries as bf16 channel pairs
//   u32   pw[NW][GP][32]       per-wavefront weights: 16 high pairs, 16 remainder pairs
//   float m[NW][GP], l[NW][GP] per-wavefront softmax statistics
//   float acc[NW][GP][128]     per-wavefront outputs
template <int GP>
__host__ __device__ constexpr size_t valu_lds_bytes(int tw) {
  return static_cast<size_t>(tw) * 4 + GP * 64 * 4 + kValuNW * GP * 32 * 4 + 2 * kValuNW * GP * 4 +
         static_cast<size_t>(kValuNW) * GP * kValuD * 4;
}

template <int BS, int GP>
__global__ __launch_bounds__(kValuNW * 64) __attribute__((amdgpu_waves_per_eu(GP <= 2 ? 4 : 2)))
void decode_valu_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int TW = p.tbl_window;
  int32_t *tbl = reinterpret_cast<int32_t *>(smem);
  uint32_t *qs = reinterpret_cast<uint32_t *>(smem + static_cast<size_t>(TW) * 4);
  uint32_t *pw = qs + GP * 64;
  float *sm_m = reinterpret_cast<float *>(pw + kValuNW * GP * 32);
  float *sm_l = sm_m + kValuNW * GP;
  float *sm_acc = sm_l + kValuNW * GP;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int b = blockIdx.x / p.num_kv_heads;
  const int kvh = blockIdx.x % p.num_kv_heads;
  const int G = p.group;
  const int32_t *table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  const int L = min(max(p.context_lens[b], 0), p.max_blocks_per_seq * BS);

  // queries of the kv head's G heads (rows past G stay zero), first table window
  for (int i = threadIdx.x; i < GP * 64; i += kValuNW * 64) {
    const int g = i / 64;
    uint32_t v = 0u;
    if (g < G)
      v = reinterpret_cast<const uint32_t *>(p.q)[(static_cast<size_t>(b) * p.num_heads + kvh * G + g) * 64 + i % 64];
    qs[i] = v;
  }
  for (int i = threadIdx.x; i < min(TW, p.max_blocks_per_seq); i += kValuNW * 64) tbl[i] = table[i];

  const u32x4 *kpool = static_cast<const u32x4 *>(p.k_cache);
  const u32x4 *vpool = static_cast<const u32x4 *>(p.v_cache);
  const uint32_t nb_m1 = static_cast<uint32_t>(p.num_blocks - 1);
  const int t = lane & 31;
  const int half = lane >> 5;

  float acc[GP][2];
  float m_run[GP], l_run[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    acc[g][0] = acc[g][1] = 0.f;
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
  }
  uint32_t *my_pw = pw + w * GP * 32;
  __syncthreads();

  for (int ws = 0; ws < L; ws += TW * BS) {
    const int we = min(ws + TW * BS, L);
    const int lb0 = ws / BS;
    if (ws != 0) {
      __syncthreads();  // readers of the previous window are done
      for (int i = threadIdx.x; i < (we + BS - 1) / BS - lb0; i += kValuNW * 64) tbl[i] = table[lb0 + i];
      __syncthreads();
    }
    const int nbv = (we + BS - 1) / BS - lb0;  // window entries holding positions < we
    const int nch = (we - ws + kValuChunk - 1) / kValuChunk;

    // physical block of in-window position pos (clamped: a bad id never forms an address)
    auto blk = [&](int pos) -> uint32_t {
      const int lb = min(pos / BS - lb0, nbv - 1);
      return min(static_cast<uint32_t>(tbl[lb]), nb_m1);
    };
    u32x4 kb[8], vb[8];
    auto issue_k = [&](int cs) {
      const int pos = cs + t;
      const size_t tile = static_cast<size_t>(blk(pos)) * p.num_kv_heads + kvh;
      const u32x4 *kp = kpool + tile * (kValuD / 8) * BS + bf16_k_slot(pos % BS);
#pragma unroll
      for (int i = 0; i < 8; ++i) kb[i] = __builtin_nontemporal_load(kp + (8 * half + i) * BS);
    };
    auto issue_v = [&](int cs) {
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const int pos = cs + 8 * o;
        const size_t tile = static_cast<size_t>(blk(pos)) * p.num_kv_heads + kvh;
        const u32x4 *vp = vpool + (tile * (BS / 8) + (pos % BS) / 8) * kValuD + lane;
        vb[2 * o] = __builtin_nontemporal_load(vp);
        vb[2 * o + 1] = __builtin_nontemporal_load(vp + 64);
      }
    };

    // one chunk: QK, online softmax, PV; REFILL issues the loads of chunk cn
    // into each buffer as soon as it has been read (the last chunk of a
    // wavefront has no refill, so every load issued is consumed)
    auto consume = [&](int cs, int cn, auto refill) {
      constexpr bool REFILL = decltype(refill)::value;
      // ---- QK ---------------------------------------------------------------
      float s[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) s[g] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const u32x4 qq = reinterpret_cast<const u32x4 *>(qs + g * 64 + 32 * half)[i];
#pragma unroll
          for (int k = 0; k < 4; ++k) s[g] = dot2(kb[i][k], qq[k], s[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) s[g] += __shfl_xor(s[g], 32);
      if constexpr (REFILL) {
        __builtin_amdgcn_sched_barrier(0);
        issue_k(cn);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- online softmax, weights to LDS -------------------------------------
      const bool valid = cs + t < we;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float sv = valid ? s[g] * p.scale_log2 : -INFINITY;
        float cm = sv;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
        const float m_new = fmaxf(m_run[g], cm);
        const bool move = m_new > m_run[g] + kValuLazyLog2;  // uniform over the wavefront
        const float alpha = move ? fast_exp2(m_run[g] - m_new) : 1.f;
        m_run[g] = move ? m_new : m_run[g];
        acc[g][0] *= alpha;
        acc[g][1] *= alpha;
        l_run[g] *= alpha;
        const float pe = fast_exp2(sv - m_run[g]);
        if (half == 0) l_run[g] += pe;
        const uint32_t hbits = float_to_bf16_bits(pe);
        const uint32_t lbits = float_to_bf16_bits(pe - bf16_bits_to_float(hbits));
        const uint32_t hn = __shfl_xor(hbits, 1);
        const uint32_t ln = __shfl_xor(lbits, 1);
        if (half == 0 && (t & 1) == 0) {
          my_pw[g * 32 + t / 2] = hbits | (hn << 16);
          my_pw[g * 32 + 16 + t / 2] = lbits | (ln << 16);
        }
      }
      __builtin_amdgcn_wave_barrier();  // a wavefront's LDS accesses are performed in order
      // ---- PV ---------------------------------------------------------------
      if (cs + kValuChunk > we) {
        // V of positions >= we may hold NaN: zero it (0 * NaN would poison the sum)
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int tok = cs + 8 * o + 2 * k;
            const uint32_t keep = (tok < we ? 0x0000ffffu : 0u) | (tok + 1 < we ? 0xffff0000u : 0u);
            vb[2 * o][k] &= keep;
            vb[2 * o + 1][k] &= keep;
          }
      }
#pragma unroll
      for (int o = 0; o < 4; ++o) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const u32x4 *ph = reinterpret_cast<const u32x4 *>(my_pw + g * 32);
          const u32x4 h = ph[o];
          const u32x4 lo = ph[4 + o];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[g][0] = dot2(vb[2 * o][k], h[k], acc[g][0]);
            acc[g][0] = dot2(vb[2 * o][k], lo[k], acc[g][0]);
            acc[g][1] = dot2(vb[2 * o + 1][k], h[k], acc[g][1]);
            acc[g][1] = dot2(vb[2 * o + 1][k], lo[k], acc[g][1]);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // the weights are read before the next chunk overwrites them
      if constexpr (REFILL) {
        __builtin_amdgcn_sched_barrier(0);
        issue_v(cn);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // this wavefront's chunks of the window: w, w + NW, ...
    const int n = w < nch ? (nch - w + kValuNW - 1) / kValuNW : 0;
    if (n > 0) {
      int cs = ws + w * kValuChunk;
      issue_k(cs);
      issue_v(cs);
      for (int k = 0; k + 1 < n; ++k) {
        consume(cs, cs + kValuNW * kValuChunk, std::true_type{});
        cs += kValuNW * kValuChunk;
      }
      consume(cs, 0, std::false_type{});
    }
  }

  // ---- merge the wavefronts' states ---------------------------------------------
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    float l = l_run[g];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) l += __shfl_xor(l, off);
    sm_acc[(w * GP + g) * kValuD + lane] = acc[g][0];
    sm_acc[(w * GP + g) * kValuD + lane + 64] = acc[g][1];
    if (lane == 0) {
      sm_m[w * GP + g] = m_run[g];
      sm_l[w * GP + g] = l;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * kValuD; e += kValuNW * 64) {
    const int g = e / kValuD;
    const int d = e % kValuD;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kValuNW; ++v) M = fmaxf(M, sm_m[v * GP + g]);
    float o = 0.f;
    if (M != -INFINITY) {
      float lsum = 0.f, osum = 0.f;
#pragma unroll
      for (int v = 0; v < kValuNW; ++v) {
        const float f = fast_exp2(sm_m[v * GP + g] - M);
        lsum += f * sm_l[v * GP + g];
        osum += f * sm_acc[(v * GP + g) * kValuD + d];
      }
      o = osum / lsum;
    }
    const size_t row = static_cast<size_t>(b) * p.num_heads + kvh * G + g;
    if (p.out_bf16)
      static_cast<uint16_t *>(p.out)[row * kValuD + d] = float_to_bf16_bits(o);
    else
      static_cast<float *>(p.out)[row * kValuD + d] = o;
  }
}

template <int BS, int GP>
hipError_t launch_gp(const DecodeParams &p, hipStream_t s) {
  const size_t lds = valu_lds_bytes<GP>(p.tbl_window);
  const int64_t nwg = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads;
  if (nwg > INT32_MAX) return hipErrorInvalidValue;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_valu_kernel<BS, GP>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_valu_kernel<BS, GP>), dim3(static_cast<uint32_t>(nwg)), dim3(kValuNW * 64), lds, s, p);
  return hipGetLastError();
}

template <int BS>
hipError_t launch_bs(const DecodeParams &p, hipStream_t s) {
  if (p.group <= 1) return launch_gp<BS, 1>(p, s);
  if (p.group <= 2) return launch_gp<BS, 2>(p, s);
  if (p.group <= 4) return launch_gp<BS, 4>(p, s);
  if (p.group <= 8) return launch_gp<BS, 8>(p, s);
  return launch_gp<BS, 16>(p, s);
}

}  // namespace

bool decode_valu_applies(const DecodeParams &p, pa_dtype kv_dtype, int head_dim) {
  return kv_dtype == PA_BF16 && head_dim == kValuD && p.group >= 1 && p.group <= 16 && p.partition_size == 0 &&
         p.q_start == nullptr && p.append.slot_mapping == nullptr;
}

hipError_t launch_decode_valu(const DecodeParams &p, int head_dim, int block_size, hipStream_t s) {
  if (head_dim != kValuD || p.group < 1 || p.group > 16) return hipErrorInvalidValue;
  switch (block_size) {
    case 16: return launch_bs<16>(p, s);
    case 32: return launch_bs<32>(p, s);
    case 64: return launch_bs<64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
