// Cache append: write each new token's K and V rows into its slot.
//
// The cache grows by one row per token before attention reads it (page
// "字节跳动 AI Infra (2)", KV-cache question, step-t equations).  Slot s names
// physical block s / block_size at offset s % block_size.  fp32 and bf16
// caches take the source bits unchanged; int8 caches (INT8 KV cache: page
// "字节跳动 AI Infra (2)", optimisation table; page "LLM推理优化", section 1.3)
// take per (token, kv head) the fp16 scale fp16_rne(fp32(max|x| / 127)) and
// codes rint_even(fp32(x / scale)) clamped to [-127, 127], all zero when the
// scale is zero; int4 caches (page "LLM推理优化", section 1.3) the same with
// 7 in place of 127.  The divisions are IEEE fp32 (the compiler's default
// correctly rounded division), so the result is bit-exact.
//
// int4 stores two codes per byte.  A K byte holds two channels of one token
// (one lane's pair, or two neighbouring lanes' codes), so it is written
// whole.  A V byte holds one channel of two neighbouring tokens, which one
// call may write from two work-groups: each nibble is replaced with a pair
// of 32-bit atomic AND / OR operations, so neither write can undo the other.
//
// Cache layout as documented in pa.h (bf16 K tiles store offsets in the
// bit-2/3-exchanged slot order).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Element offsets in the two pools (see the layout in pa.h).
template <int D, int BS, int X>
__device__ __forceinline__ size_t k_off(size_t tile, int o, int d) {
  return ((tile * (D / X) + d / X) * BS + o) * X + d % X;
}
template <int D, int BS, int X>
__device__ __forceinline__ size_t v_off(size_t tile, int o, int d) {
  return ((tile * (BS / X) + o / X) * D + d) * X + o % X;
}

// PER consecutive elements of type E packed in one register-sized value.
template <typename E, int PER>
struct Pack {
  E e[PER];
};

template <typename E, int PER>
__device__ __forceinline__ Pack<E, PER> load_pack(const E *ptr) {
  return *reinterpret_cast<const Pack<E, PER> *>(ptr);
}
template <typename E, int PER>
__device__ __forceinline__ void store_pack(E *ptr, const Pack<E, PER> &v) {
  *reinterpret_cast<Pack<E, PER> *>(ptr) = v;
}

constexpr int kAppendWaves = 4;

// One wavefront per (token, kv head) pair, four pairs per work-group.  Lane
// l owns channels PER*l .. PER*l + PER - 1, which are adjacent in a K tile
// (one store per lane) and X elements apart in a V tile.  The source rows are
// loaded alongside the slot, so the only dependent access is the cache write.
template <int KIND, int D, int BS>  // KIND: 0 fp32, 1 bf16, 2 int8, 3 int4
__global__ __launch_bounds__(kAppendWaves * 64) void append_kernel(AppendParams p) {
  constexpr int PER = D / 64;
  constexpr int X = KIND == 0 ? 4 : (KIND == 1 ? 8 : 16);  // elements per storage vector
  typedef typename std::conditional<KIND == 0, float, uint16_t>::type Src;
  const int lane = threadIdx.x & 63;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * kAppendWaves + (threadIdx.x >> 6);
  if (pair >= static_cast<int64_t>(p.num_tokens) * p.num_kv_heads) return;  // whole wavefront
  const int i = static_cast<int>(pair / p.num_kv_heads);
  const int h = static_cast<int>(pair % p.num_kv_heads);
  const int d0 = PER * lane;
  const int32_t slot = p.slot_mapping[i];
  const size_t src = (static_cast<size_t>(i) * p.num_kv_heads + h) * D + d0;
  const Pack<Src, PER> kk = load_pack<Src, PER>(static_cast<const Src *>(p.key) + src);
  const Pack<Src, PER> vv = load_pack<Src, PER>(static_cast<const Src *>(p.value) + src);
  if (slot < 0 || static_cast<int64_t>(slot) >= static_cast<int64_t>(p.num_blocks) * BS) return;
  const int pb = slot / BS;
  const int o = slot % BS;
  {
    const size_t tile = static_cast<size_t>(pb) * p.num_kv_heads + h;

    if constexpr (KIND <= 1) {
      // bf16 K tiles hold offset o at its bit-2/3-exchanged slot
      const int ks = KIND == 1 ? bf16_k_slot(o) : o;
      Src *kc = static_cast<Src *>(p.k_cache);
      Src *vc = static_cast<Src *>(p.v_cache);
      store_pack<Src, PER>(kc + k_off<D, BS, X>(tile, ks, d0), kk);
#pragma unroll
      for (int k = 0; k < PER; ++k) vc[v_off<D, BS, X>(tile, o, d0 + k)] = vv.e[k];
    } else {
      constexpr float kQmax = KIND == 2 ? 127.0f : 7.0f;
      int8_t *kc = static_cast<int8_t *>(p.k_cache);
      int8_t *vc = static_cast<int8_t *>(p.v_cache);
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const Pack<Src, PER> &row = which == 0 ? kk : vv;
        float xv[PER];
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          xv[k] = bf16_bits_to_float(row.e[k]);
          amax = fmaxf(amax, fabsf(xv[k]));
        }
        amax = wave_max(amax);
        const uint16_t s16 = float_to_half_bits(amax / kQmax);
        const float sf = half_bits_to_float(s16);
        Pack<int8_t, PER> q;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          float qf = 0.f;
          if (sf != 0.f) qf = fminf(fmaxf(rintf(xv[k] / sf), -kQmax), kQmax);
          q.e[k] = static_cast<int8_t>(static_cast<int>(qf));
        }
        if constexpr (KIND == 2) {
          if (which == 0) {
            store_pack<int8_t, PER>(kc + k_off<D, BS, X>(tile, o, d0), q);
          } else {
#pragma unroll
            for (int k = 0; k < PER; ++k) vc[v_off<D, BS, X>(tile, o, d0 + k)] = q.e[k];
          }
        } else if (which == 0) {
          // K: channels 2i, 2i + 1 of this token share byte i of its vector
          uint32_t byte;
          if constexpr (PER == 2) {
            byte = (static_cast<uint32_t>(q.e[0]) & 0xfu) | ((static_cast<uint32_t>(q.e[1]) & 0xfu) << 4);
          } else {
            const int other = __shfl_xor(static_cast<int>(q.e[0]), 1);  // the neighbouring channel
            byte = (static_cast<uint32_t>(q.e[0]) & 0xfu) | ((static_cast<uint32_t>(other) & 0xfu) << 4);
          }
          if (PER == 2 || (lane & 1) == 0) {
            const size_t e = k_off<D, BS, X>(tile, o, d0);  // element index; two per byte
            reinterpret_cast<uint8_t *>(kc)[e / 2] = static_cast<uint8_t>(byte);
          }
        } else {
          // V: channel d's byte holds tokens o & ~1 (low nibble) and o | 1
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const size_t e = v_off<D, BS, X>(tile, o, d0 + k);
            const size_t byte_at = e / 2;
            uint32_t *word = reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(vc) + (byte_at & ~size_t(3)));
            const int shift = 8 * static_cast<int>(byte_at & 3) + 4 * (o & 1);
            atomicAnd(word, ~(0xfu << shift));
            atomicOr(word, (static_cast<uint32_t>(q.e[k]) & 0xfu) << shift);
          }
        }
        if (lane == 0) (which == 0 ? p.k_scale : p.v_scale)[tile * BS + o] = s16;
      }
    }
  }
}

template <int KIND, int D>
hipError_t launch_bs(const AppendParams &p, hipStream_t s) {
  const int64_t pairs = static_cast<int64_t>(p.num_tokens) * p.num_kv_heads;
  const uint32_t nwg = static_cast<uint32_t>((pairs + kAppendWaves - 1) / kAppendWaves);
  const dim3 block(kAppendWaves * 64);
  switch (p.block_size) {
    case 16: hipLaunchKernelGGL((append_kernel<KIND, D, 16>), dim3(nwg), block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((append_kernel<KIND, D, 32>), dim3(nwg), block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((append_kernel<KIND, D, 64>), dim3(nwg), block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_d(const AppendParams &p, hipStream_t s) {
  if (p.head_dim == 128) return launch_bs<KIND, 128>(p, s);
  if (p.head_dim == 64) return launch_bs<KIND, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_append(const AppendParams &p, pa_dtype kv_dtype, hipStream_t s) {
  switch (kv_dtype) {
    case PA_F32: return launch_d<0>(p, s);
    case PA_BF16: return launch_d<1>(p, s);
    case PA_I8: return launch_d<2>(p, s);
    case PA_I4: return launch_d<3>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
