// One wavefront writes one (token, kv head) row of K and V into its cache
// slot: the body of the cache append, shared by the append kernel and the
// fused append + decode.  What is stored is documented in pa_append.hip and
// pa.h (bf16 K tiles store offsets in the bit-2/3-exchanged slot order; int8
// and int4 caches store symmetric codes and an fp16 scale per row).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace append_row_detail {

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

}  // namespace append_row_detail

// The source rows of one (token, kv head), held by one wavefront: lane l
// owns channels PER*l .. PER*l + PER - 1 of K and of V.
template <int KIND, int D>  // KIND: 0 fp32, 1 bf16, 2 int8, 3 int4
struct AppendRowData {
  typedef typename std::conditional<KIND == 0, float, uint16_t>::type Src;
  append_row_detail::Pack<Src, D / 64> k, v;
  int32_t slot;
};

// Load token i's K and V rows for kv head h and its slot (independent loads).
template <int KIND, int D>
__device__ __forceinline__ AppendRowData<KIND, D> load_append_row(const AppendParams &p, int i, int h, int lane) {
  using namespace append_row_detail;
  using Src = typename AppendRowData<KIND, D>::Src;
  constexpr int PER = D / 64;
  AppendRowData<KIND, D> r;
  r.slot = p.slot_mapping[i];
  const size_t src = (static_cast<size_t>(i) * p.num_kv_heads + h) * D + PER * lane;
  r.k = load_pack<Src, PER>(static_cast<const Src *>(p.key) + src);
  r.v = load_pack<Src, PER>(static_cast<const Src *>(p.value) + src);
  return r;
}

// Symmetric quantisation of a loaded row (int8: KIND 2, qmax 127; int4:
// KIND 3, qmax 7): per row, the fp16 scale fp16_rne(fp32(max|x| / qmax)) and
// codes rint_even(fp32(x / scale)) clamped to [-qmax, qmax], all 0 when the
// scale is 0.  Lane l gets the codes of its channels.  The whole wavefront
// must call it (the maximum is taken over the wavefront).
template <int PER>
struct QuantRow {
  append_row_detail::Pack<int8_t, PER> k, v;
  uint16_t sk, sv;
};

template <int KIND, int D>
__device__ __forceinline__ QuantRow<D / 64> quantize_row(const AppendRowData<KIND, D> &r) {
  using namespace append_row_detail;
  constexpr int PER = D / 64;
  constexpr float kQmax = KIND == 2 ? 127.0f : 7.0f;
  QuantRow<PER> out;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const auto &row = which == 0 ? r.k : r.v;
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
    (which == 0 ? out.k : out.v) = q;
    (which == 0 ? out.sk : out.sv) = s16;
  }
  return out;
}

// Write loaded rows into their slot of kv head h.  Lane l's channels are
// adjacent in a K tile (one store per lane) and X elements apart in a V tile.
// The whole wavefront must call it (int8 / int4 reduce over it).
template <int KIND, int D, int BS>
__device__ __forceinline__ void store_append_row(const AppendParams &p, const AppendRowData<KIND, D> &r, int h,
                                                 int lane) {
  using namespace append_row_detail;
  using Src = typename AppendRowData<KIND, D>::Src;
  constexpr int PER = D / 64;
  constexpr int X = KIND == 0 ? 4 : (KIND == 1 ? 8 : 16);  // elements per storage vector
  const int d0 = PER * lane;
  const int32_t slot = r.slot;
  const Pack<Src, PER> &kk = r.k;
  const Pack<Src, PER> &vv = r.v;
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
      int8_t *kc = static_cast<int8_t *>(p.k_cache);
      int8_t *vc = static_cast<int8_t *>(p.v_cache);
      const QuantRow<PER> qr = quantize_row<KIND, D>(r);
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const Pack<int8_t, PER> &q = which == 0 ? qr.k : qr.v;
        const uint16_t s16 = which == 0 ? qr.sk : qr.sv;
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

// Token i, kv head h, on the calling wavefront (lane = its lane id): the
// rows and the slot are loaded together, so the only dependent access is the
// cache write.  The whole wavefront must call it.
template <int KIND, int D, int BS>
__device__ __forceinline__ void append_row(const AppendParams &p, int i, int h, int lane) {
  store_append_row<KIND, D, BS>(p, load_append_row<KIND, D>(p, i, h, lane), h, lane);
}

}  // namespace pa
