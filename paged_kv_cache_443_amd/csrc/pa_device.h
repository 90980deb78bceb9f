// Device-side helpers shared by the kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// float -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Slot of in-block token offset t on the token axis of a bf16 K tile: bits
// 2 and 3 exchanged, so the two 4-token runs a matrix-core row group takes
// from every 8 tokens sit side by side (one 128-byte line per load).
__host__ __device__ __forceinline__ int bf16_k_slot(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// 2^x on the transcendental unit (inputs here are <= 0 or -inf).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight signed int8 codes (little-endian in lo, hi) -> eight bf16.  Every
// |code| <= 128 has at most 8 significant bits, so the float's upper half is
// the exact bf16.
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = (k < 2) ? lo : hi;
    const int sh = (k & 1) * 16;
    const float f0 = static_cast<float>(static_cast<int8_t>((w >> sh) & 0xffu));
    const float f1 = static_cast<float>(static_cast<int8_t>((w >> (sh + 8)) & 0xffu));
    r[k] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, r);
}

// Eight 4-bit two's-complement codes (nibble k = element k, low nibble
// first) -> eight bf16 values, exactly (|code| <= 8 needs 4 significant bits).
__device__ __forceinline__ bf16x8 i4x8_to_bf16x8(uint32_t w) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // sign-extend nibbles 2k and 2k+1 by shifting each to the top of a word
    const float f0 = static_cast<float>(static_cast<int32_t>(w << (28 - 8 * k)) >> 28);
    const float f1 = static_cast<float>(static_cast<int32_t>(w << (24 - 8 * k)) >> 28);
    r[k] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8, r);
}

}  // namespace pa
