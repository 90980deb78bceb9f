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

// Work-group barrier for LDS hand-offs inside a streaming loop.  It waits for
// this wavefront's LDS operations only (lgkmcnt) before s_barrier, not for
// its global loads still in flight, which __syncthreads() (a work-group
// fence) would drain: a prefetch issued before the barrier stays in flight
// across it.  The memory clobber keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Maximum of v over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four
// 16-lane rows of the wavefront; a matrix-core output row's lane groups j).
// gfx950's row-swap instructions exchange the halves (permlane32_swap) and
// then the odd and even rows (permlane16_swap) of a register in the vector
// ALU; with both operands the same value, each lane gets its partner's value
// in one of the two results.  An exact maximum, so the order does not matter;
// no LDS permute round trip.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

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

// Eight 4-bit two's-complement codes (nibble e = element e, low nibble
// first) -> eight bf16 values 136 + code, in the element order
// 0, 2, 4, 6, 1, 3, 5, 7.  With the codes in offset binary (code + 8 in
// 0..15), bf16 0x4300 | (code + 8) is exactly 128 + code + 8: one byte
// permute under the constant 0x43 per two values, no conversion.  The
// caller removes the 136 offset and lays the other operand out in the same
// element order.
constexpr float kInt4Bias = 136.f;

__device__ __forceinline__ bf16x8 i4x8_to_bf16x8_biased(uint32_t w) {
  const uint32_t t = w ^ 0x88888888u;         // offset binary in every nibble
  const uint32_t lo = t & 0x0f0f0f0fu;         // bytes: elements 0, 2, 4, 6
  const uint32_t hi = (t >> 4) & 0x0f0f0f0fu;  // bytes: elements 1, 3, 5, 7
  const uint32_t c = 0x43434343u;
  u32x4 r;
  // result byte i takes selector byte i: 0-3 pick the second operand's bytes, 4-7 the first's
  r[0] = __builtin_amdgcn_perm(c, lo, 0x04010400u);  // elements 0, 2
  r[1] = __builtin_amdgcn_perm(c, lo, 0x04030402u);  // elements 4, 6
  r[2] = __builtin_amdgcn_perm(c, hi, 0x04010400u);  // elements 1, 3
  r[3] = __builtin_amdgcn_perm(c, hi, 0x04030402u);  // elements 5, 7
  return __builtin_bit_cast(bf16x8, r);
}

// Slot s of an i4x8_to_bf16x8_biased result holds element kEvenFirst[s].
__device__ constexpr int kEvenFirst[8] = {0, 2, 4, 6, 1, 3, 5, 7};

}  // namespace pa
