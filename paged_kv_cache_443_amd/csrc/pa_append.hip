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

#include "pa_append_row.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kAppendWaves = 4;

// One wavefront per (token, kv head) pair, four pairs per work-group.
template <int KIND, int D, int BS>  // KIND: 0 fp32, 1 bf16, 2 int8, 3 int4
__global__ __launch_bounds__(kAppendWaves * 64) void append_kernel(AppendParams p) {
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * kAppendWaves + (threadIdx.x >> 6);
  if (pair >= static_cast<int64_t>(p.num_tokens) * p.num_kv_heads) return;  // whole wavefront
  append_row<KIND, D, BS>(p, static_cast<int>(pair / p.num_kv_heads), static_cast<int>(pair % p.num_kv_heads),
                          threadIdx.x & 63);
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
