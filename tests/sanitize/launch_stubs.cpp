// Kernel launchers for a host-only build of the library's C ABI layer.
//
// The host-side core (argument validation, the C entry points and the block
// manager) is compiled with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer, without the HIP kernels.  Every launcher here
// reports that no GPU is present, so a call that passes validation returns
// PA_ERR_HIP and computes nothing; the tests run only the calls that
// validation must refuse, and the block manager, which is pure host code.
#include <hip/hip_runtime_api.h>

#include "pa_internal.h"

namespace pa {

hipError_t launch_decode_mfma(const DecodeParams &, pa_dtype, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_f32(const DecodeParams &, int, int, hipStream_t) { return hipErrorNoDevice; }
bool decode_valu_applies(const DecodeParams &, pa_dtype, int) { return false; }
hipError_t launch_decode_valu(const DecodeParams &, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_reduce(const ReduceParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append(const AppendParams &, pa_dtype, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_copy_blocks(const CopyParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_mla_decode(const MlaParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_mla_append(const MlaAppendParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_probe_read(const void *, size_t, int, int, uint32_t *, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}

}  // namespace pa
