// The library's own device scratch for pa_decode_split_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get a KV-split decode
// whose partials live here instead of in a caller workspace.  The array is a
// file-scope __device__ object: every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code the name
// `scratch` is only a host-side stand-in; the device address is looked up
// once per device with hipGetSymbolAddress (which allocates nothing) and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pa {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current: this device's copy
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pa
