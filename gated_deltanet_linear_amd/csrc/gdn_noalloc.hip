// The scratch of gdn_chunk_fwd_noalloc: a file-scope device array that takes the
// place of the caller's workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Every GPU the library runs on holds its own copy of the array,
// kGdnNoAllocScratchBytes of it, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept, and only that address is ever handed to a kernel.
// Calls on one GPU share its array: calls that overlap in time on one GPU race.
#include <mutex>

#include <hip/hip_runtime.h>

#include "gdn_internal.hpp"

namespace gdn {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace gdn
