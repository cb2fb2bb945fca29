// Device scratch of the no-allocation entry point (bsk_run_noalloc).
//
// The partial states of split units normally go to the caller's float
// workspace.  Callers that cannot allocate get them in this file-scope
// device array instead: it is part of the library's device code, so each
// GPU the library runs on holds its own copy, from the code's load until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device memory, so the device address is looked up once per device
// (with that device current) and cached; only that address is ever handed
// to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/bsk.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = BSK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace bsk {

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace bsk
