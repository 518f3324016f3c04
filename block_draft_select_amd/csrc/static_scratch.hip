// Scratch memory of dflash_cycle_static: one file-scope device array per GPU,
// so that the cycle can run without any allocation (for callers that cannot
// call hipMalloc: code under HIP graph capture, tight serving loops).
//
// In host code the array's name is only a host-side stand-in; its device
// address is looked up once per device, with that device current, through
// hipGetSymbolAddress and kept here.  Kernels receive that address as their
// workspace pointer, exactly as they receive a caller's workspace.  Every
// call on one GPU shares that GPU's array: calls that overlap in time on one
// GPU race.  The workspace contents need no initialisation, so nothing is
// cleared between calls.
#include <mutex>

#include "internal.hpp"

namespace dfk {

namespace {

static __device__ __align__(256) unsigned char scratch[DFLASH_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** out, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  *bytes = DFLASH_STATIC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace dfk
