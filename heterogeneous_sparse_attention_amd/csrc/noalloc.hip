// noalloc.hip - the fixed scratch buffer of hsa_decode_step_noalloc: a file-scope
// device array, one copy per GPU, held until the process ends.
//
// Host code must not pass the array's name to a kernel or a copy: on the host it is
// only a stand-in for the symbol. noalloc_scratch() looks up the array's device
// address once per device, with that device current, and every user takes that
// address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "noalloc.h"

namespace hsa {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;   // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
  }
  *ptr = g_ptr[device];
  return hipSuccess;
}

}  // namespace hsa
