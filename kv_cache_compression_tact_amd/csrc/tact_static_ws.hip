// Library-owned workspace of tact_roundtrip_noalloc, for callers that cannot
// allocate device memory.  The array lives in the code object: every GPU the
// library runs on holds its own copy, at its own address, from the module's
// load on that GPU until the process ends.  In host code its name is only a
// stand-in for the symbol, so its device address is looked up once per GPU
// (with that GPU current) and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tact_internal.h"

namespace tact {

static __device__ __align__(256) unsigned char scratch[TACT_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of each GPU's copy
}  // namespace

hipError_t static_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tact
