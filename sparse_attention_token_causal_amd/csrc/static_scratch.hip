// Fixed device scratch for the entry point that allocates nothing
// (idx_score_topk_static).  The array is a file-scope device symbol: every
// GPU the library runs on holds its own copy, at its own address, until the
// process ends.  Host code never passes the symbol's name to a kernel (in
// host code it only names a host-side stand-in); it resolves the device
// address once per device with hipGetSymbolAddress and passes that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace idx {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch_ptr(void** out) {
  int dev = -1;
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
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace idx
