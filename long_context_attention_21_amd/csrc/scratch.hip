// scratch.hip -- the device scratch of the allocation-free entry point
// (csa_index_topk_noalloc, for callers that cannot allocate device memory):
// a file-scope device array, of which every GPU holds its own copy for the
// life of the process.  Host code never uses the array's name as an address:
// the address is taken once per device, with that device current, and the
// kernels receive it as their workspace pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace csa {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // per device, taken on the first call there
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace csa
