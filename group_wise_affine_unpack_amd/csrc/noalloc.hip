// The fixed scratch array of qmm_affine_noalloc, the one entry point that
// allocates no device memory.  Its kernels take the array's device address,
// looked up here once per device (with that device current) by
// hipGetSymbolAddress: in host code the name `scratch` is only a host-side
// stand-in and must never be passed to a kernel.  Each device holds its own
// copy of the array, from the library's loading until the process ends.
#include <mutex>

#include "../../include/qaff.h"
#include "common.h"

namespace qaff {
namespace {

constexpr size_t kScratchBytes = size_t(QAFF_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = kScratchBytes;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace qaff
