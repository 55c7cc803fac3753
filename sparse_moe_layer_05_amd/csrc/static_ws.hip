// Library-owned workspace for callers that cannot allocate device memory: one file-scope device
// array per GPU, used by moe_layer_forward_static in place of a caller workspace.
//
// In host code `scratch` names a host-side stand-in, not the device memory: a kernel handed that
// name would fault. Its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is ever passed on.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.hpp"

namespace moe {
namespace {

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
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
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace moe
