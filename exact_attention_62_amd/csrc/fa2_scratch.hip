// Library-owned device scratch for fa2_fwd_splitkv_noalloc: the float32
// partial results of the split-KV pass live in a file-scope device array
// instead of a caller workspace, so that the call allocates nothing.
//
// Host code must never pass `scratch` itself to a kernel: on the host that
// name is only a stand-in for the device variable.  The device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and cached; every later use goes through the cached address.
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa2_internal.h"

static __device__ __align__(256) char scratch[fa2::kScratchBytes];

namespace fa2 {

hipError_t scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa2
