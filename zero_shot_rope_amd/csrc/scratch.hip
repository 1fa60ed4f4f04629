// scratch.hip -- the static device scratch of bifocal_decode_noalloc, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation). The decode kernels write their split partials here instead of into a
// caller's workspace; nothing in it needs to start at zero.
#include <mutex>

#include "launch.hpp"

namespace bifocal {

// Split partials of the decode entry point that allocates nothing, for callers that cannot
// allocate. Every device the library runs on holds its own copy of this array until the process
// ends. In host code the name stands for a host-side shadow, not a device address: host code only
// ever uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace bifocal
