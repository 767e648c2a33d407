// Scratch memory of the allocation-free whole-block call (moe_forward_noalloc):
// a fixed device array in the library's code object instead of a caller
// workspace, for callers that cannot allocate (code under graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends. Its address on a device comes from hipGetSymbolAddress, taken
// once per device with that device current; host code only ever passes that
// address on (the array's name on the host is a stand-in, not device memory).
#include <mutex>

#include "common.hpp"

namespace moe {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace moe
