// The library's one fixed scratch buffer, for the entry point that must not
// allocate (callers under stream capture, tight serving loops, harnesses
// that forbid device allocation).
//
// `scratch` is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is looked up once per device (with that device current) and cached;
// kernels are given that address, never the name.
#include <mutex>

#include "kvsel_internal.hpp"

static __device__ __align__(256) unsigned char scratch[kvsel::kNoAllocScratchBytes];

namespace kvsel {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
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
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace kvsel
