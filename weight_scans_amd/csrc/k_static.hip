// k_static.hip -- the scratch memory of gl_scan_bwd_static, the backward
// entry point for callers that cannot allocate (code under graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// The buffer is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is taken once per device with hipGetSymbolAddress and kept; only that
// address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace gls {
namespace {

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace gls
