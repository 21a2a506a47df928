// Library-owned scratch memory for the no-allocation GEMM entry point.
//
// Some callers cannot allocate device memory at call time (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc). For
// them inv_gemm_noalloc keeps the GEMM's partial sums (leaf groups or rank
// partials, fp32) in a file-scope device array of fixed size instead of a
// caller workspace. Every GPU the library runs on holds its own copy of the
// array until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device
// address. Its address on a device is looked up once per device, with that
// device current, by hipGetSymbolAddress; host code only ever passes that
// looked-up pointer to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace inv {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t scratch_device_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      // device `dev` is current: this returns its copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace inv
