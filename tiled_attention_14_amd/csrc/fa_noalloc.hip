// fa_noalloc.hip — the fixed device scratch behind fa_bwd_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) still need the
// backward pass's workspace (two float32 per query row, plus the float32
// partial dK/dV of sliced GQA groups).  It lives here, in a file-scope device
// array of kNoallocScratchBytes that every GPU the library runs on holds for
// the life of the process.  Host code never passes the array's name to a
// kernel (on the host it names a stand-in, not device memory): the device
// address is looked up once per device with hipGetSymbolAddress and cached.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_kernels.h"

namespace fa {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace fa
