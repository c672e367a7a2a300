// Scratch memory of the forward entry point that allocates nothing
// (skv_attn_fwd_partial_noalloc).
//
// The array lives in the library's device code object, so every GPU the
// library runs on holds its own copy, at its own address, from the first use
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol): the device address of
// the current device's copy is looked up once per device with
// hipGetSymbolAddress and kept.  Calls on one GPU share its copy, so calls
// that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace skv {
namespace {

__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace skv
