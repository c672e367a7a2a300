// Optional per-kernel timing with HIP events (benchmark support).
//
// When enabled on the calling thread, every kernel the library launches is
// bracketed by two hipEventRecord calls on its launch stream; the pairs are
// kept per kernel name until read.  Disabled (the default), launches are
// plain.
#pragma once
#include <hip/hip_runtime.h>

namespace skv {

bool timing_on();
// Record the start event for `name` on `stream` (no-op when disabled).
void timing_begin(const char* name, hipStream_t stream);
// Record the stop event of the last begun pair (no-op when disabled).
void timing_end(hipStream_t stream);

// Kernels that can stamp each workgroup's start and end.
enum WgClockKernel : int { kClockFwd = 0, kClockDq = 1, kClockKv = 2, kClockKernels = 3 };
// Where kernel `k` launched with n_wg workgroups writes its stamps: null
// when no buffer is set on this thread.  Sets *fits = false (and returns
// null) when the buffer set is too small for n_wg.
unsigned long long* wg_clock_region(int k, int32_t n_wg, bool* fits);

}  // namespace skv

// Launch a kernel, bracketed by timing events when timing is on.
#define SKV_LAUNCH(name, kernel, grid, block, lds, stream, ...)           \
  do {                                                                    \
    ::skv::timing_begin(name, stream);                                    \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);    \
    ::skv::timing_end(stream);                                            \
  } while (0)
