// Per-kernel timing with HIP events; see timing.h and the skv_timing_*
// entry points in splitkv.h.
#include "timing.h"

#include <cstring>
#include <string>
#include <vector>

#include "splitkv.h"

namespace skv {
namespace {

struct Pair {
  std::string name;
  hipEvent_t start = nullptr, stop = nullptr;
};

struct State {
  bool on = false;
  std::vector<Pair> pairs;
  std::vector<hipEvent_t> pool;
  // results after a read
  std::vector<std::string> names;
  std::vector<long long> launches;
  std::vector<double> ms;
  std::string err;
};

thread_local State g_state;

// caller's buffer for per-workgroup clock stamps (device memory)
thread_local unsigned long long* g_clock = nullptr;
thread_local int64_t g_clock_bytes = 0;

hipEvent_t get_event() {
  State& s = g_state;
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool timing_on() { return g_state.on; }

unsigned long long* wg_clock_region(int k, int32_t n_wg, bool* fits) {
  *fits = true;
  if (!g_clock) return nullptr;
  if (g_clock_bytes < int64_t(kClockKernels) * n_wg * 32) {
    *fits = false;
    return nullptr;
  }
  return g_clock + int64_t(k) * n_wg * 4;
}

void timing_begin(const char* name, hipStream_t stream) {
  State& s = g_state;
  if (!s.on) return;
  Pair p;
  p.name = name;
  p.start = get_event();
  p.stop = get_event();
  if (p.start) (void)hipEventRecord(p.start, stream);
  s.pairs.push_back(p);
}

void timing_end(hipStream_t stream) {
  State& s = g_state;
  if (!s.on || s.pairs.empty()) return;
  if (s.pairs.back().stop) (void)hipEventRecord(s.pairs.back().stop, stream);
}

}  // namespace skv

extern "C" {

skv_status skv_timing_wg_clock(void* buffer, int64_t bytes) {
  if (buffer && (bytes < 0 || reinterpret_cast<uintptr_t>(buffer) % 8 != 0))
    return SKV_ERR_INVALID_ARG;
  if (buffer) {
    // the kernels store to it: refuse anything but device (or managed) memory
    hipPointerAttribute_t attr{};
    const hipError_t e = hipPointerGetAttributes(&attr, buffer);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // leave no error for a later launch check to find
      return SKV_ERR_INVALID_ARG;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
      return SKV_ERR_INVALID_ARG;
  }
  skv::g_clock = static_cast<unsigned long long*>(buffer);
  skv::g_clock_bytes = buffer ? bytes : 0;
  return SKV_OK;
}

skv_status skv_timing_enable(int32_t on) {
  skv::g_state.on = on != 0;
  return SKV_OK;
}

skv_status skv_timing_collect(int32_t* n_kernels) {
  using namespace skv;
  State& s = g_state;
  s.names.clear();
  s.launches.clear();
  s.ms.clear();
  for (Pair& p : s.pairs) {
    float t = 0.f;
    if (!p.start || !p.stop || hipEventSynchronize(p.stop) != hipSuccess ||
        hipEventElapsedTime(&t, p.start, p.stop) != hipSuccess)
      return SKV_ERR_HIP;
    size_t k = 0;
    while (k < s.names.size() && s.names[k] != p.name) ++k;
    if (k == s.names.size()) {
      s.names.push_back(p.name);
      s.launches.push_back(0);
      s.ms.push_back(0.0);
    }
    s.launches[k] += 1;
    s.ms[k] += t;
    s.pool.push_back(p.start);
    s.pool.push_back(p.stop);
  }
  s.pairs.clear();
  if (n_kernels) *n_kernels = int32_t(s.names.size());
  return SKV_OK;
}

skv_status skv_timing_result(int32_t k, char* name, int32_t name_cap, int64_t* launches,
                             double* total_ms) {
  using namespace skv;
  State& s = g_state;
  if (k < 0 || size_t(k) >= s.names.size() || !name || name_cap < 1)
    return SKV_ERR_INVALID_ARG;
  std::strncpy(name, s.names[k].c_str(), size_t(name_cap) - 1);
  name[name_cap - 1] = 0;
  if (launches) *launches = s.launches[k];
  if (total_ms) *total_ms = s.ms[k];
  return SKV_OK;
}

}  // extern "C"
