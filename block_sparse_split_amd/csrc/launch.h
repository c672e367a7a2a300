// Internal interface between the C entry points and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace skv {

// A kernel's dynamic-LDS limit, raised once per device (the setting lasts
// for the process), so launches do not repeat the runtime call.  One static
// instance per kernel.
struct LdsLimit {
  std::atomic<uint64_t> done{0};  // bit d: set on device d (d < 64)
  hipError_t ensure(const void* fn, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
  }
};

// Bytes at the end of a workspace that hold the per-XCD queue counters of a
// schedule built for per-XCD speeds (forward: 8 words; backward: 8 for dQ,
// then 8 for dK/dV).
constexpr int64_t kXcdCounterBytes = 256;

struct FwdArgs {
  const int32_t* sched;     // device schedule image
  const void* Q;            // [Nq, hq, d]
  const void* K;            // [n_local, hkv, d]
  const void* V;
  const void* Kd;           // [Nq, hkv, d] or null
  const void* Vd;
  void* O;                  // [Nq, hq, d]
  float* LSE;               // [Nq, hq]
  float* ws_O;              // partial slots [n_slots, 256, d] fp32
  float* ws_LSE;            // [n_slots, 256]
  unsigned long long* wg_clock;  // per-workgroup (start, end) stamps, or null
  uint32_t* xcd_count;      // per-XCD queue counters (schedule with per-XCD speeds), or null
  int32_t o_bf16, dtype_bf16;
  int32_t hq, hkv, d, nb, n_local;
  int32_t n_wg, n_split, n_slots;
  float scale;
};

struct BwdArgs {
  const int32_t* sched;
  const void* Q;
  const void* K;
  const void* V;
  const void* Kd;
  const void* Vd;
  const void* O;            // final merged output
  const void* dO;
  const float* LSE;         // final merged LSE (natural log)
  float* dQ;                // [Nq, hq, d] fp32
  void* dK;                 // [n_local, hkv, d]
  void* dV;
  void* dKd;                // [Nq, hkv, d]
  void* dVd;
  float* ws_nD;             // -rowsum(dO * O), [hkv][Nq * G + kStatPad] in query-tile row
                            //   order; padding rows see no key
  float* ws_L2;             // LSE * log2(e) (+inf: no key), same layout
  int32_t* ws_LO;           // first / end context key each row may see (its
  int32_t* ws_HI;           //   anchor block's lo and anchor), same layout
  float* ws_dQ;             // partial slots [n_slots, 256, d]
  int64_t stat_words;       // distance between the -D, L2, LO and HI arrays
  unsigned long long* wg_clock_dq;  // per-workgroup (start, end) stamps, or null
  unsigned long long* wg_clock_kv;
  uint32_t* xcd_count;      // dQ then dK/dV per-XCD queue counters, or null (zeroed by pre)
  uint32_t* kv_front;       // per dK/dV queue: positions claimed (n_wg words, zeroed by pre)
  int32_t grad_bf16, dtype_bf16;
  int32_t hq, hkv, d, nb, n_local;
  int32_t n_wg, n_split, n_slots, with_draft;
  float scale;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// Scratch of skv_attn_fwd_partial_noalloc: a static device array of this
// size; *out gets the current device's copy.
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
hipError_t noalloc_scratch(void** out);
// dQ finalize: out[i] = sum over k < n of parts[k * stride + i], i < elems.
hipError_t launch_dq_finalize(int32_t n, int64_t elems, int64_t stride, const float* parts,
                              void* out, bool out_bf16, hipStream_t s);
hipError_t launch_merge(int32_t n_parts, int64_t rows, int32_t d, const void* O_parts,
                        bool in_bf16, const float* LSE_parts, void* O_out, bool out_bf16,
                        float* LSE_out, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace skv
