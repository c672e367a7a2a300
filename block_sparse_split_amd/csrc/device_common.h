// Device-side helpers shared by the libsplitkv kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.h"

namespace skv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

__device__ __forceinline__ uint16_t bf16_bits(__bf16 b) { return __builtin_bit_cast(uint16_t, b); }

// The schedule image is read-only for the whole launch.  Reading it through
// the constant address space lets wave-uniform reads become scalar loads:
// a vector load would make the compiler wait on vmcnt, which also counts the
// tile DMA in flight, and drain the staging ring.
typedef const __attribute__((address_space(4))) int32_t* sched_t;

__device__ __forceinline__ sched_t sched_const(const int32_t* p) {
  return reinterpret_cast<sched_t>(reinterpret_cast<uintptr_t>(p));
}

// Draft-key rows a query tile may see: tokens [dtok0, dtok1) of Kd/Vd.
struct QTileSpan {
  int32_t tok0, tok1;    // tokens of the tile (rows / G), clipped to Nq
  int32_t dtok0, dtok1;  // draft tokens of the tile's blocks
};

__device__ __forceinline__ QTileSpan qtile_span(int32_t qt, int32_t G, int32_t nq) {
  QTileSpan s;
  const int32_t tpq = kQTile / G;
  s.tok0 = qt * tpq;
  s.tok1 = min(nq, s.tok0 + tpq);
  s.dtok0 = (s.tok0 / kBlock) * kBlock;
  s.dtok1 = min(nq, ((s.tok1 + kBlock - 1) / kBlock) * kBlock);
  return s;
}

// One key step of an item: either a context tile or up to 64 draft keys.
struct Step {
  int32_t row;     // first global row of K/V (context) or Kd/Vd (draft)
  int32_t base;    // absolute position of key 0 (context) or its draft token
  int32_t n;       // keys in the step (<= 64)
  int32_t draft;   // 1 for draft keys
};

__device__ __forceinline__ Step item_step(sched_t tiles, int32_t s, int32_t n_draft,
                                          int32_t t0, const QTileSpan& sp) {
  Step st;
  if (s < n_draft) {
    st.row = sp.dtok0 + s * kTileK;
    st.base = st.row;
    st.n = min(kTileK, sp.dtok1 - st.row);
    st.draft = 1;
  } else {
    const sched_t t = tiles + (t0 + s - n_draft) * T_WORDS;
    st.row = t[T_ROW];
    st.base = t[T_POS];
    st.n = t[T_LEN];
    st.draft = 0;
  }
  return st;
}

// Visible key range [klo, khi) of one query row inside a step.
__device__ __forceinline__ void step_bounds(const Step& st, int32_t lo, int32_t a, int32_t blk,
                                            int32_t& klo, int32_t& khi) {
  if (st.draft) {
    klo = blk * kBlock - st.base;
    khi = klo + kBlock;
  } else {
    klo = lo - st.base;
    khi = a - st.base;
  }
  klo = max(klo, 0);
  khi = min(khi, st.n);
}

// max / sum of x over lanes l and l ^ 32.  v_permlane32_swap exchanges the
// two 32-lane halves in registers (no LDS round trip); the sum adds the lower
// half's value first in both halves, so both get bit-identical results.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace skv
