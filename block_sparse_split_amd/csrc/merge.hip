// Exact merge of split partial attention results by their log-sum-exp
// (rit.work blog post on Split-KV, section "Split-KV moves queries, not keys
// and values": the participants reconcile the softmax normalisation and the
// split reproduces single-device attention exactly).
//
// For one row with partials (O_k, LSE_k), M = max_k LSE_k,
// LSE = M + ln sum_k exp(LSE_k - M) and O = sum_k exp(LSE_k - LSE) O_k.
// Partials with LSE_k = -inf weigh zero; a row without a finite LSE_k gets
// O = 0, LSE = -inf.
//
// The merge is HBM-bound (a few flops per byte): each thread owns 8
// consecutive elements of one row (16-byte loads for bf16), rows are
// contiguous, so every wave streams whole rows; partial loads are unrolled
// (sixteen in flight per thread) for memory-level parallelism.
#include "device_common.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Partials are read exactly once: non-temporal loads keep them from
// displacing reusable lines in the caches (about 7 % more HBM bandwidth for
// the 64-way merge on MI355X).
template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  static __device__ __forceinline__ void load(const __bf16* p, float* x) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(__bf16* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f32_to_bf16(x[i]);
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
};

// Merge one row: partial k of this row is at O + k*ostride, L + k*lstride.
// The TPR threads of a row (consecutive lanes, `sub` = 0 .. TPR-1) each own 8
// elements; they first split the partials' LSE values between them for the
// row max and the sum of exp(LSE_k - M), combined by lane shuffles, so the
// statistics take n / TPR dependent loads instead of n.
template <typename Tin, typename Tout, int TPR>
__device__ __forceinline__ void merge_row(int n, const Tin* O, int64_t ostride, const float* L,
                                          int64_t lstride, Tout* out, float* lse_out, int sub) {
  float M = kNegInf;
  for (int k = sub; k < n; k += TPR) M = fmaxf(M, L[k * lstride]);
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (M == kNegInf) {
    Vec8<Tout>::store(out, acc);
    if (sub == 0) *lse_out = kNegInf;
    return;
  }
  float sum = 0.f;
  for (int k = sub; k < n; k += TPR) sum += exp2_fast((L[k * lstride] - M) * kLog2e);
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  const float lse = M + logf(sum);
  const float lse2 = lse * kLog2e;
  constexpr int U = 16;  // partials in flight per thread
  int k = 0;
  for (; k + U <= n; k += U) {
    float x[U][8], w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      w[u] = exp2_fast(L[(k + u) * lstride] * kLog2e - lse2);
      Vec8<Tin>::load(O + (k + u) * ostride, x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = w[u] > 0.f ? fmaf(w[u], x[u][i], acc[i]) : acc[i];
  }
  for (; k < n; ++k) {
    float x[8];
    const float w = exp2_fast(L[k * lstride] * kLog2e - lse2);
    Vec8<Tin>::load(O + k * ostride, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = w > 0.f ? fmaf(w, x[i], acc[i]) : acc[i];
  }
  Vec8<Tout>::store(out, acc);
  if (sub == 0) *lse_out = lse;
}

template <typename Tin, typename Tout, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(int n, int64_t rows, const Tin* O,
                                                         const float* L, Tout* Oo, float* Lo) {
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  // whole rows leave together, so the row's lanes stay complete for the
  // shuffles
  if (row >= rows) return;
  merge_row<Tin, Tout, TPR>(n, O + row * D + c, rows * D, L + row, rows, Oo + row * D + c,
                            Lo + row, threadIdx.x % TPR);
}

// Merge the in-GPU segments of split query tiles from the forward workspace.
template <typename Tout, int D>
__global__ __launch_bounds__(kThreads) void merge_split_kernel(const int32_t* S, const float* wsO,
                                                               const float* wsL, Tout* O,
                                                               float* LSE) {
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  constexpr int BPT = kQTile / RPB;  // blocks per split query tile
  const int sidx = blockIdx.x / BPT;
  const int32_t* rec = S + S[H_OFF_SPLIT] + sidx * S_WORDS;
  const int head = rec[S_HEAD], qt = rec[S_QT], slot0 = rec[S_SLOT0], ns = rec[S_NSLOT];
  const int rloc = (blockIdx.x % BPT) * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  const int G = S[H_G], hq = S[H_HQ], nq = S[H_NB] * kBlock;
  const int rho = qt * kQTile + rloc;
  if (rho >= nq * G) return;
  const int64_t orow = (int64_t)(rho / G) * hq + head * G + rho % G;
  const int64_t prow = (int64_t)slot0 * kQTile + rloc;
  merge_row<float, Tout, TPR>(ns, wsO + prow * D + c, (int64_t)kQTile * D, wsL + prow, kQTile,
                              O + orow * D + c, LSE + orow, threadIdx.x % TPR);
}

template <int D>
hipError_t launch_merge_d(int32_t n, int64_t rows, const void* O, bool in_bf16, const float* L,
                          void* Oo, bool out_bf16, float* Lo, hipStream_t s) {
  constexpr int RPB = kThreads / (D / 8);
  const int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>(blocks)), b(kThreads);
  if (in_bf16 && out_bf16)
    SKV_LAUNCH("merge", (merge_kernel<__bf16, __bf16, D>), g, b, 0, s, n, rows,
                       static_cast<const __bf16*>(O), L, static_cast<__bf16*>(Oo), Lo);
  else if (in_bf16)
    SKV_LAUNCH("merge", (merge_kernel<__bf16, float, D>), g, b, 0, s, n, rows,
                       static_cast<const __bf16*>(O), L, static_cast<float*>(Oo), Lo);
  else if (out_bf16)
    SKV_LAUNCH("merge", (merge_kernel<float, __bf16, D>), g, b, 0, s, n, rows,
                       static_cast<const float*>(O), L, static_cast<__bf16*>(Oo), Lo);
  else
    SKV_LAUNCH("merge", (merge_kernel<float, float, D>), g, b, 0, s, n, rows,
                       static_cast<const float*>(O), L, static_cast<float*>(Oo), Lo);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge_split_d(const FwdArgs& a, hipStream_t s) {
  constexpr int RPB = kThreads / (D / 8);
  const dim3 g(a.n_split * (kQTile / RPB)), b(kThreads);
  if (a.o_bf16)
    SKV_LAUNCH("merge_split", (merge_split_kernel<__bf16, D>), g, b, 0, s, a.sched, a.ws_O, a.ws_LSE,
                       static_cast<__bf16*>(a.O), a.LSE);
  else
    SKV_LAUNCH("merge_split", (merge_split_kernel<float, D>), g, b, 0, s, a.sched, a.ws_O, a.ws_LSE,
                       static_cast<float*>(a.O), a.LSE);
  return hipGetLastError();
}

// dQ finalize: the sum of n fp32 dQ shares (one per shard whose keys the
// queries saw), converted to the output type.  HBM-bound like the merge:
// each thread owns 8 consecutive elements and adds the shares in index
// order, so the bits do not depend on the launch shape.  The last thread
// of a ragged tail goes element by element.
__device__ __forceinline__ void store1(float* p, float x) { *p = x; }
__device__ __forceinline__ void store1(__bf16* p, float x) { *p = f32_to_bf16(x); }

template <typename TO>
__global__ __launch_bounds__(kThreads) void dq_finalize_kernel(int32_t n, int64_t elems,
                                                               int64_t stride,
                                                               const float* __restrict__ parts,
                                                               TO* __restrict__ out) {
  const int64_t i = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 8;
  if (i >= elems) return;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if (i + 8 <= elems) {
#pragma unroll 4
    for (int32_t k = 0; k < n; ++k) {
      float x[8];
      Vec8<float>::load(parts + k * stride + i, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += x[j];
    }
    Vec8<TO>::store(out + i, acc);
  } else {
    for (int64_t j = 0; j < elems - i; ++j) {
      float a = 0.f;
      for (int32_t k = 0; k < n; ++k) a += parts[k * stride + i + j];
      store1(out + i + j, a);
    }
  }
}

}  // namespace

hipError_t launch_merge(int32_t n, int64_t rows, int32_t d, const void* O, bool in_bf16,
                        const float* L, void* Oo, bool out_bf16, float* Lo, hipStream_t s) {
  return d == 128 ? launch_merge_d<128>(n, rows, O, in_bf16, L, Oo, out_bf16, Lo, s)
                  : launch_merge_d<64>(n, rows, O, in_bf16, L, Oo, out_bf16, Lo, s);
}

hipError_t launch_merge_split(const FwdArgs& a, hipStream_t s) {
  return a.d == 128 ? launch_merge_split_d<128>(a, s) : launch_merge_split_d<64>(a, s);
}

hipError_t launch_dq_finalize(int32_t n, int64_t elems, int64_t stride, const float* parts,
                              void* out, bool out_bf16, hipStream_t s) {
  const int64_t blocks = (elems + 8 * kThreads - 1) / (8 * kThreads);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(blocks)), b(kThreads);
  if (out_bf16)
    SKV_LAUNCH("dq_finalize", dq_finalize_kernel<__bf16>, g, b, 0, s, n, elems, stride, parts,
               static_cast<__bf16*>(out));
  else
    SKV_LAUNCH("dq_finalize", dq_finalize_kernel<float>, g, b, 0, s, n, elems, stride, parts,
               static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace skv
