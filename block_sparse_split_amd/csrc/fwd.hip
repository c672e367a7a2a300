// Forward partial attention of the draft queries over one key shard (gfx950).
//
// What is computed (rit.work blog post on Split-KV, section "Split-KV moves
// queries, not keys and values"): every participant computes, for the whole
// draft-query set, the attention over its own keys and reports the output
// together with the softmax normaliser, so that the parts can later be
// combined exactly.  Mask: anchor block i sees context keys
// lo_i <= j < a_i plus its own 16 draft keys.
//
// Work decomposition.  A work item is (kv head g, 256-row query tile, run of
// 64-key tiles); items were placed on persistent workgroups by LPT on the
// host.  A query tile holds the rows (token, head) of the G query heads that
// share kv head g, token-major, so the rows of one anchor block are adjacent
// and share one mask bound.  Four waves per workgroup each own 64 rows (two
// 32-query MFMA columns blocks).
//
// Per 64-key step, each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T held in registers),
// so every lane owns one query column: the softmax max/sum over keys is a
// per-lane reduction plus one exchange with lane ^ 32.  P^T is rounded to
// bf16 in place and feeds O^T += V^T P^T directly as the B operand; V is
// staged transposed in LDS (keys of a 16-key group permuted to match the
// accumulator layout of S^T), so no register transpose is needed.  The
// online softmax works in base 2 with the scale folded into one FMA and
// rescales O only when the running maximum grows by more than 2^8, which is
// exact (the same maximum is used for O and for the sum).  K/V tiles are
// double-buffered in LDS: the next step's global loads are in flight while
// the current step computes.  Tiles that straddle an anchor bound are masked
// per element; fully visible tiles skip the mask, invisible ones skip the
// MFMAs.
#include "device_common.h"
#include "launch.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 2;             // 32-query column blocks per wave
constexpr int kKB = kTileK / 32;   // 32-key blocks per step

template <int D>
struct Bf16Lds {
  static constexpr int kPitch = D + 8;        // K row pitch (elements)
  static constexpr int vPitch = kTileK + 8;   // V^T row pitch (elements)
  static constexpr int kElems = kTileK * kPitch;
  static constexpr int vElems = D * vPitch;
  static constexpr int bufElems = kElems + vElems;
  static constexpr int bytes = 2 * bufElems * 2;
};

template <int D>
struct StepRegs {
  static constexpr int NK = kTileK * D / 8 / kThreads;
  uint4 k[NK];
  uint4 v[4];
};

__device__ __forceinline__ uint4 ld16(const __bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int D>
__device__ __forceinline__ void load_step(StepRegs<D>& r, const __bf16* Kg, const __bf16* Vg,
                                          const Step& st, int head, int hkv, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < StepRegs<D>::NK; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / CPR, col = (c % CPR) * 8;
    r.k[i] = row < st.n ? ld16(Kg + ((int64_t)(st.row + row) * hkv + head) * D + col)
                        : make_uint4(0, 0, 0, 0);
  }
  if (tid < (kTileK / 4) * CPR) {
    const int m = tid / CPR, dr = tid % CPR;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = 4 * m + j;
      r.v[j] = key < st.n ? ld16(Vg + ((int64_t)(st.row + key) * hkv + head) * D + dr * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t half_of(const uint4& u, int e) {
  const uint32_t word = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

template <int D>
__device__ __forceinline__ void store_step(const StepRegs<D>& r, __bf16* buf, int tid) {
  using L = Bf16Lds<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < StepRegs<D>::NK; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / CPR, col = (c % CPR) * 8;
    *reinterpret_cast<uint4*>(buf + row * L::kPitch + col) = r.k[i];
  }
  if (tid < (kTileK / 4) * CPR) {
    const int m = tid / CPR, dr = tid % CPR;
    // keys 4m..4m+3 land at a permuted position inside their 16-key group:
    // sub-group 0,1,2,3 -> offset 0,8,4,12 (matches the S^T accumulator)
    const int pos = 16 * (m >> 2) + ((m & 1) ? 8 : 0) + ((m & 2) ? 4 : 0);
    __bf16* vt = buf + L::kElems;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w;
      w.x = half_of(r.v[0], e) | (half_of(r.v[1], e) << 16);
      w.y = half_of(r.v[2], e) | (half_of(r.v[3], e) << 16);
      *reinterpret_cast<uint2*>(vt + (dr * 8 + e) * L::vPitch + pos) = w;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using L = Bf16Lds<D>;
  extern __shared__ __align__(16) char smem_raw[];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);
  const int32_t* S = a.sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int nq = nb * kBlock, rows_per_head = nq * G;
  const int32_t* anchors = S + S[H_OFF_ANCHORS];
  const int32_t* los = S + S[H_OFF_LO];
  const int32_t* tiles = S + S[H_OFF_TILES];
  const int32_t* items = S + S[H_OFF_ITEMS];
  const int32_t* queue = S + S[H_OFF_QUEUE];
  const int qbeg = S[S[H_OFF_QOFF] + blockIdx.x], qend = S[S[H_OFF_QOFF] + blockIdx.x + 1];
  const float c = a.scale * kLog2e;
  const __bf16* Qg = static_cast<const __bf16*>(a.Q);

  for (int qi = qbeg; qi < qend; ++qi) {
    const int32_t* it = items + queue[qi] * I_WORDS;
    const int head = it[I_HEAD], qt = it[I_QT], t0 = it[I_T0], t1 = it[I_T1];
    const int slot = it[I_SLOT], flags = it[I_FLAGS];
    const QTileSpan sp = qtile_span(qt, G, nq);
    const int n_draft = (flags & kItemDraft) ? (sp.dtok1 - sp.dtok0 + kTileK - 1) / kTileK : 0;
    const int n_steps = n_draft + (t1 - t0);

    int rloc[kQB], tok[kQB], qh[kQB], blk[kQB], lo_[kQB], an[kQB];
    bool valid[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      rloc[qb] = wave * 64 + qb * 32 + l32;
      const int rho = qt * kQTile + rloc[qb];
      valid[qb] = rho < rows_per_head;
      tok[qb] = valid[qb] ? rho / G : 0;
      qh[qb] = head * G + (valid[qb] ? rho % G : 0);
      blk[qb] = tok[qb] / kBlock;
      lo_[qb] = valid[qb] ? los[blk[qb]] : 0;
      an[qb] = valid[qb] ? anchors[blk[qb]] : 0;
    }
    bf16x8 qf[kQB][D / 16];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const __bf16* qrow = Qg + ((int64_t)tok[qb] * hq + qh[qb]) * D + 8 * h32;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        uint4 u = valid[qb] ? ld16(qrow + 16 * t) : make_uint4(0, 0, 0, 0);
        qf[qb][t] = __builtin_bit_cast(bf16x8, u);
      }
    }
    f32x16 o[kQB][D / 32];
    float m_used[kQB], l[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      m_used[qb] = kNegInf;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    }

    StepRegs<D> regs;
    if (n_steps > 0) {
      const Step st = item_step(tiles, 0, n_draft, t0, sp);
      const __bf16* Kg = static_cast<const __bf16*>(st.draft ? a.Kd : a.K);
      const __bf16* Vg = static_cast<const __bf16*>(st.draft ? a.Vd : a.V);
      load_step<D>(regs, Kg, Vg, st, head, hkv, tid);
      store_step<D>(regs, smem, tid);
    }
    __syncthreads();
    for (int s = 0; s < n_steps; ++s) {
      const Step st = item_step(tiles, s, n_draft, t0, sp);
      if (s + 1 < n_steps) {
        const Step nx = item_step(tiles, s + 1, n_draft, t0, sp);
        const __bf16* Kg = static_cast<const __bf16*>(nx.draft ? a.Kd : a.K);
        const __bf16* Vg = static_cast<const __bf16*>(nx.draft ? a.Vd : a.V);
        load_step<D>(regs, Kg, Vg, nx, head, hkv, tid);
      }
      const __bf16* Kl = smem + (s & 1) * L::bufElems;
      const __bf16* Vl = Kl + L::kElems;
      int klo[kQB], khi[kQB];
      bool lane_full = true, lane_any = false;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        if (valid[qb]) {
          step_bounds(st, lo_[qb], an[qb], blk[qb], klo[qb], khi[qb]);
          lane_full = lane_full && klo[qb] <= 0 && khi[qb] >= kTileK;
          lane_any = lane_any || klo[qb] < khi[qb];
        } else {
          klo[qb] = 0;
          khi[qb] = kTileK;
        }
      }
      if (__any(lane_any)) {
        const bool wave_full = __all(lane_full);
        f32x16 sacc[kKB][kQB];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
                Kl + (kb * 32 + l32) * L::kPitch + 16 * t + 8 * h32);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
              sacc[kb][qb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][t], sacc[kb][qb], 0, 0, 0);
          }
        }
        if (!wave_full) {
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kappa = 32 * kb + 8 * (r >> 2) + 4 * h32 + (r & 3);
#pragma unroll
              for (int qb = 0; qb < kQB; ++qb)
                if (kappa < klo[qb] || kappa >= khi[qb]) sacc[kb][qb][r] = kNegInf;
            }
        }
        bf16x8 pf[kQB][kKB][2];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          float mx = kNegInf;
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mt = mx * c;
          const bool need = mt > m_used[qb] + 8.0f;
          if (__any(need)) {
            const float alpha = need ? exp2_fast(m_used[qb] - mt) : 1.0f;
            l[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[qb][db] *= alpha;
            if (need) m_used[qb] = mt;
          }
          const float msub = m_used[qb] == kNegInf ? 0.f : m_used[qb];
          float ls = 0.f;
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = exp2_fast(fmaf(sacc[kb][qb][r], c, -msub));
              ls += p;
              pf[qb][kb][r >> 3][r & 7] = f32_to_bf16(p);
            }
          l[qb] += ls;
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                  Vl + (db * 32 + l32) * L::vPitch + kb * 32 + t2 * 16 + 8 * h32);
#pragma unroll
              for (int qb = 0; qb < kQB; ++qb)
                o[qb][db] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][t2], o[qb][db], 0, 0, 0);
            }
      }
      if (s + 1 < n_steps) store_step<D>(regs, smem + ((s + 1) & 1) * L::bufElems, tid);
      __syncthreads();
    }

    // Epilogue: normalise, write O and the natural-log LSE (or a partial).
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float lt = l[qb] + __shfl_xor(l[qb], 32);
      if (!valid[qb]) continue;
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const float lse = lt > 0.f ? (m_used[qb] + log2f(lt)) * kLn2 : kNegInf;
      if (slot < 0) {
        const int64_t row = (int64_t)tok[qb] * hq + qh[qb];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * h32;
            if (a.o_bf16) {
              bf16x4 w;
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(o[qb][db][4 * j + i] * inv);
              *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.O) + row * D + d0) = w;
            } else {
              f32x4 w;
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = o[qb][db][4 * j + i] * inv;
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.O) + row * D + d0) = w;
            }
          }
        if (h32 == 0) a.LSE[row] = lse;
      } else {
        const int64_t prow = (int64_t)slot * kQTile + rloc[qb];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * h32;
            f32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = o[qb][db][4 * j + i] * inv;
            *reinterpret_cast<f32x4*>(a.ws_O + prow * D + d0) = w;
          }
        if (h32 == 0) a.ws_LSE[prow] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: same decomposition with v_mfma_f32_32x32x2_f32 (exact fp32
// products, fp32 P).  K and V stay in natural layout in LDS; one step is
// loaded, then computed (no double buffering: the fp32 path serves small
// problems).
template <int D>
struct F32Lds {
  static constexpr int kPitch = D + 4;
  static constexpr int elems = kTileK * kPitch;
  static constexpr int bytes = 2 * elems * 4;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(FwdArgs a) {
  using L = F32Lds<D>;
  extern __shared__ __align__(16) char smem_raw[];
  float* Kl = reinterpret_cast<float*>(smem_raw);
  float* Vl = Kl + L::elems;
  const int32_t* S = a.sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int nq = nb * kBlock, rows_per_head = nq * G;
  const int32_t* anchors = S + S[H_OFF_ANCHORS];
  const int32_t* los = S + S[H_OFF_LO];
  const int32_t* tiles = S + S[H_OFF_TILES];
  const int32_t* items = S + S[H_OFF_ITEMS];
  const int32_t* queue = S + S[H_OFF_QUEUE];
  const int qbeg = S[S[H_OFF_QOFF] + blockIdx.x], qend = S[S[H_OFF_QOFF] + blockIdx.x + 1];
  const float c = a.scale * kLog2e;
  const float* Qg = static_cast<const float*>(a.Q);

  for (int qi = qbeg; qi < qend; ++qi) {
    const int32_t* it = items + queue[qi] * I_WORDS;
    const int head = it[I_HEAD], qt = it[I_QT], t0 = it[I_T0], t1 = it[I_T1];
    const int slot = it[I_SLOT], flags = it[I_FLAGS];
    const QTileSpan sp = qtile_span(qt, G, nq);
    const int n_draft = (flags & kItemDraft) ? (sp.dtok1 - sp.dtok0 + kTileK - 1) / kTileK : 0;
    const int n_steps = n_draft + (t1 - t0);
    int rloc[kQB], tok[kQB], qh[kQB], blk[kQB], lo_[kQB], an[kQB];
    bool valid[kQB];
    float qf[kQB][D / 2];
    f32x16 o[kQB][D / 32];
    float m_used[kQB], l[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      rloc[qb] = wave * 64 + qb * 32 + l32;
      const int rho = qt * kQTile + rloc[qb];
      valid[qb] = rho < rows_per_head;
      tok[qb] = valid[qb] ? rho / G : 0;
      qh[qb] = head * G + (valid[qb] ? rho % G : 0);
      blk[qb] = tok[qb] / kBlock;
      lo_[qb] = valid[qb] ? los[blk[qb]] : 0;
      an[qb] = valid[qb] ? anchors[blk[qb]] : 0;
      const float* qrow = Qg + ((int64_t)tok[qb] * hq + qh[qb]) * D;
#pragma unroll
      for (int t = 0; t < D / 2; ++t) qf[qb][t] = valid[qb] ? qrow[2 * t + h32] : 0.f;
      m_used[qb] = kNegInf;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    }
    for (int s = 0; s < n_steps; ++s) {
      const Step st = item_step(tiles, s, n_draft, t0, sp);
      const float* Kg = static_cast<const float*>(st.draft ? a.Kd : a.K);
      const float* Vg = static_cast<const float*>(st.draft ? a.Vd : a.V);
      __syncthreads();
      for (int e = tid; e < kTileK * D / 4; e += kThreads) {
        const int row = e / (D / 4), col = (e % (D / 4)) * 4;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (row < st.n) {
          const int64_t off = ((int64_t)(st.row + row) * hkv + head) * D + col;
          kv = *reinterpret_cast<const float4*>(Kg + off);
          vv = *reinterpret_cast<const float4*>(Vg + off);
        }
        *reinterpret_cast<float4*>(Kl + row * L::kPitch + col) = kv;
        *reinterpret_cast<float4*>(Vl + row * L::kPitch + col) = vv;
      }
      __syncthreads();
      int klo[kQB], khi[kQB];
      bool lane_any = false;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        if (valid[qb]) {
          step_bounds(st, lo_[qb], an[qb], blk[qb], klo[qb], khi[qb]);
          lane_any = lane_any || klo[qb] < khi[qb];
        } else {
          klo[qb] = 0;
          khi[qb] = kTileK;
        }
      }
      if (!__any(lane_any)) continue;
      f32x16 sacc[kKB][kQB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;
#pragma unroll 8
      for (int t = 0; t < D / 2; ++t)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
          const float kf = Kl[(kb * 32 + l32) * L::kPitch + 2 * t + h32];
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[qb][t], sacc[kb][qb], 0, 0, 0);
        }
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kappa = 32 * kb + 8 * (r >> 2) + 4 * h32 + (r & 3);
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            if (kappa < klo[qb] || kappa >= khi[qb]) sacc[kb][qb][r] = kNegInf;
        }
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * c;
        const bool need = mt > m_used[qb] + 8.0f;
        if (__any(need)) {
          const float alpha = need ? exp2_fast(m_used[qb] - mt) : 1.0f;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) o[qb][db] *= alpha;
          if (need) m_used[qb] = mt;
        }
        const float msub = m_used[qb] == kNegInf ? 0.f : m_used[qb];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(fmaf(sacc[kb][qb][r], c, -msub));
            sacc[kb][qb][r] = p;
            l[qb] += p;
          }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kappa = 32 * kb + 8 * (r >> 2) + 4 * h32 + (r & 3);
            const float vf = Vl[kappa * L::kPitch + 32 * db + l32];
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
              o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, sacc[kb][qb][r], o[qb][db], 0, 0, 0);
          }
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float lt = l[qb] + __shfl_xor(l[qb], 32);
      if (!valid[qb]) continue;
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const float lse = lt > 0.f ? (m_used[qb] + log2f(lt)) * kLn2 : kNegInf;
      const bool direct = slot < 0;
      const int64_t row = direct ? (int64_t)tok[qb] * hq + qh[qb] : (int64_t)slot * kQTile + rloc[qb];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = 32 * db + 8 * j + 4 * h32;
          if (direct && a.o_bf16) {
            bf16x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(o[qb][db][4 * j + i] * inv);
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.O) + row * D + d0) = w;
          } else {
            f32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = o[qb][db][4 * j + i] * inv;
            float* dst = direct ? static_cast<float*>(a.O) : a.ws_O;
            *reinterpret_cast<f32x4*>(dst + row * D + d0) = w;
          }
        }
      if (h32 == 0) (direct ? a.LSE : a.ws_LSE)[row] = lse;
    }
  }
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  if (a.dtype_bf16) {
    constexpr int bytes = Bf16Lds<D>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_bf16_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    SKV_LAUNCH("fwd_bf16", fwd_bf16_kernel<D>, dim3(a.n_wg), dim3(kThreads), bytes, stream, a);
  } else {
    constexpr int bytes = F32Lds<D>::bytes;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_f32_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    SKV_LAUNCH("fwd_f32", fwd_f32_kernel<D>, dim3(a.n_wg), dim3(kThreads), bytes, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_split(const FwdArgs& a, hipStream_t stream);

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  hipError_t e = a.d == 128 ? launch_fwd_d<128>(a, stream) : launch_fwd_d<64>(a, stream);
  if (e != hipSuccess) return e;
  if (a.n_split > 0) return launch_merge_split(a, stream);
  return hipSuccess;
}

}  // namespace skv
