// Backward of the draft cross-attention over one key shard (gfx950, bf16).
//
// Only the queries and their gradients cross participants; key/value
// gradients stay with the keys (rit.work blog post on Split-KV, section
// "Split-KV moves queries, not keys and values").  With the FINAL merged
// output O and normaliser LSE, P = exp(scale * q k^T - LSE) are the true
// attention weights restricted to this shard's keys, so the shard's
// gradients are exact shares:
//   D  = rowsum(dO * O)
//   dP = dO V^T,  dS = P * (dP - D)
//   dQ = scale dS K   (this shard's share; shares over shards sum to dQ)
//   dK = scale dS^T Q,  dV = P^T dO   (query heads of a kv head summed)
//
// Kernels (no atomics, deterministic):
//   pre   D and LSE*log2(e) for every query row, stored per kv head in the
//         row order of the query tiles (so both can be DMA'd as rows);
//   dq    query-stationary, the forward's work items and LPT queues, eight
//         waves of 32 rows: per 64-key step S^T = K Q^T and dP^T = V dO^T
//         (lanes own query columns), dS^T in registers, dQ^T += K^T dS^T;
//         K (read naturally for S^T and transposed for dQ^T) and V arrive by
//         DMA in a 3-stage ring; split query tiles write partial slots that
//         a reduction kernel sums;
//   dkdv  key-stationary: a wave owns 32 keys (K^T, V^T B operands in
//         registers) and walks 64-row tiles of the query rows that may see
//         them: S = Q K^T and dP = dO V^T (lanes own key columns), then
//         dV^T += dO^T P and dK^T += Q^T dS; Q and dO tiles and
//         the row statistics arrive by DMA in a 3-stage
//         ring; each key's gradients are written once.
#include "launch.h"
#include "tile_stage.h"
#include "timing.h"

namespace skv {
namespace {

// ---------------------------------------------------------------- pre
// Row r (token, q-head h) of a kv head g = h / G has per-head index
// rho = token * G + h % G.  Writes, at [g * Nq * G + rho]: -D (the dP
// accumulators start from it, so they end as dP - D), LSE * log2(e) (+inf
// for a row that sees no key) and the row's visible context interval
// [lo, anchor) of its anchor block.  It also zeroes the per-XCD queue
// counters of the dQ and dK/dV kernels that follow it on the stream, and
// the dK/dV kernel's claim counters (one per queue).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const int32_t* sched, const __bf16* O,
                                                      const __bf16* dO, const float* LSE,
                                                      float* nDrm, float* L2rm, int32_t* LOrm,
                                                      int32_t* HIrm, int64_t rows, int hq, int G,
                                                      uint32_t* xcd_count, uint32_t* kv_front,
                                                      int n_wg) {
  if (xcd_count != nullptr && blockIdx.x == 0 && threadIdx.x < 2 * kXcds)
    xcd_count[threadIdx.x] = 0u;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_wg; i += 256) kv_front[i] = 0u;
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  {
    // padding rows after each kv head's rows: no visible key
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int hkv = hq / G;
    if (gt < (int64_t)hkv * kStatPad) {
      const int64_t idx = (gt / kStatPad) * (rows / hq * G + kStatPad) + rows / hq * G +
                          gt % kStatPad;
      nDrm[idx] = 0.f;
      L2rm[idx] = __builtin_inff();
      LOrm[idx] = 0;
      HIrm[idx] = 0;
    }
  }
  float s = 0.f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(O + row * D + c);
    const uint4 b = *reinterpret_cast<const uint4*>(dO + row * D + c);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(wa[i] << 16), __uint_as_float(wb[i] << 16), s);
      s = fmaf(__uint_as_float(wa[i] & 0xFFFF0000u), __uint_as_float(wb[i] & 0xFFFF0000u), s);
    }
  }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (row < rows && c == 0) {
    const int64_t token = row / hq;
    const int h = (int)(row % hq);
    const int64_t nqG = rows / hq * G;
    const int64_t idx = (int64_t)(h / G) * (nqG + kStatPad) + token * G + h % G;
    const float L = LSE[row];
    const int blk = (int)(token / kBlock);
    nDrm[idx] = -s;
    L2rm[idx] = L == kNegInf ? __builtin_inff() : L * kLog2e;
    LOrm[idx] = sched[sched[H_OFF_LO] + blk];
    HIrm[idx] = sched[sched[H_OFF_ANCHORS] + blk];
  }
}

// ---------------------------------------------------------------- dQ
template <int D>
struct DqCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  // K (natural and transposed reads), then V (natural reads)
  static constexpr int kVOff = ITile<D>::kBytes;
  static constexpr int kStageBytes = 2 * ITile<D>::kBytes;
  static constexpr int kStages = 3;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kDmaPerWave = 2 * ITile<D>::kBlocks / kWaves;
  static constexpr int kPrefetchNat = 6;
  static constexpr int kPrefetchTr = 4;
};

// This wave's share of one step's DMA: waves 0-3 copy the K blocks of the
// interleaved row tile, waves 4-7 the V blocks.  The step's first key row is
// in the buffer base, block g adds a scalar offset and `lane_off` is the
// lane's row (lane % kRB) and 16-byte column.  Rows past the end of a ragged
// step read the keys that follow it (masked), or zeros past the tensor's end.
template <int D>
__device__ __forceinline__ void dq_issue(const __bf16* Kg, const __bf16* Vg, int64_t kv_rows,
                                         const Step& st, int head, int hkv, uint32_t stage,
                                         int wave, uint32_t lane_off) {
  using C = DqCfg<D>;
  using T = ITile<D>;
  const bool isv = wave >= 4;
  const int64_t row_bytes = (int64_t)hkv * D * 2;
  const int64_t off = st.row * row_bytes + (int64_t)head * D * 2;
  const i32x4 res = buf_res(reinterpret_cast<const char*>(isv ? Vg : Kg) + off,
                            kv_rows * row_bytes - off);
#pragma unroll
  for (int i = 0; i < C::kDmaPerWave; ++i) {
    const int g = (wave & 3) * C::kDmaPerWave + i;
    dma16_buf(res, lane_off, (uint32_t)(g * T::kRB * row_bytes),
              stage + (isv ? C::kVOff : 0) + g * T::kBlockStride);
  }
}

template <int D>
__global__ __launch_bounds__(DqCfg<D>::kThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<D>;
  const uint64_t t_wg = wg_clock_now();
  extern __shared__ __align__(16) char smem[];
  const sched_t S = sched_const(a.sched);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int nq = nb * kBlock, rows_per_head = nq * G;
  const sched_t anchors = S + S[H_OFF_ANCHORS];
  const sched_t los = S + S[H_OFF_LO];
  const sched_t tiles = S + S[H_OFF_TILES];
  const sched_t items = S + S[H_OFF_DQ_ITEMS];
  const sched_t queue = S + S[H_OFF_DQ_QUEUE];
  const int vq = claim_queue(S, a.xcd_count);
  const int qbeg = S[S[H_OFF_DQ_QOFF] + vq], qend = S[S[H_OFF_DQ_QOFF] + vq + 1];
  const float c = a.scale * kLog2e;
  const __bf16* Qg = static_cast<const __bf16*>(a.Q);
  const __bf16* dOg = static_cast<const __bf16*>(a.dO);
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t knoff = itile_nat_offset<D>(lane);
  const uint32_t voff = C::kVOff + itile_nat_offset<D>(lane);
  const uint32_t troff = itile_tr_offset<D>(lane);
  // per-lane byte offset of this lane's DMA source inside a K/V block
  int drow, dcol;
  itile_rc<D>(0, lane, drow, dcol);
  const uint32_t dma_off = (uint32_t)((drow * hkv * D + dcol) * 2);

  for (int qi = qbeg; qi < qend; ++qi) {
    const sched_t it = items + queue[qi] * I_WORDS;
    const int head = it[I_HEAD], qt = it[I_QT], t0 = it[I_T0], t1 = it[I_T1];
    const int slot = it[I_SLOT], flags = it[I_FLAGS];
    const int ws0 = it[I_WHOLE] & 0xFFFF, ws1 = it[I_WHOLE] >> 16;
    const QTileSpan sp = qtile_span(qt, G, nq);
    const int n_draft = (flags & kItemDraft) ? (sp.dtok1 - sp.dtok0 + kTileK - 1) / kTileK : 0;
    const int n_steps = n_draft + (t1 - t0);

    const int rloc = wave * 32 + l32;
    const int rho = qt * kQTile + rloc;
    const bool valid = rho < rows_per_head;
    const int tok = valid ? rho / G : 0;
    const int qh = head * G + (valid ? rho % G : 0);
    const int blk = tok / kBlock;
    const int lo_ = valid ? los[blk] : 0, an = valid ? anchors[blk] : 0;
    const int64_t qrow = (int64_t)tok * hq + qh;

    auto issue = [&](int s) {
      const Step st = item_step(tiles, s, n_draft, t0, sp);
      const __bf16* Kg = static_cast<const __bf16*>(st.draft ? a.Kd : a.K);
      const __bf16* Vg = static_cast<const __bf16*>(st.draft ? a.Vd : a.V);
      dq_issue<D>(Kg, Vg, st.draft ? nq : a.n_local, st, head, hkv,
                  lds0 + (s % C::kStages) * C::kStageBytes, wave, dma_off);
    };
    bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint4 u = valid ? *reinterpret_cast<const uint4*>(Qg + qrow * D + 16 * t + 8 * h32)
                            : make_uint4(0, 0, 0, 0);
      const uint4 v = valid ? *reinterpret_cast<const uint4*>(dOg + qrow * D + 16 * t + 8 * h32)
                            : make_uint4(0, 0, 0, 0);
      qf[t] = __builtin_bit_cast(bf16x8, u);
      df[t] = __builtin_bit_cast(bf16x8, v);
    }
    const int64_t srow = (int64_t)head * (rows_per_head + kStatPad) + rho;
    const float lse2 = valid ? a.ws_L2[srow] : __builtin_inff();
    const float nDq = valid ? a.ws_nD[srow] : 0.f;
    // settle the per-row loads while no tile DMA is in flight, so that no
    // wait for them lands inside the step loop (vmcnt also counts the DMA)
    wait_vmcnt<0>();
    if (n_steps > 0) issue(0);
    if (n_steps > 1) issue(1);
    // initial dP^T accumulator: every element of a lane is in the lane's row
    f32x16 negd;
#pragma unroll
    for (int r = 0; r < 16; ++r) negd[r] = nDq;
    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

    for (int s = 0; s < n_steps; ++s) {
      if (s + 1 < n_steps) wait_vmcnt<C::kDmaPerWave>();
      else wait_vmcnt<0>();
      block_barrier();
      if (s + 2 < n_steps) issue(s + 2);
      const uint32_t stage = lds0 + (s % C::kStages) * C::kStageBytes;
      // steps every row sees whole need no bounds
      int klo = 0, khi = kTileK;
      bool full = true;
      if (s < ws0 || s >= ws1) {
        const Step st = item_step(tiles, s, n_draft, t0, sp);
        bool lane_any = false, lane_full = true;
        if (valid) {
          step_bounds(st, lo_, an, blk, klo, khi);
          lane_any = klo < khi;
          lane_full = klo <= 0 && khi >= kTileK;
        }
        if (!__any(lane_any)) continue;
        full = __all(lane_full);
      }
      const int klo4 = klo - 4 * h32, khi4 = khi - 4 * h32;
      const uint32_t kbase = opaque(stage + knoff);
      const uint32_t vbase = opaque(stage + voff);
      bf16x8 ds[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // one 32-key block at a time keeps S, dP of a single block live
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sacc, dp = negd;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
        // MFMA i: d-step t = i / 2; even i: S^T (K), odd i: dP^T (V)
        lds_pipelined<2 * (D / 16), C::kPrefetchNat>(
            [&](int i) {
              return i % 2 == 0 ? itile_nat<D>(kbase, kb, i / 2)
                                : itile_nat<D>(vbase, kb, i / 2);
            },
            [&](int i, const bf16x8& x) {
              if (i % 2 == 0)
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, qf[i / 2], sacc, 0, 0, 0);
              else
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, df[i / 2], dp, 0, 0, 0);
            });
        // a wave-uniform branch: tiles every row sees whole take no mask
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            ds[kb][r >> 3][r & 7] = f32_to_bf16(exp2_fast(fmaf(sacc[r], c, -lse2)) * dp[r]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // key 32 kb + 8 (r / 4) + 4 h32 + r % 4 against bounds shifted by 4 h32
            const int kc = 32 * kb + 8 * (r >> 2) + (r & 3);
            float p = exp2_fast(fmaf(sacc[r], c, -lse2));
            if (kc < klo4 || kc >= khi4) p = 0.f;
            ds[kb][r >> 3][r & 7] = f32_to_bf16(p * dp[r]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t tbase = opaque(stage + troff);
      constexpr int NDB = D / 32;
      // MFMA i: key block kb, k-half t2, output block db
      lds_pipelined<4 * NDB, C::kPrefetchTr>(
          [&](int i) { return itile_tr<D>(tbase, i % NDB, i / (2 * NDB), (i / NDB) % 2); },
          [&](int i, const bf16x8& k) {
            dq[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                k, ds[i / (2 * NDB)][(i / NDB) % 2], dq[i % NDB], 0, 0, 0);
          });
    }
    block_barrier();
    if (valid) {
      float* dst = slot < 0 ? a.dQ + qrow * D : a.ws_dQ + ((int64_t)slot * kQTile + rloc) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = dq[db][4 * j + i] * a.scale;
          *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * h32) = w;
        }
    }
  }
  wg_clock_record(a.wg_clock_dq, t_wg, vq);
}

// Sum the dQ partial slots of split query tiles.
template <int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const int32_t* S, const float* ws, float* dQ) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  constexpr int BPT = kQTile / RPB;
  const int32_t* rec = S + S[H_OFF_DQ_SPLIT] + (blockIdx.x / BPT) * S_WORDS;
  const int head = rec[S_HEAD], qt = rec[S_QT], slot0 = rec[S_SLOT0], ns = rec[S_NSLOT];
  const int rloc = (blockIdx.x % BPT) * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  const int G = S[H_G], hq = S[H_HQ], nq = S[H_NB] * kBlock;
  const int rho = qt * kQTile + rloc;
  if (rho >= nq * G) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < ns; ++k) {
    const float* p = ws + ((int64_t)(slot0 + k) * kQTile + rloc) * D + c;
    const float4 x = *reinterpret_cast<const float4*>(p);
    const float4 y = *reinterpret_cast<const float4*>(p + 4);
    acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
    acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
  }
  float* o = dQ + ((int64_t)(rho / G) * hq + head * G + rho % G) * D + c;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// ---------------------------------------------------------------- dK, dV
// Key-stationary.  Eight waves in four pairs; the waves of a pair share a
// SIMD (waves w and w + 4) and own the same 32 keys of the item:
//   P wave  (w < 4):  S = Q K^T, P = exp2(c S - L2) on visible pairs,
//                     dV^T += dO^T P;
//   dS wave (w >= 4): dP = dO V^T, dS = P (dP - D) with P taken from the P
//                     wave through LDS, dK^T += Q^T dS.
// Each holds one stationary operand (K or V of its keys) and one gradient,
// so a wave needs half the registers of one doing both, two waves fit per
// SIMD and one hides the other's LDS latency.  A 64-row query tile takes two
// half steps: S/P and dP (P goes to the exchange buffer), barrier, then dV
// and dK.  Q and dO tiles (natural reads for S and dP, transposed reads for
// dV and dK) and the per-row statistics (D, L2 and the row's visible
// interval) arrive by DMA in a 3-stage ring.  Every key's gradients are
// written once.
template <int D>
struct KvCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  // Q, dO (interleaved row tiles), then 1 KB of row statistics:
  // -D [0, 256), L2 [256, 512), lo [512, 768), anchor [768, 1024)
  static constexpr int kOOff = ITile<D>::kBytes;
  static constexpr int kStatOff = 2 * ITile<D>::kBytes;
  static constexpr int kStageBytes = kStatOff + 1024;
  static constexpr int kStages = 3;
  // P exchange: per pair 64 rows x 32 keys of bf16, in MFMA B-operand order
  static constexpr int kXOff = kStages * kStageBytes;
  static constexpr int kLdsBytes = kXOff + 4 * 4096;
  // the four dS waves issue all tile DMA (the P waves issue none)
  static constexpr int kDmaPerWave = 2 * ITile<D>::kBlocks / 4;
  static constexpr int kPrefetchNat = 6;
  static constexpr int kPrefetchTr = 4;
};

// Work claiming of the dK/dV kernel, called by every thread of the
// workgroup (one barrier).  A workgroup first runs its own queue v in order:
// front[v] (zero at launch) counts its claimed positions, and lane 0 of
// wave 0 claims the next one a call ahead (`pending`) so that the atomic's
// latency overlaps an item.  Once its queue is exhausted (`own` cleared),
// wave 0 reads every queue's counter and takes the next position of the
// queue with the most planned work left (the image's suffix costs), until
// no queue has any: idle workgroups take over the items of slow ones, so
// speed differences the static plan did not foresee even out.  Every item
// is claimed exactly once (atomic counters), and its outputs do not depend
// on the workgroup that runs it.  A failed claim finds its queue
// exhausted for good, so the search ends within n_wg + n_items tries.
// Returns the item, or -1 when none is left.
__device__ __forceinline__ int kv_claim(sched_t S, uint32_t* front, int v, int& own,
                                        int& pending, int call) {
  __shared__ int slot[2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave == 0) {
    const sched_t qoff = S + S[H_OFF_KVQOFF];
    const sched_t queue = S + S[H_OFF_KVQUEUE];
    const sched_t suf = S + S[H_OFF_KVSUF];
    int item = -1;
    if (own) {
      const int b = qoff[v], len = qoff[v + 1] - b;
      const int i = __shfl(pending, 0);
      if (i < len) {
        item = queue[b + i];
        if (lane == 0) pending = (int)atomicAdd(&front[v], 1u);
      } else {
        own = 0;
      }
    }
    if (!own) {
      const int n = S[H_NWG], cap = n + S[H_NKV];
      for (int tries = 0; item < 0 && tries <= cap; ++tries) {
        int best = 0, bu = -1;
        for (int u = lane; u < n; u += 64) {
          const int b = qoff[u], len = qoff[u + 1] - b;
          const int f =
              (int)__hip_atomic_load(&front[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (f < len && suf[b + f] > best) {
            best = suf[b + f];
            bu = u;
          }
        }
        // the most work left over the wave (ties: the lower queue)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const int ob = __shfl_xor(best, o), ou = __shfl_xor(bu, o);
          if (ob > best || (ob == best && ou >= 0 && (bu < 0 || ou < bu))) {
            best = ob;
            bu = ou;
          }
        }
        const int U = __builtin_amdgcn_readfirstlane(bu);
        if (__builtin_amdgcn_readfirstlane(best) <= 0 || U < 0) break;
        int got = -1;
        if (lane == 0) {
          const int b = qoff[U], len = qoff[U + 1] - b;
          const uint32_t i = atomicAdd(&front[U], 1u);
          if (i < (uint32_t)len) got = queue[b + (int)i];
        }
        item = __shfl(got, 0);
      }
    }
    if (lane == 0) slot[call & 1] = item;
  }
  __syncthreads();
  return slot[call & 1];
}

// The two roles run separate copies of the whole item loop, so that the
// compiler never keeps one role's loop state live in the other's.
template <int D, bool PW>
__device__ __forceinline__ void dkdv_role(const BwdArgs& a, int vq) {
  using C = KvCfg<D>;
  // distinct (empty) markers keep the optimiser from merging the two roles'
  // code back into one path with selects
  if constexpr (PW) asm volatile("; dkdv role P" ::: "memory");
  else asm volatile("; dkdv role dS" ::: "memory");
  constexpr int NDB = D / 32;
  extern __shared__ __align__(16) char smem[];
  const sched_t S = sched_const(a.sched);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  constexpr bool pwave = PW;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int rows_per_head = nb * kBlock * G;
  // G is a power of two: row -> (token, head) and row -> block are shifts
  const int lgG = __builtin_ctz(G), lgR = 4 + lgG;
  const sched_t tiles = S + S[H_OFF_TILES];
  const sched_t kvs = S + S[H_OFF_KV];
  const float c = a.scale * kLog2e;
  const __bf16* Qg = static_cast<const __bf16*>(a.Q);
  const __bf16* dOg = static_cast<const __bf16*>(a.dO);
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t noff = itile_nat_offset<D>(lane);
  const uint32_t troff = itile_tr_offset<D>(lane);
  const uint32_t xslot = lds0 + C::kXOff + pair * 4096 + 16 * lane;
  // byte offset of row r of a query tile from the tile's first row (tiles
  // start at a multiple of G rows: r / G tokens on, head r % G)
  auto qrow_bytes = [&](int r) { return (uint32_t)((((r >> lgG) * hq) + (r & (G - 1))) * D * 2); };
  const int64_t q_bytes = (int64_t)nb * kBlock * hq * D * 2;
  int drow, dcol;
  itile_rc<D>(0, lane, drow, dcol);
  const uint32_t dma_off = qrow_bytes(drow) + 2 * dcol;
  const i32x4 stat_res = buf_res(a.ws_nD, 16 * a.stat_words);
  const uint32_t stat_off = (uint32_t)(((lane >> 4) * a.stat_words + 4 * (lane & 15)) * 4);

  // items: the own queue, then the others' (kv_claim)
  int own = 1, pending = 0;
  if (tid == 0) pending = (int)atomicAdd(&a.kv_front[vq], 1u);
  for (int call = 0;; ++call) {
    const int item = kv_claim(S, a.kv_front, vq, own, pending, call);
    if (item < 0) break;
    const sched_t it = kvs + item * K_WORDS;
    const int head = it[K_HEAD], t0 = it[K_T0], nt = it[K_NT];
    const int dtok0 = it[K_DTOK0], nd = it[K_NDRAFT], b0 = it[K_B0], b1 = it[K_B1];
    // row tiles every row of which sees all of the item's keys
    const int kw0 = it[K_WHOLE] & 0xFFFF, kw1 = it[K_WHOLE] >> 16;
    const bool draft = nd > 0;
    // the pair's 32 keys: rows of K/V (or Kd/Vd) and absolute positions
    // (draft keys: their draft token)
    int krow = 0, kpos = 0, nk = 0;
    if (draft) {
      krow = dtok0 + 32 * pair;
      kpos = krow;
      nk = max(0, min(32, nd - 32 * pair));
    } else if ((pair >> 1) < nt) {
      const sched_t tl = tiles + (t0 + (pair >> 1)) * T_WORDS;
      krow = tl[T_ROW] + 32 * (pair & 1);
      kpos = tl[T_POS] + 32 * (pair & 1);
      nk = max(0, min(32, tl[T_LEN] - 32 * (pair & 1)));
    }
    const bool kvalid = l32 < nk;
    const int mypos = kpos + l32;
    const int kp0 = kpos, kp1 = kpos + nk;
    const int r_begin = b0 * kBlock * G, r_end = b1 * kBlock * G;
    const int n_rt = (r_end - r_begin + kTileK - 1) / kTileK;

    auto stage_of = [&](int rt) { return lds0 + (rt % C::kStages) * C::kStageBytes; };
    // dS waves only: this wave's share of tile rt -- waves 4, 5 the Q blocks,
    // waves 6, 7 the dO blocks (wave 4 also the row statistics).  The tile's
    // first row is in the buffer base, block g adds the scalar qrow_bytes(g
    // kRB) and `dma_off` is the lane's row and column.  Rows past r_end read
    // the rows that follow (their statistics mask them), or zeros past the
    // tensor's end.
    auto issue = [&](int rt) {
      const uint32_t stage = stage_of(rt);
      const int rho0 = r_begin + kTileK * rt;
      const bool iso = (wave & 2) != 0;
      const int64_t off = ((int64_t)(rho0 >> lgG) * hq + head * G) * D * 2;
      const i32x4 res =
          buf_res(reinterpret_cast<const char*>(iso ? dOg : Qg) + off, q_bytes - off);
#pragma unroll
      for (int i = 0; i < C::kDmaPerWave; ++i) {
        const int g = (wave & 1) * C::kDmaPerWave + i;
        dma16_buf(res, dma_off, qrow_bytes(g * ITile<D>::kRB),
                  stage + (iso ? C::kOOff : 0) + g * ITile<D>::kBlockStride);
      }
      if ((wave & 3) == 0) {
        // 16 lanes per statistic (-D, L2, lo, anchor: consecutive arrays of
        // stat_words each), 4 rows per lane; a tile ends at most 63 rows
        // past the head's rows, inside its padding
        dma16_buf(stat_res, stat_off,
                  (uint32_t)(((int64_t)head * (rows_per_head + kStatPad) + rho0) * 4),
                  stage + C::kStatOff);
      }
    };
    // this wave's stationary B operand: K (P wave) or V (dS wave) of its keys
    const void* ksrc = pwave ? (draft ? a.Kd : a.K) : (draft ? a.Vd : a.V);
    const int64_t kaddr = ((int64_t)(krow + (kvalid ? l32 : 0)) * hkv + head) * D;
    bf16x8 kv[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint4 u = kvalid ? *reinterpret_cast<const uint4*>(
                                   static_cast<const __bf16*>(ksrc) + kaddr + 16 * t + 8 * h32)
                             : make_uint4(0, 0, 0, 0);
      kv[t] = __builtin_bit_cast(bf16x8, u);
    }
    // settle the per-item loads before any tile DMA is in flight
    wait_vmcnt<0>();
    if (!pwave) {
      if (n_rt > 0) issue(0);
      if (n_rt > 1) issue(1);
    }
    f32x16 acc[NDB];  // dV^T (P wave) or dK^T (dS wave) of the pair's keys
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // Opening barrier of tile rt: a dS wave's share of tile rt has landed
    // once at most tile rt+1's loads are in flight.  Tile rt+2 goes into the
    // stage of tile rt-1, free after this barrier; the dS waves issue it
    // after their dP MFMAs, where they would otherwise wait for the P
    // waves' softmax.
    // Returns whether any row of the tile sees any of the pair's keys, and
    // whether all rows see all of them.
    auto open_tile = [&](int rt, bool& full) -> bool {
      if (!pwave) {
        if (rt + 1 < n_rt) {
          if ((wave & 3) == 0) wait_vmcnt<C::kDmaPerWave + 1>();
          else wait_vmcnt<C::kDmaPerWave>();
        } else {
          wait_vmcnt<0>();
        }
      }
      block_barrier();
      if (rt >= kw0 && rt < kw1) {
        full = true;
        return nk > 0;
      }
      // Rows past r_end belong to blocks that see none of the item's keys
      // (their statistics, or the padding rows, say so), so every row's own
      // interval decides; draft keys: the row's block.
      const uint32_t stat = stage_of(rt) + C::kStatOff;
      const int row = r_begin + kTileK * rt + lane;
      int lo, hi;
      if (draft) {
        lo = (row >> lgR) * kBlock;
        hi = lo + kBlock;
      } else {
        lo = lds_read_i32(stat + 512 + 4 * lane);
        hi = lds_read_i32(stat + 768 + 4 * lane);
      }
      full = __all(lo <= kp0 && hi >= kp1);
      return __any(max(lo, kp0) < min(hi, kp1));
    };
    if constexpr (PW) {
      for (int rt = 0; rt < n_rt; ++rt) {
        bool full;
        const bool any = open_tile(rt, full);
        const uint32_t stage = stage_of(rt);
        const uint32_t stat = stage + C::kStatOff;
        const int rho0 = r_begin + kTileK * rt;
        bf16x8 pb[2][2];
        if (any) {
          f32x16 sacc[2];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[qb][r] = 0.f;
          const uint32_t qfb = opaque(stage + noff);
          // MFMA i: query block qb = i % 2, d-step t = i / 2
          lds_pipelined<2 * (D / 16), C::kPrefetchNat>(
              [&](int i) { return itile_nat<D>(qfb, i % 2, i / 2); },
              [&](int i, const bf16x8& q) {
                sacc[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q, kv[i / 2], sacc[i % 2],
                                                                      0, 0, 0);
              });
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r8 = qb * 32 + 8 * j;
              const int rr = r8 + 4 * h32;  // rows rr .. rr+3 of the tile
              const f32x4 l2 = lds_read_f4(stat + 256 + 4 * rr);
              if (!full) {
                // key visible to row i iff lo_i <= pos < hi_i
                i32x4 lo, hi;
                if (draft) {
                  const int b = ((rho0 + rr) >> lgR) * kBlock;  // the 4 rows share a block
                  lo = i32x4{b, b, b, b};
                  hi = lo + kBlock;
                } else {
                  lo = lds_read_i4(stat + 512 + 4 * rr);
                  hi = lds_read_i4(stat + 768 + 4 * rr);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if ((uint32_t)(mypos - lo[i]) >= (uint32_t)(hi[i] - lo[i]))
                    sacc[qb][4 * j + i] = kNegInf;
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = 4 * j + i;
                pb[qb][r >> 3][r & 7] = f32_to_bf16(exp2_fast(fmaf(sacc[qb][r], c, -l2[i])));
              }
            }
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) lds_write16(xslot + (2 * qb + t2) * 1024, pb[qb][t2]);
        }
        wait_lgkmcnt0();
        block_barrier();
        if (any) {
          const uint32_t otb = opaque(stage + troff + C::kOOff);
          // MFMA i: query block qb, k-half t2, output block db
          lds_pipelined<4 * NDB, C::kPrefetchTr>(
              [&](int i) { return itile_tr<D>(otb, i % NDB, i / (2 * NDB), (i / NDB) % 2); },
              [&](int i, const bf16x8& o) {
                acc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    o, pb[i / (2 * NDB)][(i / NDB) % 2], acc[i % NDB], 0, 0, 0);
              });
        }
      }
    } else {
      for (int rt = 0; rt < n_rt; ++rt) {
        bool full;
        const bool any = open_tile(rt, full);
        const uint32_t stage = stage_of(rt);
        const uint32_t stat = stage + C::kStatOff;
        f32x16 dp[2];
        if (any) {
          // the accumulators start from -D of their rows, so they end as
          // dP - D
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // rows 8 j + 4 h32 + 0..3 of query block qb
              const f32x4 nd = lds_read_f4(stat + 4 * (qb * 32 + 8 * j + 4 * h32));
#pragma unroll
              for (int i = 0; i < 4; ++i) dp[qb][4 * j + i] = nd[i];
            }
          const uint32_t ofb = opaque(stage + noff + C::kOOff);
          lds_pipelined<2 * (D / 16), C::kPrefetchNat>(
              [&](int i) { return itile_nat<D>(ofb, i % 2, i / 2); },
              [&](int i, const bf16x8& o) {
                dp[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, kv[i / 2], dp[i % 2], 0,
                                                                    0, 0);
              });
        }
        if (rt + 2 < n_rt) issue(rt + 2);
        block_barrier();
        if (any) {
          bf16x8 dsb[2][2];
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const bf16x8 pr = lds_read16(xslot + (2 * qb + t2) * 1024);
#pragma unroll
              for (int e = 0; e < 8; ++e)
                dsb[qb][t2][e] = f32_to_bf16(static_cast<float>(pr[e]) * dp[qb][8 * t2 + e]);
            }
          const uint32_t qtb = opaque(stage + troff);
          lds_pipelined<4 * NDB, C::kPrefetchTr>(
              [&](int i) { return itile_tr<D>(qtb, i % NDB, i / (2 * NDB), (i / NDB) % 2); },
              [&](int i, const bf16x8& q) {
                acc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    q, dsb[i / (2 * NDB)][(i / NDB) % 2], acc[i % NDB], 0, 0, 0);
              });
        }
      }
    }
    // the ring and the exchange buffer are free before the next item's DMA
    block_barrier();
    if (kvalid) {
      const int64_t orow = (int64_t)(krow + l32) * hkv + head;
      void* dst = pwave ? (draft ? a.dVd : a.dV) : (draft ? a.dKd : a.dK);
      const float mul = pwave ? 1.0f : a.scale;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = 32 * db + 8 * j + 4 * h32;
          if (a.grad_bf16) {
            bf16x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(acc[db][4 * j + i] * mul);
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(dst) + orow * D + d0) = w;
          } else {
            f32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = acc[db][4 * j + i] * mul;
            *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + orow * D + d0) = w;
          }
        }
    }
  }
}

template <int D>
__global__ __launch_bounds__(KvCfg<D>::kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  const uint64_t t_wg = wg_clock_now();
  const int vq = claim_queue(sched_const(a.sched), a.xcd_count ? a.xcd_count + kXcds : nullptr);
  if (threadIdx.x < 256) dkdv_role<D, true>(a, vq);
  else dkdv_role<D, false>(a, vq);
  wg_clock_record(a.wg_clock_kv, t_wg, vq);
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.nb * kBlock * a.hq;
  constexpr int RPB = 256 / (D / 8);
  SKV_LAUNCH("bwd_pre", bwd_pre_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(256), 0, s,
             a.sched, static_cast<const __bf16*>(a.O), static_cast<const __bf16*>(a.dO), a.LSE,
             a.ws_nD, a.ws_L2, a.ws_LO, a.ws_HI, rows, a.hq, a.hq / a.hkv, a.xcd_count,
             a.kv_front, a.n_wg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  static LdsLimit lds_dq, lds_kv;
  e = lds_dq.ensure(reinterpret_cast<const void*>(&bwd_dq_kernel<D>), DqCfg<D>::kLdsBytes);
  if (e != hipSuccess) return e;
  SKV_LAUNCH("bwd_dq", bwd_dq_kernel<D>, dim3(a.n_wg), dim3(DqCfg<D>::kThreads),
             DqCfg<D>::kLdsBytes, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.n_split > 0) {
    SKV_LAUNCH("dq_reduce", dq_reduce_kernel<D>, dim3(a.n_split * (kQTile / RPB)), dim3(256), 0,
               s, a.sched, a.ws_dQ, a.dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  e = lds_kv.ensure(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D>), KvCfg<D>::kLdsBytes);
  if (e != hipSuccess) return e;
  SKV_LAUNCH("bwd_dkdv", bwd_dkdv_kernel<D>, dim3(a.n_wg), dim3(KvCfg<D>::kThreads),
             KvCfg<D>::kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  if (!a.dtype_bf16) return hipErrorNotSupported;
  return a.d == 128 ? launch_bwd_d<128>(a, s) : launch_bwd_d<64>(a, s);
}

}  // namespace skv
