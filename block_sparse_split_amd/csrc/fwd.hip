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
// and share one mask bound.  The bf16 kernel runs eight waves of 32 rows
// (two groups half a step apart, below); the fp32 kernel four waves of 64
// rows (two 32-query MFMA column blocks).
//
// Per 64-key step, each wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T held in registers),
// so every lane owns one query column: the softmax max/sum over keys is a
// per-lane reduction plus one exchange with lane ^ 32.  P^T is rounded to
// bf16 in place and feeds O^T += V^T P^T directly as the B operand; the V^T
// operand comes from transposed LDS reads whose key order matches the
// accumulator layout of S^T, so no register transpose is needed.  The
// online softmax works in base 2 with the scale folded into one FMA.  It
// first exponentiates against the maximum already in use and keeps the
// result if no weight exceeds 2^16; only otherwise (and at a row's first
// visible keys) does it take the step's row maximum, and it rescales O only
// where that maximum grew by more than 2^8.  Both are exact: the same
// maximum is used for O and for the sum, and it never exceeds the true
// running maximum, so the sum stays at least 1.  Tiles that
// straddle an anchor bound are masked per element; fully visible tiles skip
// the mask, invisible ones skip the MFMAs.
#include "launch.h"
#include "tile_stage.h"
#include "timing.h"

namespace skv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 2;             // 32-query column blocks per wave
constexpr int kKB = kTileK / 32;   // 32-key blocks per step

// ---------------------------------------------------------------------------
// bf16 path.  Eight waves (two per SIMD) each own 32 query rows of the
// 256-row tile.  K and V tiles reach LDS by direct global->LDS DMA
// (buffer_load_dwordx4 ... lds, whole rows per instruction) into a 4-stage ring
// of interleaved row tiles, so loads run two steps ahead and no registers
// hold staged data; K is read as natural MFMA operands, V as transposed ones,
// each one base register plus an immediate offset, without bank conflicts.
template <int D>
struct FwdCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kTileBytes = ITile<D>::kBytes;     // 17 KB (d=128) / 9 KB
  static constexpr int kStageBytes = 2 * kTileBytes;       // K then V
  static constexpr int kStages = 4;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  // group B (waves 4-7) issues all tile DMA, in its softmax half steps, so
  // the issue latency stays off the MFMA group's path
  static constexpr int kDmaPerWave = 2 * ITile<D>::kBlocks / 4;
  // LDS operand reads kept in flight ahead of the MFMAs (K: one read per
  // fragment, V: two transposed reads per fragment)
  static constexpr int kPrefetchK = 6;
  static constexpr int kPrefetchV = 4;
};

// Issue this group-B wave's share of the DMA for one step into `stage`:
// waves 4, 5 copy the K blocks of the interleaved row tile, waves 6, 7 the V
// blocks.  Block g holds key rows g kRB .. g kRB + kRB - 1 of the step, so a
// lane's address is the step's first row (in the buffer base), a per-block
// scalar offset and a per-lane offset `lane_off` (row lane % kRB, its 16-byte
// column).  Rows past the end of a ragged step read the keys that follow it
// (masked), or zeros past the end of the tensor.
template <int D>
__device__ __forceinline__ void issue_step(const __bf16* Kg, const __bf16* Vg, int64_t kv_rows,
                                           const Step& st, int head, int hkv, uint32_t stage,
                                           int wave, uint32_t lane_off) {
  using C = FwdCfg<D>;
  using T = ITile<D>;
  const bool isv = wave >= 6;
  const int64_t row_bytes = (int64_t)hkv * D * 2;
  const int64_t off = st.row * row_bytes + (int64_t)head * D * 2;
  const i32x4 res = buf_res(reinterpret_cast<const char*>(isv ? Vg : Kg) + off,
                            kv_rows * row_bytes - off);
#pragma unroll
  for (int i = 0; i < C::kDmaPerWave; ++i) {
    const int g = (wave & 1) * C::kDmaPerWave + i;
    dma16_buf(res, lane_off, (uint32_t)(g * T::kRB * row_bytes),
              stage + (isv ? C::kTileBytes : 0) + g * T::kBlockStride);
  }
}

// Two groups of four waves (waves w and w + 4 share a SIMD) run the same
// per-step work -- QK (MFMA), softmax (VALU), PV (MFMA) -- half a step apart.
// Every half step ends in a workgroup barrier; within a half step one group
// issues PV of its previous step and QK of its next step while the other
// group runs the softmax, so each SIMD always has one wave feeding the matrix
// cores and one feeding the vector ALU.  Half step k (k = -1 .. 2n):
//   group A (waves 0-3): k odd  -> PV(s-1), QK(s) with s = (k+1)/2;  k even -> softmax(k/2)
//   group B (waves 4-7): k even -> PV(s-1), QK(s) with s = k/2;      k odd  -> softmax((k-1)/2)
// Tile s is read in half steps 2s-1 .. 2s+2; a 4-stage ring re-fills the
// stage of tile j with tile j+4 at the start of half step 2j+3.
template <int D>
__global__ __launch_bounds__(FwdCfg<D>::kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  const uint64_t t_wg = wg_clock_now();
  extern __shared__ __align__(16) char smem[];
  const sched_t S = sched_const(a.sched);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool groupA = wave < 4;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int nq = nb * kBlock, rows_per_head = nq * G;
  const sched_t anchors = S + S[H_OFF_ANCHORS];
  const sched_t los = S + S[H_OFF_LO];
  const sched_t tiles = S + S[H_OFF_TILES];
  const sched_t items = S + S[H_OFF_ITEMS];
  const sched_t queue = S + S[H_OFF_QUEUE];
  const int vq = claim_queue(S, a.xcd_count);
  const int qbeg = S[S[H_OFF_QOFF] + vq], qend = S[S[H_OFF_QOFF] + vq + 1];
  const float c = a.scale * kLog2e;
  const __bf16* Qg = static_cast<const __bf16*>(a.Q);
  const uint32_t lds0 = lds_addr(smem);
  // per-lane LDS byte offsets inside a stage: K fragment lane slot and the
  // transposed V read
  const uint32_t koff = itile_nat_offset<D>(lane);
  const uint32_t voff = C::kTileBytes + itile_tr_offset<D>(lane);
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

    auto stage_of = [&](int s) { return lds0 + (s & (C::kStages - 1)) * C::kStageBytes; };
    auto issue = [&](int s) {
      const Step st = item_step(tiles, s, n_draft, t0, sp);
      const __bf16* Kg = static_cast<const __bf16*>(st.draft ? a.Kd : a.K);
      const __bf16* Vg = static_cast<const __bf16*>(st.draft ? a.Vd : a.V);
      issue_step<D>(Kg, Vg, st.draft ? nq : a.n_local, st, head, hkv, stage_of(s), wave,
                    dma_off);
    };
    bf16x8 qf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint4 u = valid ? *reinterpret_cast<const uint4*>(Qg + qrow * D + 16 * t + 8 * h32)
                            : make_uint4(0, 0, 0, 0);
      qf[t] = __builtin_bit_cast(bf16x8, u);
    }
    // settle the per-row loads while no tile DMA is in flight, so that no
    // wait for them lands inside the step loop (vmcnt also counts the DMA)
    wait_vmcnt<0>();
#pragma unroll
    for (int s = 0; s < C::kStages; ++s)
      if (s < n_steps && !groupA) issue(s);
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_used = kNegInf, l = 0.f;
    // P of the step whose softmax ran last, carried to the next MFMA phase
    bf16x8 pf[2][2];
    bool p_act = false;

    // Barrier of half step k, with the ring bookkeeping of odd half steps
    // (group B is then in its softmax half): before it, a group-B wave waits
    // for its share of tile (k+1)/2 (at most the following tile's loads may
    // still be in flight); after it, group B re-fills the stage that tile
    // (k-3)/2 has left with tile (k-3)/2 + kStages.
    auto half_step = [&](int k) {
      if ((k & 1) != 0 && !groupA) {
        const int sn = (k + 1) / 2;
        if (sn < n_steps) {
          if (sn + 1 < n_steps) wait_vmcnt<C::kDmaPerWave>();
          else wait_vmcnt<0>();
        }
      }
      block_barrier();
      if ((k & 1) != 0 && k >= 3 && !groupA) {
        const int sj = (k - 3) / 2 + C::kStages;
        if (sj < n_steps) issue(sj);
      }
    };
    // MFMA phase p runs in half step 2p - 1 (group A) or 2p (group B), the
    // softmax of step p in the half step after it.  Group B starts with an
    // idle half step and skips the (empty) last one, so both groups pass the
    // same 2 n + 2 barriers.
    const int k0 = groupA ? -1 : 0;
    constexpr int NDB = D / 32;
    constexpr int NMF = D / 8;  // MFMAs of PV, and of QK
    // PV MFMA i: O^T += V^T P^T (P from the last softmax) for key block kb,
    // k-half t2, output block db
    auto pv_read = [&](uint32_t vbase, int i) {
      return itile_tr<D>(vbase, i % NDB, i / (2 * NDB), (i / NDB) % 2);
    };
    auto pv_mfma = [&](int i, const bf16x8& v) {
      o[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, pf[i / (2 * NDB)][(i / NDB) % 2],
                                                           o[i % NDB], 0, 0, 0);
    };
    auto pv = [&](int s) {
      const uint32_t vbase = opaque(stage_of(s) + voff);
      lds_pipelined<NMF, C::kPrefetchV>([&](int i) { return pv_read(vbase, i); }, pv_mfma);
    };
    if (!groupA) half_step(-1);
    for (int p = 0; p < n_steps; ++p) {
      half_step(2 * p + k0);
      // PV of step p-1, then QK of step p, in one operand pipeline (the
      // first QK operands load during the last PV MFMAs).  QK runs even for
      // a step no row sees; its softmax is skipped.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      const uint32_t kbase = opaque(stage_of(p) + koff);
      // QK MFMA i: d-step t = i / 2, key block kb = i % 2
      auto qk_read = [&](int i) { return itile_nat<D>(kbase, i % 2, i / 2); };
      auto qk_mfma = [&](int i, const bf16x8& k) {
        sacc[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, qf[i / 2], sacc[i % 2], 0, 0, 0);
      };
      if (p_act) {
        const uint32_t vbase = opaque(stage_of(p - 1) + voff);
        lds_pipelined<2 * NMF, C::kPrefetchK>(
            [&](int i) { return i < NMF ? pv_read(vbase, i) : qk_read(i - NMF); },
            [&](int i, const bf16x8& x) {
              if (i < NMF) pv_mfma(i, x);
              else qk_mfma(i - NMF, x);
            });
      } else {
        lds_pipelined<NMF, C::kPrefetchK>(qk_read, qk_mfma);
      }
      half_step(2 * p + k0 + 1);
      // softmax of step p; steps every row sees whole need no bounds
      int klo = 0, khi = kTileK;
      bool s_act = true, s_full = true;
      if (p < ws0 || p >= ws1) {
        const Step st = item_step(tiles, p, n_draft, t0, sp);
        bool lane_any = false, lane_full = true;
        if (valid) {
          step_bounds(st, lo_, an, blk, klo, khi);
          lane_any = klo < khi;
          lane_full = klo <= 0 && khi >= kTileK;
        }
        s_act = __any(lane_any);
        s_full = __all(lane_full);
      }
      p_act = s_act;
      if (s_act) {
        if (!s_full) {
          // key kappa = 32 kb + 8 (r / 4) + 4 h32 + r % 4: fold the lane
          // part into the bounds so the per-element index is a constant
          const int lo4 = klo - 4 * h32, hi4 = khi - 4 * h32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kc = 32 * kb + 8 * (r >> 2) + (r & 3);
              if (kc < lo4 || kc >= hi4) sacc[kb][r] = kNegInf;
            }
        }
        // P = 2^(c s - m_used) with the maximum already in use: valid while
        // every row has a finite m_used and no P exceeds 2^16, which the
        // lane's partial sum bounds; otherwise the row maximum is taken and
        // O is rescaled where it grew by more than 2^8.
        auto exp_pass = [&](float msub) {
          float ls = 0.f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pv_ = exp2_fast(fmaf(sacc[kb][r], c, -msub));
              ls += pv_;
              pf[kb][r >> 3][r & 7] = f32_to_bf16(pv_);
            }
          return ls;
        };
        float ls = 0.f;
        bool slow = __any(m_used == kNegInf);
        if (!slow) {
          ls = exp_pass(m_used);
          slow = __any(!(ls <= 65536.f));
        }
        if (slow) {
          float mx = kNegInf;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
          mx = max_xor32(mx);
          const float mt = mx * c;
          const bool need = mt > m_used + 8.0f;
          if (__any(need)) {
            const float alpha = need ? exp2_fast(m_used - mt) : 1.0f;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            if (need) m_used = mt;
          }
          ls = exp_pass(m_used == kNegInf ? 0.f : m_used);
        }
        l += ls;
      }
    }
    // last MFMA phase: PV of the last step only
    half_step(2 * n_steps + k0);
    if (p_act) pv(n_steps - 1);
    if (groupA) half_step(2 * n_steps + k0 + 1);
    // all waves are done with the ring before the next item's DMA reuses it
    block_barrier();

    const float lt = sum_xor32(l);
    if (valid) {
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      const float lse = lt > 0.f ? (m_used + log2f(lt)) * kLn2 : kNegInf;
      if (slot < 0) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * h32;
            if (a.o_bf16) {
              bf16x4 w;
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(o[db][4 * j + i] * inv);
              *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.O) + qrow * D + d0) = w;
            } else {
              f32x4 w;
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = o[db][4 * j + i] * inv;
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.O) + qrow * D + d0) = w;
            }
          }
        if (h32 == 0) a.LSE[qrow] = lse;
      } else {
        const int64_t prow = (int64_t)slot * kQTile + rloc;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * h32;
            f32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = o[db][4 * j + i] * inv;
            *reinterpret_cast<f32x4*>(a.ws_O + prow * D + d0) = w;
          }
        if (h32 == 0) a.ws_LSE[prow] = lse;
      }
    }
  }
  wg_clock_record(a.wg_clock, t_wg, vq);
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
  const sched_t S = sched_const(a.sched);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int nq = nb * kBlock, rows_per_head = nq * G;
  const sched_t anchors = S + S[H_OFF_ANCHORS];
  const sched_t los = S + S[H_OFF_LO];
  const sched_t tiles = S + S[H_OFF_TILES];
  const sched_t items = S + S[H_OFF_ITEMS];
  const sched_t queue = S + S[H_OFF_QUEUE];
  const int vq = claim_queue(S, a.xcd_count);
  const int qbeg = S[S[H_OFF_QOFF] + vq], qend = S[S[H_OFF_QOFF] + vq + 1];
  const float c = a.scale * kLog2e;
  const float* Qg = static_cast<const float*>(a.Q);

  for (int qi = qbeg; qi < qend; ++qi) {
    const sched_t it = items + queue[qi] * I_WORDS;
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
        mx = max_xor32(mx);
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

// Zeroes the forward's per-XCD queue counters before a launch that claims
// queues by XCD.
__global__ __launch_bounds__(64) void xcd_reset_kernel(uint32_t* count) {
  if (threadIdx.x < kXcds) count[threadIdx.x] = 0u;
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  if (a.xcd_count != nullptr) {
    SKV_LAUNCH("xcd_reset", xcd_reset_kernel, dim3(1), dim3(64), 0, stream, a.xcd_count);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dtype_bf16) {
    constexpr int bytes = FwdCfg<D>::kLdsBytes;
    static LdsLimit lds;
    const hipError_t e = lds.ensure(reinterpret_cast<const void*>(&fwd_bf16_kernel<D>), bytes);
    if (e != hipSuccess) return e;
    SKV_LAUNCH("fwd_bf16", fwd_bf16_kernel<D>, dim3(a.n_wg), dim3(FwdCfg<D>::kThreads), bytes,
               stream, a);
  } else {
    constexpr int bytes = F32Lds<D>::bytes;
    static LdsLimit lds;
    const hipError_t e = lds.ensure(reinterpret_cast<const void*>(&fwd_f32_kernel<D>), bytes);
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
