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
//   pre   D for every query row;
//   dq    query-stationary, same work items and LPT queues as the forward:
//         per 64-key step, S^T = K Q^T and dP^T = V dO^T (lanes own query
//         columns), dS^T in registers, dQ^T += K^T dS^T with K^T staged in
//         LDS in the permuted transposed layout; split query tiles write
//         partial slots that a reduction kernel sums;
//   dkdv  key-stationary: a wave owns 32 keys (K^T, V^T as B operands in
//         registers) and walks 64-row tiles of the query rows that may see
//         them: S = Q K^T and dP = dO V^T (lanes own key columns), then
//         dV^T += dO^T P and dK^T += Q^T dS with Q^T / dO^T staged
//         transposed; each key's gradients are written once.
#include "launch.h"
#include "tile_stage.h"
#include "timing.h"

namespace skv {
namespace {

// ---------------------------------------------------------------- D = rowsum
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* O, const __bf16* dO, float* Dv,
                                                      int64_t rows) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  float s = 0.f;
  if (row < rows) {
    const uint4 a = ld16(O + row * D + c), b = ld16(dO + row * D + c);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(wa[i] << 16), __uint_as_float(wb[i] << 16), s);
      s = fmaf(__uint_as_float(wa[i] & 0xFFFF0000u), __uint_as_float(wb[i] & 0xFFFF0000u), s);
    }
  }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (row < rows && c == 0) Dv[row] = s;
}

// ---------------------------------------------------------------- dQ
constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * 64;

template <int D>
struct DqLds {
  static constexpr int buf = 2 * Stage<D>::natElems + Stage<D>::trElems;  // K, V nat; K^T
  static constexpr int bytes = 2 * buf * 2;
};

template <int D>
__global__ __launch_bounds__(kQThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using St = Stage<D>;
  using L = DqLds<D>;
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
  const __bf16* dOg = static_cast<const __bf16*>(a.dO);
  // staging roles: threads [0, nQuads) take K quads, the next nQuads V quads
  const bool k_stager = tid < St::nQuads;
  const bool v_stager = tid >= St::nQuads && tid < 2 * St::nQuads;
  const int sq = k_stager ? tid : tid - St::nQuads;
  const int sm = sq / St::CPR, sdr = sq % St::CPR;

  for (int qi = qbeg; qi < qend; ++qi) {
    const int32_t* it = items + queue[qi] * I_WORDS;
    const int head = it[I_HEAD], qt = it[I_QT], t0 = it[I_T0], t1 = it[I_T1];
    const int slot = it[I_SLOT], flags = it[I_FLAGS];
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
    bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint4 u = valid ? ld16(Qg + qrow * D + 16 * t + 8 * h32) : make_uint4(0, 0, 0, 0);
      const uint4 v = valid ? ld16(dOg + qrow * D + 16 * t + 8 * h32) : make_uint4(0, 0, 0, 0);
      qf[t] = __builtin_bit_cast(bf16x8, u);
      df[t] = __builtin_bit_cast(bf16x8, v);
    }
    float lse2 = __builtin_inff(), Dq = 0.f;
    if (valid) {
      const float L = a.LSE[qrow];
      lse2 = L == kNegInf ? __builtin_inff() : L * kLog2e;
      Dq = a.ws_D[qrow];
    }
    f32x16 dq[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

    Quad qd;
    auto load = [&](int s) {
      const Step st = item_step(tiles, s, n_draft, t0, sp);
      const __bf16* src = static_cast<const __bf16*>(
          k_stager ? (st.draft ? a.Kd : a.K) : (st.draft ? a.Vd : a.V));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * sm + j;
        qd.v[j] = row < st.n ? ld16(src + ((int64_t)(st.row + row) * hkv + head) * D + sdr * 8)
                             : make_uint4(0, 0, 0, 0);
      }
    };
    auto store = [&](int s) {
      __bf16* buf = smem + (s & 1) * L::buf;
      if (k_stager) {
        store_nat<D>(buf, sm, sdr, qd);
        store_tr<D>(buf + 2 * St::natElems, sm, sdr, qd);
      } else if (v_stager) {
        store_nat<D>(buf + St::natElems, sm, sdr, qd);
      }
    };
    if (n_steps > 0 && (k_stager || v_stager)) {
      load(0);
      store(0);
    }
    __syncthreads();
    for (int s = 0; s < n_steps; ++s) {
      const Step st = item_step(tiles, s, n_draft, t0, sp);
      if (s + 1 < n_steps && (k_stager || v_stager)) load(s + 1);
      const __bf16* Kn = smem + (s & 1) * L::buf;
      const __bf16* Vn = Kn + St::natElems;
      const __bf16* Kt = Kn + 2 * St::natElems;
      int klo = 0, khi = kTileK;
      bool lane_any = false, lane_full = true;
      if (valid) {
        step_bounds(st, lo_, an, blk, klo, khi);
        lane_any = klo < khi;
        lane_full = klo <= 0 && khi >= kTileK;
      }
      if (__any(lane_any)) {
        f32x16 sacc[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_nat<D>(Kn, kb * 32, l32, h32, t),
                                                               qf[t], sacc[kb], 0, 0, 0);
            dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_nat<D>(Vn, kb * 32, l32, h32, t),
                                                             df[t], dp[kb], 0, 0, 0);
          }
        const bool full = __all(lane_full);
        bf16x8 ds[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kappa = 32 * kb + 8 * (r >> 2) + 4 * h32 + (r & 3);
            float p = exp2_fast(fmaf(sacc[kb][r], c, -lse2));
            if (!full && (kappa < klo || kappa >= khi)) p = 0.f;
            ds[kb][r >> 3][r & 7] = f32_to_bf16(p * (dp[kb][r] - Dq));
          }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
              dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  frag_tr<D>(Kt, db * 32, l32, h32, kb, t2), ds[kb][t2], dq[db], 0, 0, 0);
      }
      if (s + 1 < n_steps) store(s + 1);
      __syncthreads();
    }
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
}

// Sum the dQ partial slots of split query tiles.
template <int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(const int32_t* S, const float* ws, float* dQ) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  constexpr int BPT = kQTile / RPB;
  const int32_t* rec = S + S[H_OFF_SPLIT] + (blockIdx.x / BPT) * S_WORDS;
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
constexpr int kKWaves = 4;
constexpr int kKThreads = kKWaves * 64;

template <int D>
struct KvLds {
  // Q nat, dO nat, Q^T, dO^T, then lse2[64] and D[64] (fp32)
  static constexpr int bufElems = 2 * Stage<D>::natElems + 2 * Stage<D>::trElems + 2 * 64 * 2;
  static constexpr int bytes = 2 * bufElems * 2;
};

template <int D>
__global__ __launch_bounds__(kKThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using St = Stage<D>;
  using L = KvLds<D>;
  extern __shared__ __align__(16) char smem_raw[];
  __bf16* smem = reinterpret_cast<__bf16*>(smem_raw);
  const int32_t* S = a.sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h32 = lane >> 5, l32 = lane & 31;
  const int G = S[H_G], hq = S[H_HQ], hkv = S[H_HKV], nb = S[H_NB];
  const int rows_per_block = kBlock * G;
  const int32_t* anchors = S + S[H_OFF_ANCHORS];
  const int32_t* los = S + S[H_OFF_LO];
  const int32_t* tiles = S + S[H_OFF_TILES];
  const int32_t* kvs = S + S[H_OFF_KV];
  const int32_t* queue = S + S[H_OFF_KVQUEUE];
  const int qbeg = S[S[H_OFF_KVQOFF] + blockIdx.x], qend = S[S[H_OFF_KVQOFF] + blockIdx.x + 1];
  const float c = a.scale * kLog2e;
  const __bf16* Qg = static_cast<const __bf16*>(a.Q);
  const __bf16* dOg = static_cast<const __bf16*>(a.dO);
  const bool stager = tid < St::nQuads;
  const int sm = tid / St::CPR, sdr = tid % St::CPR;

  for (int qi = qbeg; qi < qend; ++qi) {
    const int32_t* it = kvs + queue[qi] * K_WORDS;
    const int head = it[K_HEAD], t0 = it[K_T0], nt = it[K_NT];
    const int dtok0 = it[K_DTOK0], nd = it[K_NDRAFT], b0 = it[K_B0], b1 = it[K_B1];
    const bool draft = nd > 0;
    // this wave's 32 keys
    int krow = 0, kpos = 0, nk = 0;
    if (draft) {
      krow = dtok0 + 32 * wave;
      kpos = krow;
      nk = max(0, min(32, nd - 32 * wave));
    } else if ((wave >> 1) < nt) {
      const int32_t* tl = tiles + (t0 + (wave >> 1)) * T_WORDS;
      krow = tl[T_ROW] + 32 * (wave & 1);
      kpos = tl[T_POS] + 32 * (wave & 1);
      nk = max(0, min(32, tl[T_LEN] - 32 * (wave & 1)));
    }
    const bool kvalid = l32 < nk;
    const int mypos = kpos + l32;
    const __bf16* Ksrc = static_cast<const __bf16*>(draft ? a.Kd : a.K);
    const __bf16* Vsrc = static_cast<const __bf16*>(draft ? a.Vd : a.V);
    const int64_t kaddr = ((int64_t)(krow + l32) * hkv + head) * D;
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint4 u = kvalid ? ld16(Ksrc + kaddr + 16 * t + 8 * h32) : make_uint4(0, 0, 0, 0);
      const uint4 v = kvalid ? ld16(Vsrc + kaddr + 16 * t + 8 * h32) : make_uint4(0, 0, 0, 0);
      kf[t] = __builtin_bit_cast(bf16x8, u);
      vf[t] = __builtin_bit_cast(bf16x8, v);
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;
    // wave-uniform key interval for skipping row tiles
    const int kp0 = kpos, kp1 = kpos + nk;

    const int r_begin = b0 * rows_per_block, r_end = b1 * rows_per_block;
    const int n_rt = (r_end - r_begin + 63) / 64;
    Quad qq, qo;
    auto load = [&](int rt) {
      if (!stager) return;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rho = r_begin + 64 * rt + 4 * sm + j;
        if (rho < r_end) {
          const int64_t row = (int64_t)(rho / G) * hq + head * G + rho % G;
          qq.v[j] = ld16(Qg + row * D + sdr * 8);
          qo.v[j] = ld16(dOg + row * D + sdr * 8);
        } else {
          qq.v[j] = qo.v[j] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto store = [&](int rt) {
      __bf16* buf = smem + (rt & 1) * L::bufElems;
      if (stager) {
        store_nat<D>(buf, sm, sdr, qq);
        store_nat<D>(buf + St::natElems, sm, sdr, qo);
        store_tr<D>(buf + 2 * St::natElems, sm, sdr, qq);
        store_tr<D>(buf + 2 * St::natElems + St::trElems, sm, sdr, qo);
      }
      if (tid < 64) {
        float* f = reinterpret_cast<float*>(buf + 2 * St::natElems + 2 * St::trElems);
        const int rho = r_begin + 64 * rt + tid;
        float l2 = __builtin_inff(), dd = 0.f;
        if (rho < r_end) {
          const int64_t row = (int64_t)(rho / G) * hq + head * G + rho % G;
          const float Lr = a.LSE[row];
          l2 = Lr == kNegInf ? __builtin_inff() : Lr * kLog2e;
          dd = a.ws_D[row];
        }
        f[tid] = l2;
        f[64 + tid] = dd;
      }
    };
    if (n_rt > 0) {
      load(0);
      store(0);
    }
    __syncthreads();
    for (int rt = 0; rt < n_rt; ++rt) {
      if (rt + 1 < n_rt) load(rt + 1);
      const __bf16* buf = smem + (rt & 1) * L::bufElems;
      const __bf16* Qn = buf;
      const __bf16* On = buf + St::natElems;
      const __bf16* Qt = buf + 2 * St::natElems;
      const __bf16* Ot = Qt + St::trElems;
      const float* lse2s = reinterpret_cast<const float*>(Ot + St::trElems);
      const float* Ds = lse2s + 64;
      const int rho0 = r_begin + 64 * rt;
      // does any row of this tile see any of this wave's keys?
      const int bA = rho0 / rows_per_block;
      const int bB = min(b1, (rho0 + 63) / rows_per_block + 1);
      bool any = false;
      for (int b = bA; b < bB && nk > 0; ++b) {
        if (draft) any = any || (b * kBlock < kp1 && (b + 1) * kBlock > kp0);
        else any = any || (max(los[b], kp0) < min(anchors[b], kp1));
      }
      if (any) {
        bf16x8 pb[2][2], dsb[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x16 sacc, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = dp[r] = 0.f;
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_nat<D>(Qn, qb * 32, l32, h32, t),
                                                           kf[t], sacc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_nat<D>(On, qb * 32, l32, h32, t),
                                                         vf[t], dp, 0, 0, 0);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r8 = qb * 32 + 8 * j;              // first of 8 rows, same block
            const int bj = (rho0 + r8) / rows_per_block;
            bool vis;
            if (draft) vis = kvalid && (mypos / kBlock) == bj;
            else vis = kvalid && bj < nb && mypos >= los[min(bj, nb - 1)] &&
                       mypos < anchors[min(bj, nb - 1)];
            const f32x4 l2 = *reinterpret_cast<const f32x4*>(lse2s + r8 + 4 * h32);
            const f32x4 dd = *reinterpret_cast<const f32x4*>(Ds + r8 + 4 * h32);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * j + i;
              const float p = vis ? exp2_fast(fmaf(sacc[r], c, -l2[i])) : 0.f;
              pb[qb][r >> 3][r & 7] = f32_to_bf16(p);
              dsb[qb][r >> 3][r & 7] = f32_to_bf16(p * (dp[r] - dd[i]));
            }
          }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  frag_tr<D>(Ot, db * 32, l32, h32, qb, t2), pb[qb][t2], dv[db], 0, 0, 0);
              dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  frag_tr<D>(Qt, db * 32, l32, h32, qb, t2), dsb[qb][t2], dk[db], 0, 0, 0);
            }
      }
      if (rt + 1 < n_rt) store(rt + 1);
      __syncthreads();
    }
    if (kvalid) {
      const int64_t orow = (int64_t)(krow + l32) * hkv + head;
      void* dKp = draft ? a.dKd : a.dK;
      void* dVp = draft ? a.dVd : a.dV;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = 32 * db + 8 * j + 4 * h32;
          if (a.grad_bf16) {
            bf16x4 wk, wv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              wk[i] = f32_to_bf16(dk[db][4 * j + i] * a.scale);
              wv[i] = f32_to_bf16(dv[db][4 * j + i]);
            }
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(dKp) + orow * D + d0) = wk;
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(dVp) + orow * D + d0) = wv;
          } else {
            f32x4 wk, wv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              wk[i] = dk[db][4 * j + i] * a.scale;
              wv[i] = dv[db][4 * j + i];
            }
            *reinterpret_cast<f32x4*>(static_cast<float*>(dKp) + orow * D + d0) = wk;
            *reinterpret_cast<f32x4*>(static_cast<float*>(dVp) + orow * D + d0) = wv;
          }
        }
    }
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.nb * kBlock * a.hq;
  constexpr int RPB = 256 / (D / 8);
  SKV_LAUNCH("bwd_pre", bwd_pre_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(256), 0, s,
                     static_cast<const __bf16*>(a.O), static_cast<const __bf16*>(a.dO), a.ws_D,
                     rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dq_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, DqLds<D>::bytes);
  if (e != hipSuccess) return e;
  SKV_LAUNCH("bwd_dq", bwd_dq_kernel<D>, dim3(a.n_wg), dim3(kQThreads), DqLds<D>::bytes, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.n_split > 0) {
    SKV_LAUNCH("dq_reduce", dq_reduce_kernel<D>, dim3(a.n_split * (kQTile / RPB)), dim3(256), 0, s,
                       a.sched, a.ws_dQ, a.dQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, KvLds<D>::bytes);
  if (e != hipSuccess) return e;
  SKV_LAUNCH("bwd_dkdv", bwd_dkdv_kernel<D>, dim3(a.n_wg), dim3(kKThreads), KvLds<D>::bytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  if (!a.dtype_bf16) return hipErrorNotSupported;
  return a.d == 128 ? launch_bwd_d<128>(a, s) : launch_bwd_d<64>(a, s);
}

}  // namespace skv
