// Direct-to-LDS tile staging and LDS operand reads (gfx950 kernels).
//
// Tiles of 64 rows x D bf16 (rows are keys or query rows) are copied from
// HBM into LDS with buffer_load_dwordx4 ... lds: every lane of a wave moves
// 16 bytes and writes them at lds_base + 16 * lane.  All tiles use one
// layout (the interleaved row tile below): each DMA instruction moves whole
// rows, and MFMA operands are read either naturally (lane = row,
// ds_read_b128) or transposed (lane = column, ds_read_b64_tr_b16) without
// bank conflicts and without any register transpose.  Reads use one base
// register plus an immediate offset.  The DMA is issued as inline asm so the
// compiler neither waits on it nor serialises it against LDS reads; kernels
// wait with explicit vmcnt counts and a bare s_barrier.
#pragma once
#include "device_common.h"

namespace skv {

typedef short short4v __attribute__((ext_vector_type(4)));

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over the bytes [base, base + bytes) of global memory
// (bytes above 2^32 - 1 are clamped).  A buffer load's range check covers
// voffset + soffset: a lane whose offset lands at or past `bytes` reads no
// memory and its 16 LDS bytes become zero.  base and bytes must be
// wave-uniform.
__device__ __forceinline__ i32x4 buf_res(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  // 32-bit halves the optimiser cannot fuse back into a 64-bit compare keep
  // the clamp on the scalar unit
  uint32_t lo = (uint32_t)bytes, hi = (uint32_t)((uint64_t)bytes >> 32);
  asm volatile("" : "+s"(lo), "+s"(hi));
  const uint32_t n = (int32_t)hi < 0 ? 0u : hi != 0 ? 0xFFFFFFFFu : lo;
  // word 1: base[47:32], stride 0; word 3: 32-bit data format, no swizzle
  i32x4 r = {(int32_t)(uint32_t)b, (int32_t)((b >> 32) & 0xFFFFu), (int32_t)n, 0x00020000};
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
  return r;
}

// 16 bytes per lane from buffer `res` at byte offset voff + soff into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds).  The per-lane part of
// the address is one 32-bit register and the rest is scalar, so issuing
// costs no vector ALU work.  soff and lds_base must be wave-uniform.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_buf(const i32x4& res, uint32_t voff, uint32_t soff,
                                          uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(res), "s"(soff), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt vmcnt(n) (n < 64: bits 3:0 and 15:14 of the immediate), leaving
// lgkmcnt/expcnt alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Start and end of a workgroup on the constant-rate (100 MHz) clock, for
// measuring the realised balance of a plan, with the hardware ids of where
// it ran (XCC_ID and HW_ID registers: XCD, shader engine, CU, SIMD); `clk`
// is null unless a caller asked for the stamps (then each workgroup writes
// its four words).
__device__ __forceinline__ uint64_t wg_clock_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID, 32 bits
}
// Entry v of the stamps belongs to queue v (the workgroup that ran it).
__device__ __forceinline__ void wg_clock_record(unsigned long long* clk, uint64_t t0, int v) {
  if (clk == nullptr) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    const uint32_t xcc = hw_xcc_id();
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID, 32 bits
    clk[4 * v] = t0;
    clk[4 * v + 1] = t1;
    clk[4 * v + 2] = xcc;
    clk[4 * v + 3] = hw;
  }
}

// The queue this workgroup runs (see schedule.h): its own index, unless
// the schedule has per-XCD queues and `count` (this kernel's kXcds per-XCD
// counters, zero at launch) is given.  Then thread 0 reads the XCD it runs
// on, x, and takes the next free queue of x, v = x + kXcds * slot, or of
// the next XCD when all of x's are taken (a failed try only raises that
// counter).  With n_wg workgroups claiming, counters starting at zero and
// n_wg / kXcds queues per XCD, every workgroup finds a queue within kXcds
// tries (if all its tries failed, every XCD's queues would be held by
// other workgroups, n_wg of them) and no queue is taken twice.
__device__ __forceinline__ int claim_queue(sched_t S, uint32_t* count) {
  if (count == nullptr || S[H_XCD] == 0) return blockIdx.x;
  __shared__ int v_claimed;
  if (threadIdx.x == 0) {
    const int per = S[H_NWG] / kXcds;
    const int x = int(hw_xcc_id() & 0xF) % kXcds;
    int v = blockIdx.x;  // kept only if the counters did not start at zero
    for (int i = 0; i < kXcds; ++i) {
      const int y = (x + i) % kXcds;
      const uint32_t slot = atomicAdd(&count[y], 1u);
      if (slot < uint32_t(per)) {
        v = y + kXcds * int(slot);
        break;
      }
    }
    v_claimed = v;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(v_claimed);
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// An LDS byte address the optimiser cannot see through, so that each read
// becomes `base + immediate` rather than one hoisted address register per read.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
      static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ void lds_write16(uint32_t addr, const bf16x8& v) {
  *reinterpret_cast<__attribute__((address_space(3))) bf16x8*>(static_cast<uintptr_t>(addr)) = v;
}

__device__ __forceinline__ int32_t lds_read_i32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) int32_t*>(
      static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ i32x4 lds_read_i4(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(
      static_cast<uintptr_t>(addr));
}

// s_waitcnt lgkmcnt(0): this wave's LDS writes have completed (before a
// barrier that publishes them to other waves).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ f32x4 lds_read_f4(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
      static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ short4v ds_read_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(static_cast<uintptr_t>(addr)));
}

// ---------------------------------------------------------------------------
// Interleaved row tile: the one LDS layout of every K, V, Q and dO tile.
// A DMA instruction moves whole rows: lane i of block g reads 16 bytes
// (8 columns) of row g*RB + i % RB, column chunk i / RB, where RB = 1024 /
// (2 D) rows fill one 1 KB block (RB = 4 for d = 128, 8 for d = 64), so each
// instruction covers 8 full 128-byte lines of K/V rows.  In LDS, block g
// sits at g * (1024 + 16 RB): the 16-byte chunk c of row r is at
//   (r / RB) * (1024 + 16 RB) + (c * RB + r % RB) * 16.
// The chunk of 16 consecutive rows then falls in 16 distinct 16-byte bank
// groups (natural reads: lane = row), and 4 rows x 32 columns of a
// transposed read fall in distinct banks for d = 128.
template <int D>
struct ITile {
  static constexpr int kRB = 1024 / (2 * D);
  static constexpr int kBlockStride = 1024 + 16 * kRB;
  static constexpr int kBlocks = kTileK / kRB;
  static constexpr int kBytes = kBlocks * kBlockStride;
};

// Row and column (first of 8) that DMA lane `lane` of block g carries.
template <int D>
__device__ __forceinline__ void itile_rc(int g, int lane, int& row, int& col) {
  row = g * ITile<D>::kRB + lane % ITile<D>::kRB;
  col = 8 * (lane / ITile<D>::kRB);
}

template <int D>
__device__ __forceinline__ uint32_t itile_addr(int row, int chunk) {
  using T = ITile<D>;
  return (row / T::kRB) * T::kBlockStride + (chunk * T::kRB + row % T::kRB) * 16;
}

// Natural A operand (lane = row 32 kb + lane % 32, columns 16 t + 8 (lane /
// 32) .. +7): base = tile + itile_nat_offset(lane).
template <int D>
__device__ __forceinline__ uint32_t itile_nat_offset(int lane) {
  return itile_addr<D>(lane & 31, lane >> 5);
}
template <int D>
__device__ __forceinline__ bf16x8 itile_nat(uint32_t base, int kb, int t) {
  using T = ITile<D>;
  return lds_read16(base + kb * (32 / T::kRB) * T::kBlockStride + t * 2 * T::kRB * 16);
}

// Transposed A operand (lane = column 32 db + lane % 32; its 8 k values are
// rows 32 rb + 16 t2 + {4 h + 0..3, 8 + 4 h + 0..3}, h = lane / 32, the row
// order of a 32x32 accumulator lane): two ds_read_b64_tr_b16, each over 4
// rows.  Source lane j of 16-lane group G reads row 4 h + j / 4, columns
// 16 (G % 2) + 4 (j % 4) .. +3.
template <int D>
__device__ __forceinline__ uint32_t itile_tr_offset(int lane) {
  const int j = lane & 15, grp = (lane >> 4) & 1, h = lane >> 5;
  const int row = 4 * h + j / 4, col = 16 * grp + 4 * (j % 4);
  return itile_addr<D>(row, col / 8) + ((col % 8) / 4) * 8;
}
template <int D>
__device__ __forceinline__ bf16x8 itile_tr(uint32_t base, int db, int rb, int t2) {
  using T = ITile<D>;
  const uint32_t c = ((32 * rb + 16 * t2) / T::kRB) * T::kBlockStride + 4 * db * T::kRB * 16;
  const short4v lo4 = ds_read_tr(base + c);
  const short4v hi4 = ds_read_tr(base + c + (8 / T::kRB) * T::kBlockStride);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

// N MFMAs whose A operands come from LDS, with P reads kept in flight:
// read(i) returns operand i (i is a compile-time constant after unrolling),
// mfma(i, a) issues MFMA i.  A scheduling barrier before every MFMA stops
// the compiler from moving each read next to its consumer, so the read
// latency hides behind the P MFMAs issued in between.
template <int N, int P, class Read, class Mfma>
__device__ __forceinline__ void lds_pipelined(Read read, Mfma mfma) {
  bf16x8 buf[P];
#pragma unroll
  for (int i = 0; i < P && i < N; ++i) buf[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 a = buf[i % P];
    if (i + P < N) buf[i % P] = read(i + P);
    mfma(i, a);
  }
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace skv
