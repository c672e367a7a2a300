// Direct-to-LDS tile staging and LDS fragment reads (gfx950 kernels).
//
// Tiles of 64 rows x D bf16 (rows are keys or query rows) are copied from
// HBM into LDS with global_load_lds_dwordx4: every lane of a wave moves 16
// bytes and writes them at lds_base + 16 * lane.  Because each lane chooses
// its own global address, a tile can be written directly in the order the
// MFMAs consume it, in one of two layouts (both 64 x D x 2 bytes):
//
//   fragment-major  1 KB block (kb, t), kb in {0,1}, t < D/16, holds the A
//                   operand of a 32x32x16 MFMA with lane = row: lane L's 16
//                   bytes are row 32 kb + L % 32, columns 16 t + 8 (L / 32).
//   block-major     4-row quads (8 D bytes each) of 4 x 16 blocks (128 bytes,
//                   row-major inside).  A 16-lane ds_read_b64_tr_b16 over one
//                   block returns, in lane i, column i of its 4 rows; two such
//                   reads form the A operand with lane = column and the 8
//                   rows {4h + 0..3, 8 + 4h + 0..3} that a 32x32 accumulator
//                   lane (half h) holds, so results feed MFMAs without any
//                   register transpose.
//
// Reads are contiguous per instruction (no bank conflicts) and use one base
// register plus an immediate offset.  The DMA is issued as inline asm so the
// compiler neither waits on it nor serialises it against LDS reads; kernels
// wait with explicit vmcnt counts and a bare s_barrier.
#pragma once
#include "device_common.h"

namespace skv {

typedef short short4v __attribute__((ext_vector_type(4)));

template <int D>
struct Tile {
  static constexpr int kBytes = kTileK * D * 2;   // 16 KB for d = 128
  static constexpr int kBlocks = kBytes / 1024;   // DMA blocks per tile
  static constexpr int kFragsPerKb = D / 16;      // fragment-major: t range
  static constexpr int kQuadBytes = 4 * D * 2;    // block-major: one 4-row quad
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane;
// lds_base must be wave-uniform.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt vmcnt(n) (n < 16), leaving lgkmcnt/expcnt alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
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

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
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

// Row and column that byte 16*lane of DMA block u carries, per layout.
template <int D>
__device__ __forceinline__ void frag_major_rc(int u, int lane, int& row, int& col) {
  row = (u / Tile<D>::kFragsPerKb) * 32 + (lane & 31);
  col = 16 * (u % Tile<D>::kFragsPerKb) + 8 * (lane >> 5);
}
template <int D>
__device__ __forceinline__ void block_major_rc(int u, int lane, int& row, int& col) {
  const int byte = u * 1024 + 16 * lane;
  const int q = byte / Tile<D>::kQuadBytes, w = byte % Tile<D>::kQuadBytes;
  row = 4 * q + (w & 127) / 32;
  col = 16 * (w / 128) + 8 * ((w & 31) / 16);
}

// Per-lane byte offset of the transposed read within a block-major tile: the
// 16-lane group G = lane / 16 reads quad (base + G / 2), block (2 db + G % 2).
template <int D>
__device__ __forceinline__ uint32_t tr_lane_offset(int lane) {
  return (lane >> 5) * Tile<D>::kQuadBytes + ((lane >> 4) & 1) * 128 + 8 * (lane & 15);
}

// A operand (lane = column d = 32 db + lane % 32) for rows
// 32 rb + 16 t2 + {4h + 0..3, 8 + 4h + 0..3} of a block-major tile at `base`
// (base already includes tr_lane_offset).
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(uint32_t base, int db, int rb, int t2) {
  const uint32_t q0 = base + (8 * rb + 4 * t2) * Tile<D>::kQuadBytes + db * 256;
  const short4v lo4 = ds_read_tr(q0);
  const short4v hi4 = ds_read_tr(q0 + 2 * Tile<D>::kQuadBytes);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand (lane = row 32 kb + lane % 32) of d-step t of a fragment-major
// tile at `base` (base already includes 16 * lane).
template <int D>
__device__ __forceinline__ bf16x8 frag_nat(uint32_t base, int kb, int t) {
  return lds_read16(base + (kb * Tile<D>::kFragsPerKb + t) * 1024);
}

// ---------------------------------------------------------------------------
// Rotated fragment-major tile: one copy that serves both the natural A
// operand (lane = row) and the transposed one (lane = column).  Fragment
// (kb, t) sits at (kb * D/16 + t) * 1088 bytes; slot s < 32 holds row
// 32 kb + s, columns 16 t .. +7; slot s >= 32 holds row 32 kb + ((s - 24) & 31),
// columns 16 t + 8 .. +15 (the second half rotated by 8 rows).  The rotation
// puts the two column halves of a row 128 bytes apart modulo the 256-byte
// bank window and the 64-byte fragment skew separates neighbouring fragments,
// so 32 lanes of a transposed read touch 256 distinct bytes.
template <int D>
struct RTile {
  static constexpr int kFragStride = 1088;
  static constexpr int kFrags = 2 * (D / 16);
  static constexpr int kBytes = kFrags * kFragStride;
};

// Row/column of DMA lane `lane` for fragment u (written at u * kFragStride).
template <int D>
__device__ __forceinline__ void rot_major_rc(int u, int lane, int& row, int& col) {
  row = (u / (D / 16)) * 32 + (lane < 32 ? lane : ((lane - 24) & 31));
  col = 16 * (u % (D / 16)) + 8 * (lane >> 5);
}

// Natural read: lane L's 16 bytes of fragment (kb, t) are at
// base + (kb * D/16 + t) * 1088 with base = tile + rot_nat_offset(L).
__device__ __forceinline__ uint32_t rot_nat_offset(int lane) {
  return 16 * (lane < 32 ? lane : 32 + ((lane - 40) & 31));
}
template <int D>
__device__ __forceinline__ bf16x8 rot_frag_nat(uint32_t base, int kb, int t) {
  return lds_read16(base + (kb * (D / 16) + t) * RTile<D>::kFragStride);
}

// Transposed read (lane = column 32 db + lane % 32, rows of 32-row block rb
// at k-step t2).  Source lane j = lane % 16 supplies row 4h + j / 4 (+16 t2,
// +8 for the second read) and columns 4 (j % 4) .. +3 of its 16-column group.
// Rows 0..7 of a block wrap in the rotated half, so the first read of t2 = 0
// uses its own lane offset (A); every other read uses offset B.
__device__ __forceinline__ uint32_t rot_tr_offset_a(int lane) {
  const int j = lane & 15, m = j >> 2, q = j & 3, half = q >> 1;
  return 16 * (56 * half + 4 * (lane >> 5) + m) + 8 * (q & 1) + 1088 * ((lane >> 4) & 1);
}
__device__ __forceinline__ uint32_t rot_tr_offset_b(int lane) {
  const int j = lane & 15, m = j >> 2, q = j & 3, half = q >> 1;
  return 16 * (24 * half + 4 * (lane >> 5) + m) + 8 * (q & 1) + 1088 * ((lane >> 4) & 1);
}
template <int D>
__device__ __forceinline__ bf16x8 rot_frag_tr(uint32_t base_a, uint32_t base_b, int db, int rb,
                                              int t2) {
  const uint32_t f = (rb * (D / 16) + 2 * db) * RTile<D>::kFragStride;
  const short4v lo4 = t2 == 0 ? ds_read_tr(base_a + f) : ds_read_tr(base_b + f + 256 * t2);
  const short4v hi4 = ds_read_tr(base_b + f + 256 * t2 + 128);
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
