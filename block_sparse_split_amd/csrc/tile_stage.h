// Staging of 64-row bf16 tiles from HBM into LDS (gfx950 kernels).
//
// A thread owns a "quad": rows 4m .. 4m+3 of a 64-row tile at columns
// 8*dr .. 8*dr+7 (four 16-byte loads; consecutive threads take consecutive
// column groups of the same rows, so a wave reads whole 256-byte rows).  The
// quad is written to LDS in one or both of two layouts:
//   natural     [row][col]            row pitch D + 8 elements;
//   transposed  [col][row-permuted]   row pitch 64 + 8 elements, where rows
//     4m..4m+3 of each 16-row group are stored at offset 0, 8, 4, 12 for
//     m % 4 = 0, 1, 2, 3.
// The permutation makes the 8 bf16 that one lane of a 32x32x16 MFMA needs as
// its A operand contiguous when the matching B operand comes straight out of
// a 32x32 accumulator (whose lanes hold rows 8j + 4*(lane/32) + i).  The
// pitches add 16 bytes per row so that 16 lanes reading 16 bytes each at
// the same column of consecutive rows hit distinct LDS banks.
#pragma once
#include "device_common.h"

namespace skv {

template <int D>
struct Stage {
  static constexpr int natPitch = D + 8;
  static constexpr int trPitch = kTileK + 8;
  static constexpr int natElems = kTileK * natPitch;
  static constexpr int trElems = D * trPitch;
  static constexpr int CPR = D / 8;                 // 16-byte column groups
  static constexpr int nQuads = (kTileK / 4) * CPR;  // quads per 64-row tile
};

struct Quad {
  uint4 v[4];
};

__device__ __forceinline__ uint4 ld16(const __bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ uint32_t half_of(const uint4& u, int e) {
  const uint32_t word = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
  return (e & 1) ? (word >> 16) : (word & 0xFFFFu);
}

__device__ __forceinline__ int quad_perm(int m) {
  return 16 * (m >> 2) + ((m & 1) ? 8 : 0) + ((m & 2) ? 4 : 0);
}

template <int D>
__device__ __forceinline__ void store_nat(__bf16* buf, int m, int dr, const Quad& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint4*>(buf + (4 * m + j) * Stage<D>::natPitch + dr * 8) = q.v[j];
}

template <int D>
__device__ __forceinline__ void store_tr(__bf16* buf, int m, int dr, const Quad& q) {
  const int pos = quad_perm(m);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint2 w;
    w.x = half_of(q.v[0], e) | (half_of(q.v[1], e) << 16);
    w.y = half_of(q.v[2], e) | (half_of(q.v[3], e) << 16);
    *reinterpret_cast<uint2*>(buf + (dr * 8 + e) * Stage<D>::trPitch + pos) = w;
  }
}

// A-operand fragment of a 32x32x16 MFMA from a natural-layout tile:
// lane (row = r0 + l32, half h32) gets columns 16*t + 8*h32 .. +7.
template <int D>
__device__ __forceinline__ bf16x8 frag_nat(const __bf16* buf, int r0, int l32, int h32, int t) {
  return *reinterpret_cast<const bf16x8*>(buf + (r0 + l32) * Stage<D>::natPitch + 16 * t +
                                          8 * h32);
}

// A-operand fragment from a transposed tile: lane (column = c0 + l32) gets
// the 8 permuted rows of k-step (kb, t2) for its half.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* buf, int c0, int l32, int h32, int kb,
                                          int t2) {
  return *reinterpret_cast<const bf16x8*>(buf + (c0 + l32) * Stage<D>::trPitch + kb * 32 +
                                          t2 * 16 + 8 * h32);
}

}  // namespace skv
