// Layouts of the per-frame state increments (-G, B of the affine state update)
// that the gram kernels write and the state scan reads, shared by
// state_bf16.hip (increments of K', V') and fmap.hip (increments under the
// feature maps).
#pragma once

#include "ha_device.h"

namespace ha {

// Workspace per (b, h, frame), in the scan's MFMA fragment order:
//   G hi : [band i (NRB)][k-step (D/16)][lane] 16 bytes  (8 bf16 of -G)
//   G lo : the same for the low halves
//   B    : [col block (NRB)][row band (NRB)][lane] 64 bytes (16 fp32)
// G is symmetric, so the accumulator registers [8s, 8s+8) of the block
// (row band kb, column block rb) are the scan's A fragment of -G for output
// band rb and k-step 2*kb + s, under the contraction order in which k-slot
// 8*hh + e of that step is k = 32*kb + 16*s + 8*(e/4) + 4*hh + e%4.
// g8: accumulator elements [8*sh, 8*sh + 8) of the G block (row band rb,
// column block cb) of one lane; -G is split into bf16 hi + lo.
template <int D>
__device__ __forceinline__ void store_g_half(unsigned char* base, int rb, int cb, int sh, int lane,
                                             const float* g8) {
  constexpr int KS = D / 16;
  u32x4 hi, lo;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const float x0 = -g8[2 * w2], x1 = -g8[2 * w2 + 1];
    const uint32_t hp = pack_bf16x2(x0, x1);
    hi[w2] = hp;
    lo[w2] = pack_bf16x2(x0 - bf16_lo_to_f32(hp), x1 - bf16_hi_to_f32(hp));
  }
  const size_t fo = (size_t)(cb * KS + 2 * rb + sh) * 64 + lane;
  reinterpret_cast<u32x4*>(base)[fo] = hi;
  reinterpret_cast<u32x4*>(base + (size_t)D * D * 2)[fo] = lo;
}
// B block (row band rb, column block cb): accumulator elements [4*v4, 4*v4+4)
template <int D>
__device__ __forceinline__ void store_b4(unsigned char* base, int rb, int cb, int v4, int lane, f32x4 x) {
  constexpr int NRB = D / 32;
  reinterpret_cast<f32x4*>(base + (size_t)D * D * 4)[((size_t)(cb * NRB + rb) * 64 + lane) * 4 + v4] = x;
}
// fp32 partial sums of one split: [row band][col block][G, B][v4][lane] f32x4
template <int D>
__device__ __forceinline__ f32x4* partial_block(float* partial, size_t group_split, int rb, int cb) {
  constexpr int NRB = D / 32;
  return reinterpret_cast<f32x4*>(partial) + ((group_split * NRB + rb) * NRB + cb) * 2 * 4 * 64;
}

}  // namespace ha
