// Fragment layouts shared by the attention kernels (forward and backward):
// bf16, 16 heads per group, d = 128, 64-key blocks, v_mfma_f32_16x16x32_bf16.
#pragma once

#include "common.hpp"

namespace infv2 {

constexpr int AT_D = 128;
constexpr int AT_G = 16;
constexpr int AT_B = 64;
constexpr int PACK_ELEMS = AT_B * AT_D;   // 8192 bf16 = 16 KB per block

// Key held by row r (0..15) of score tile t (0..3) of a 64-key block: the
// permutation makes a lane's 8 P^T elements of k-step ks the 8 consecutive
// keys 32*ks + 8*(lane>>4) .. +7.
__device__ __forceinline__ int tile_key(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}

// The 16-byte piece u (0..1023) of a block pack, from a block staged in LDS as
// rows [64 keys][row_stride bf16]:
//  key layout (f = 4t + ks):  lane l holds X[tile_key(t, l&15)][32ks + 8(l>>4) .. +7]
//  feature layout (f = 2mt + ks): lane l holds X[32ks + 8(l>>4) .. +7][16mt + (l&15)]
// with f = u >> 6, l = u & 63.  Fragment f is the 1 KB one MFMA operand load
// needs, in lane order.
__device__ __forceinline__ u32x4 pack_piece_keys(const uint16_t* x, int row_stride, int u) {
  const int f = u >> 6, l = u & 63;
  const int t = f >> 2, ks = f & 3;
  return *(const u32x4*)(x + tile_key(t, l & 15) * row_stride + 32 * ks + 8 * (l >> 4));
}
__device__ __forceinline__ u32x4 pack_piece_features(const uint16_t* x, int row_stride, int u) {
  const int f = u >> 6, l = u & 63;
  const int mt = f >> 1, ks = f & 1;
  const int d = 16 * mt + (l & 15), k0 = 32 * ks + 8 * (l >> 4);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = (uint32_t)x[(k0 + 2 * e) * row_stride + d] |
           ((uint32_t)x[(k0 + 2 * e + 1) * row_stride + d] << 16);
  return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace infv2
