// Main loop of the bf16-MFMA GEMMs (the exact NVFP4 path and the W4A16 path).
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), 128 x 128 per
// wave as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16.  K advances in tiles of 64
// elements: each operand tile is 256 rows x 64 bf16 (128 bytes per row) in LDS,
// 16-byte chunks XOR-swizzled by row, two stages, one barrier per K-tile.
//
// A loader policy turns global data into bf16 LDS rows:
//   Loader::load(kt)         issue the global reads of K-tile kt into registers
//   Loader::store(lds_a, lds_b)  convert those registers and write both tiles
// The conversion of tile kt+1 is issued in the same basic block as the MFMAs of
// tile kt, so the VALU work can overlap the matrix pipe.
#pragma once

#include "q4_epilogue.h"

namespace q4 {

constexpr int kBf16BM = 256, kBf16BN = 256;
constexpr int kBf16KT = 64;                 // K elements per K-tile
constexpr int kBf16RowBytes = kBf16KT * 2;  // 128 bytes of bf16 per tile row
constexpr int kBf16Threads = 256;
constexpr int kBf16GroupM = 4;

__device__ __forceinline__ int lds_chunk_off(int row, int chunk) {
  return row * kBf16RowBytes + ((chunk ^ (row & 7)) << 4);
}

// 16 MFMAs per step, 4 steps: the wave's 128 x 128 region over one 64-K tile.
// acc[f][g] holds D[n][m] (A operand = weight rows, B operand = activation rows).
__device__ __forceinline__ void bf16_tile_mma(v16f (&acc)[4][4], const uint8_t* la, const uint8_t* lb,
                                              int wx, int wy, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 pa[4], pb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = wx * 128 + 32 * g + r32;
      pa[g] = ld16(la + lds_chunk_off(row, 2 * s + h));
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int row = wy * 128 + 32 * f + r32;
      pb[f] = ld16(lb + lds_chunk_off(row, 2 * s + h));
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = mfma_bf16_32x32x16(pb[f], pa[g], acc[f][g]);
  }
}

template <class Loader>
__device__ __forceinline__ void bf16_mainloop(v16f (&acc)[4][4], Loader& ld, int64_t K, uint8_t* lds,
                                              int wx, int wy, int lane) {
  constexpr int kTile = kBf16BM * kBf16RowBytes;   // bytes per operand tile
  uint8_t* stage_ptr[2] = {lds, lds + 2 * kTile};
  const int nkt = (int)((K + kBf16KT - 1) / kBf16KT);
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = v16f{};
  if (nkt > 0) {
    ld.load(0);
    ld.store(stage_ptr[0], stage_ptr[0] + kTile);
    if (nkt > 1) ld.load(1);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    uint8_t* cur = stage_ptr[kt & 1];
    uint8_t* nxt = stage_ptr[(kt & 1) ^ 1];
    if (kt + 1 < nkt) ld.store(nxt, nxt + kTile);
    if (kt + 2 < nkt) ld.load(kt + 2);
    bf16_tile_mma(acc, cur, cur + kTile, wx, wy, lane);
    __syncthreads();
  }
}

}  // namespace q4
