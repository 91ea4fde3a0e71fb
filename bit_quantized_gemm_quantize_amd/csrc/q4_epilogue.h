// Epilogue shared by the GEMM kernels.  The main loop leaves a wave with a 4 x 4
// grid of 32x32 fp32 accumulators laid out as D[n][m] (MFMA A operand = weight
// rows n, B operand = activation rows m), so lane l holds output row m = l%32 of
// each tile and, per register group v/4, four consecutive output columns n: the
// stores are 8-byte (bf16) or 16-byte (fp32) runs along a row of Y.
//
// Order of the epilogue: (optional) scale, low-rank up-projection t L2 as bf16
// MFMAs on the same accumulators with t split into bf16 hi + lo, bias, store.
#pragma once

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

// acc[f][g]: f = weight (n) sub-tile, g = activation (m) sub-tile, 32 x 32 each.
// n_base / m_base: first n / m of the wave's 128 x 128 region.
template <int R>
__device__ __forceinline__ void epilogue_lowrank(v16f (&acc)[4][4], int64_t n_base, int64_t m_base,
                                                 int64_t M, int64_t N, const float* __restrict__ t,
                                                 const uint16_t* __restrict__ l2t, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < R / 16; ++ks) {
    u32x4 thi[4], tlo[4], l2f[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t m = m_base + 32 * g + r32;
      thi[g] = u32x4{0, 0, 0, 0};
      tlo[g] = u32x4{0, 0, 0, 0};
      if (m < M) {
        const float* src = t + m * R + 16 * ks + 8 * h;
        const u32x4 a = ld16(src), b = ld16(src + 4);
        const uint32_t tv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = __uint_as_float(tv[j]);
          hi[j] = f32_to_bf16_rne(v);
          lo[j] = f32_to_bf16_rne(v - __uint_as_float(hi[j] << 16));
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          thi[g][d] = hi[2 * d] | (hi[2 * d + 1] << 16);
          tlo[g][d] = lo[2 * d] | (lo[2 * d + 1] << 16);
        }
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t n = n_base + 32 * f + r32;
      l2f[f] = (n < N) ? ld16(l2t + n * R + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[f][g] = mfma_bf16_32x32x16(l2f[f], thi[g], acc[f][g]);
        acc[f][g] = mfma_bf16_32x32x16(l2f[f], tlo[g], acc[f][g]);
      }
  }
}

template <bool OUT_F32>
__device__ __forceinline__ void epilogue_store(v16f (&acc)[4][4], int64_t n_base, int64_t m_base,
                                               int64_t M, int64_t N,
                                               const uint16_t* __restrict__ bias, void* y,
                                               int64_t ldy, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      const int64_t n = n_base + 32 * f + 8 * vq + 4 * h;   // first of 4 consecutive columns
      float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (bias) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < N) b[j] = __uint_as_float((uint32_t)bias[n + j] << 16);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t m = m_base + 32 * g + r32;
        if (m >= M) continue;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[f][g][4 * vq + j] + b[j];
        if (OUT_F32) {
          float* dst = static_cast<float*>(y) + m * ldy + n;
          if (n + 3 < N) {
            *reinterpret_cast<v4f*>(dst) = v4f{v[0], v[1], v[2], v[3]};
          } else {
            for (int j = 0; j < 4; ++j)
              if (n + j < N) dst[j] = v[j];
          }
        } else {
          uint16_t* dst = static_cast<uint16_t*>(y) + m * ldy + n;
          const v2bf p0 = {(__bf16)v[0], (__bf16)v[1]};
          const v2bf p1 = {(__bf16)v[2], (__bf16)v[3]};
          if (n + 3 < N) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2*>(dst) =
                u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
          } else {
            const uint32_t w0 = __builtin_bit_cast(uint32_t, p0), w1 = __builtin_bit_cast(uint32_t, p1);
            const uint16_t e[4] = {(uint16_t)(w0 & 0xFFFF), (uint16_t)(w0 >> 16), (uint16_t)(w1 & 0xFFFF),
                                   (uint16_t)(w1 >> 16)};
            for (int j = 0; j < 4; ++j)
              if (n + j < N) dst[j] = e[j];
          }
        }
      }
    }
  }
}

}  // namespace q4
