// Weight-only W4A16 GEMM: bf16 activations times int4 weights (asymmetric, group
// 64 along K, bf16 scale and zero point), dequantized tile by tile into LDS as
// w_hat = bf16((q - z) * s) and multiplied on the bf16 MFMA.  The K-tile is one
// quantization group, so each weight row of a tile has a single (s, z).
#include "gemm_bf16_core.h"

namespace q4 {

// 32 int4 codes (16 bytes) -> 4 chunks of bf16: (q - z) * s is exact in fp32
// (fma(q, s, -z s) with an exact z s), then one round to nearest even to bf16.
__device__ __forceinline__ void int4_dequant_chunk(u32x4 codes, float s, float zs, u32x4* out4) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = codes[d] & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 of the dword
    const uint32_t hi = (codes[d] >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
    uint32_t o[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float q0 = (float)((lo >> (8 * b)) & 0xFFu);
      const float q1 = (float)((hi >> (8 * b)) & 0xFFu);
      const v2bf p = {(__bf16)__builtin_fmaf(q0, s, -zs), (__bf16)__builtin_fmaf(q1, s, -zs)};
      o[b] = __builtin_bit_cast(uint32_t, p);
    }
    out4[d] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

struct W4A16Loader {
  const uint16_t* x; int64_t ldx;
  const uint8_t* wc; const uint16_t* ws; const uint16_t* wz;
  int64_t M, N, K, m0, n0;
  int tid;
  u32x4 xa[8], cb[2];
  uint32_t sb[2], zb[2];

  __device__ __forceinline__ void load(int kt) {
    // activations: 256 rows x 8 chunks of 8 bf16; chunk (row, c) with c = tid & 7
    const int c = tid & 7;
    const int64_t k = (int64_t)kt * kBf16KT + 8 * c;
    const bool kxok = k < K;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = (tid >> 3) + 32 * j;
      xa[j] = (kxok && m0 + row < M) ? ld16(x + (m0 + row) * ldx + k) : u32x4{0, 0, 0, 0};
    }
    // weights: 256 rows x 2 chunks of 32 codes; one group (s, z) per row
    const int cw = tid & 1;
    const int64_t kb = K >> 1, ngrp = K >> 6;
    const bool kwok = kt < ngrp;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = (tid >> 1) + 128 * j;
      const bool ok = kwok && n0 + row < N;
      cb[j] = ok ? ld16(wc + (n0 + row) * kb + (int64_t)kt * 32 + 16 * cw) : u32x4{0, 0, 0, 0};
      sb[j] = ok ? ws[(n0 + row) * ngrp + kt] : 0u;
      zb[j] = ok ? wz[(n0 + row) * ngrp + kt] : 0u;
    }
  }
  __device__ __forceinline__ void store(uint8_t* la, uint8_t* lb) {
    const int c = tid & 7;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = (tid >> 3) + 32 * j;
      st16(la + lds_chunk_off(row, c), xa[j]);
    }
    const int cw = tid & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = (tid >> 1) + 128 * j;
      const float s = __uint_as_float(sb[j] << 16);
      const float zs = __uint_as_float(zb[j] << 16) * s;
      u32x4 o[4];
      int4_dequant_chunk(cb[j], s, zs, o);
#pragma unroll
      for (int d = 0; d < 4; ++d) st16(lb + lds_chunk_off(row, 4 * cw + d), o[d]);
    }
  }
};

template <bool OUT_F32>
__global__ __launch_bounds__(kBf16Threads, 1) void gemm_w4a16_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n) {
  constexpr int kMainLds = 4 * kBf16BM * kBf16RowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMainLds > kEpilogueLdsBytes ? kMainLds : kEpilogueLdsBytes];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, kBf16GroupM, &tm, &tn);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  W4A16Loader ld;
  ld.x = x; ld.ldx = ldx; ld.wc = wc; ld.ws = ws; ld.wz = wz;
  ld.M = M; ld.N = N; ld.K = K;
  ld.m0 = (int64_t)tm * kBf16BM; ld.n0 = (int64_t)tn * kBf16BN;
  ld.tid = tid;
  v16f acc[4][4];
  bf16_mainloop(acc, ld, K, lds, wx, wy, lane);
  const int64_t n_base = ld.n0 + wy * 128, m_base = ld.m0 + wx * 128;
  __syncthreads();                           // all waves are done reading operand tiles
  epilogue_store<OUT_F32>(acc, n_base, m_base, M, N, bias, y, ldy, lane, lds + wave * kStageWaveBytes);
}

hipError_t launch_gemm_w4a16(const uint16_t* x, int64_t ldx, const uint8_t* wc,
                             const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                             int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kBf16BM - 1) / kBf16BM), tiles_n = (int)((N + kBf16BN - 1) / kBf16BN);
  if (ep.out_f32)
    hipLaunchKernelGGL(gemm_w4a16_kernel<true>, dim3(tiles_m * tiles_n), dim3(kBf16Threads), 0, s, x,
                       ldx, wc, ws, wz, M, N, K, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(gemm_w4a16_kernel<false>, dim3(tiles_m * tiles_n), dim3(kBf16Threads), 0, s, x,
                       ldx, wc, ws, wz, M, N, K, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace q4
