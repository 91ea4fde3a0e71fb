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
    uint32_t lo = codes[d] & 0x0F0F0F0Fu;                // codes 0, 2, 4, 6 of the dword
    uint32_t hi = (codes[d] >> 4) & 0x0F0F0F0Fu;         // codes 1, 3, 5, 7
    // opaque to the compiler: it would otherwise see 4-bit fields and extract each
    // code with a bit-field extract before converting, where the byte-select
    // conversion (v_cvt_f32_ubyte0..3) reads the byte directly
    asm volatile("" : "+v"(lo), "+v"(hi));
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

// Per K-tile (one quantization group of 64 K): the activation tile (256 rows x 128
// bytes of bf16) goes straight into LDS, each wave moving rows 64 w .. 64 w + 63 as
// 8 rows x 128 bytes per instruction (lane i -> row i/8, stored position i%8, which
// holds global chunk (i%8) ^ lds_swz<8>(row)); the weight tile is TN rows x 2 chunks of
// 32 codes, thread tid owning chunk tid & 1 of rows tid/2 (and tid/2 + THREADS/2),
// with each row's (s, z).  Reads past M / N / K, and rows past TN, return zeros.
// SETS register sets of weight codes and (s, z) rotate, so that a weight load is
// issued SETS K-tiles before its conversion.  THREADS: 256 (4 waves) or 512 (8).
template <int TN, int SETS, int THREADS = 256>
struct W4A16Loader {
  static constexpr int kSets = SETS;
  static constexpr int kRowsPerGroup = THREADS / 2;
  static constexpr int kRowGroups = (TN + kRowsPerGroup - 1) / kRowsPerGroup;   // weight rows per thread
  static constexpr int kRowsPerWave = kBf16BM / (THREADS / 64);               // activation rows per wave
  static constexpr int kValuPerStore = 48;   // VALU ops spread over one store part's MFMAs (tuned)
  static constexpr int kRegLoads = 3 * kRowGroups;   // VMEM instructions of issue_regs
  static constexpr bool kLateStores = false;
  static constexpr bool kF16 = false;         // bf16 operands and MFMA
  __amdgpu_buffer_rsrc_t rx, rc, rs, rz;
  uint32_t ldxb, kb, ngrp;
  int tid;
  u32x4 cb[SETS][kRowGroups];
  uint32_t sb[SETS][kRowGroups], zb[SETS][kRowGroups];

  __device__ __forceinline__ void init(const uint16_t* x, int64_t ldx, const uint8_t* wc,
                                       const uint16_t* ws, const uint16_t* wz, int64_t M,
                                       int64_t N, int64_t K, int64_t m0, int64_t n0, int t) {
    ldxb = (uint32_t)(ldx * 2); kb = (uint32_t)(K >> 1); ngrp = (uint32_t)(K >> 6);
    const uint32_t ra = rows_in(kBf16BM, M, m0), rb = rows_in(TN, N, n0);
    // the last activation row ends at K, not at ldx
    rx = make_rsrc(x + m0 * ldx, ra > 0 ? (ra - 1) * ldxb + (uint32_t)(K * 2) : 0);
    rc = make_rsrc(wc + n0 * kb, rb * kb);
    rs = make_rsrc(ws + n0 * ngrp, rb * ngrp * 2);
    rz = make_rsrc(wz + n0 * ngrp, rb * ngrp * 2);
    tid = t;
  }
  __device__ __forceinline__ void issue_lds(int kt, uint8_t* la, uint8_t*) {
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t lr = lane >> 3, lp = lane & 7;
#pragma unroll
    for (int j = 0; j < kRowsPerWave / 8; ++j) {
      // kRowsPerWave is a multiple of 16: lds_swz<8>(row) == 4 (j % 2) + lr / 2
      const uint32_t row = kRowsPerWave * wave + 8 * j + lr;
      const uint32_t off = in_range_or_oob(row * ldxb + (uint32_t)kt * 128 + ((lp ^ (4 * (j & 1) + (lr >> 1))) << 4),
                                           (uint32_t)kt, ngrp);
      buf_ld16_lds(rx, la + (kRowsPerWave * wave + 8 * j) * kBf16RowBytes, off);
    }
  }
  template <int SET>
  __device__ __forceinline__ void issue_regs(int kt) {
    const uint32_t cw = tid & 1;
#pragma unroll
    for (int j = 0; j < kRowGroups; ++j) {
      const uint32_t row = (tid >> 1) + kRowsPerGroup * j;
      cb[SET][j] = buf_ld16(rc, in_range_or_oob(row * kb + (uint32_t)kt * 32 + cw * 16, (uint32_t)kt, ngrp));
      const uint32_t go = in_range_or_oob((row * ngrp + (uint32_t)kt) * 2, (uint32_t)kt, ngrp);
      sb[SET][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)go, 0, 0);
      zb[SET][j] = __builtin_amdgcn_raw_buffer_load_b16(rz, (int)go, 0, 0);
    }
  }
  // half P: the weight chunk of row tid/2 + 128 P
  template <int P, int SET>
  __device__ __forceinline__ void store(uint8_t*, uint8_t* lb) {
    if (P >= kRowGroups) return;
    const int cw = tid & 1, r = tid >> 1;
    const int off = r * kBf16RowBytes + P * kRowsPerGroup * kBf16RowBytes;
    const float sc = __uint_as_float(sb[SET][P] << 16);
    const float zs = __uint_as_float(zb[SET][P] << 16) * sc;
    u32x4 o[4];
    int4_dequant_chunk(cb[SET][P], sc, zs, o);
#pragma unroll
    for (int d = 0; d < 4; ++d) st16(lb + off + (((4 * cw + d) ^ lds_swz<8>(r)) << 4), o[d]);
  }
};

// One output tile of 256 activation rows at (m0, n0) for 4 waves: G = 2, the waves
// stacked along M, each 64 x 32 F (32 F weight rows; the narrow tiles below).  G = 4
// (2 x 2 waves of 128 x 32 F) is the 4-wave form of the whole tiles, which run with 8
// waves instead.
template <bool OUT_F32, int F, int G>
__device__ __forceinline__ void w4a16_tile(
    uint8_t* lds, const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int64_t m0, int64_t n0) {
  static_assert(G == 4 || G == 2, "two wave layouts");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = G == 4 ? wave >> 1 : 0, wx = G == 4 ? wave & 1 : wave;
  // the narrow tile's accumulators leave room for a second register set
  W4A16Loader<(G == 4 ? 64 : 32) * F, G == 4 ? 1 : 2> ld;
  ld.init(x, ldx, wc, ws, wz, M, N, K, m0, n0, tid);
  v16f acc[F][G];
  bf16_mainloop(acc, ld, K, lds, wx, wy, lane);
  const int64_t n_base = n0 + wy * 32 * F, m_base = m0 + wx * 32 * G;
  __syncthreads();                           // all waves are done reading operand tiles
  epilogue_store<OUT_F32, F, 128, false, G>(acc, n_base, m_base, M, N, bias, y, ldy, lane,
                                            lds + wave * EpilogueShape<OUT_F32, F, 128>::kStageWaveBytes);
}

// Whole 256 x 256 tiles and halves (256 x 128) of the leftover ones (see tile_unit),
// with 8 waves, two per SIMD: wave w owns m in [128 (w % 2), +128) and n in
// [32 F (w / 2), +32 F).  Its 128 accumulators per lane (F = 2) leave room for the
// SIMD's second wave, so one wave's weight conversion and loads issue while the
// other's MFMAs run (327-329 against 348-350 us at M = 4608 for 4 waves of 128 x 128,
// same box); each thread converts one 32-code chunk per K-tile.
constexpr int kW4Threads8 = 512;
constexpr int kW4Lds8 = 8 * EpilogueShape<true, 2, 128>::kStageWaveBytes > kBf16MainLds
                            ? 8 * EpilogueShape<true, 2, 128>::kStageWaveBytes
                            : kBf16MainLds;                             // 144 KB
template <bool OUT_F32, int F>
__device__ __forceinline__ void w4a16_tile8(
    uint8_t* lds, const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int64_t m0, int64_t n0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  W4A16Loader<128 * F, 1, kW4Threads8> ld;
  ld.init(x, ldx, wc, ws, wz, M, N, K, m0, n0, tid);
  v16f acc[F][4];
  bf16_mainloop(acc, ld, K, lds, wx, wy, lane);
  const int64_t n_base = n0 + wy * 32 * F, m_base = m0 + wx * 128;
  __syncthreads();                           // all waves are done reading operand tiles
  epilogue_store<OUT_F32, F, 128, false, 4>(acc, n_base, m_base, M, N, bias, y, ldy, lane,
                                            lds + wave * EpilogueShape<OUT_F32, F, 128>::kStageWaveBytes);
}

template <bool OUT_F32>
__global__ __launch_bounds__(kW4Threads8, 1) void gemm_w4a16_kernel8(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int full) {
  static_assert(8 * EpilogueShape<true, 2, 128>::kStageWaveBytes <= kW4Lds8 &&
                    8 * EpilogueShape<false, 2, 128>::kStageWaveBytes <= kW4Lds8,
                "the epilogue stages each wave's output in the operand LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kW4Lds8];
  int vt, half, tm, tn;
  const bool is_half = tile_unit(blockIdx.x, tiles_m * tiles_n, full, &vt, &half);
  tile_of(vt, tiles_m, tiles_n, kBf16GroupM, &tm, &tn);
  if (!is_half) {
    w4a16_tile8<OUT_F32, 2>(lds, x, ldx, wc, ws, wz, M, N, K, bias, y, ldy, (int64_t)tm * kBf16BM,
                            (int64_t)tn * kBf16BN);
  } else {
    if ((int64_t)tn * 256 + 128 * half >= N) return;       // half past the last weight row
    w4a16_tile8<OUT_F32, 1>(lds, x, ldx, wc, ws, wz, M, N, K, bias, y, ldy, (int64_t)tm * kBf16BM,
                            (int64_t)tn * kBf16BN + 128 * half);
  }
}

// Few activation rows (M = 512 at N = 12288): tiles of 256 x 96, whose count fits
// one round over the CUs, where 256 x 256 tiles and their halves would leave CUs idle
// (96 tiles -> 192 halves of 256 x 128 on 256 CUs; 256 tiles of 256 x 96 do 0.75 of
// a half's work each).
constexpr int kW4NarrowN = 96;
template <bool OUT_F32>
__global__ __launch_bounds__(kBf16Threads, 1) void gemm_w4a16_narrow_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wc,
    const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wz, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBf16MainLds];
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, kBf16GroupM, &tm, &tn);
  w4a16_tile<OUT_F32, kW4NarrowN / 32, 2>(lds, x, ldx, wc, ws, wz, M, N, K, bias, y, ldy,
                                          (int64_t)tm * kBf16BM, (int64_t)tn * kW4NarrowN);
}

hipError_t launch_gemm_w4a16(const uint16_t* x, int64_t ldx, const uint8_t* wc,
                             const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                             int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kBf16BM - 1) / kBf16BM), tiles_n = (int)((N + kBf16BN - 1) / kBf16BN);
  const int64_t narrow_n = (N + kW4NarrowN - 1) / kW4NarrowN;
  if ((int64_t)tiles_m * narrow_n <= bf16_cus()) {
    const int tn = (int)narrow_n, grid = tiles_m * tn;
    if (ep.out_f32)
      hipLaunchKernelGGL(gemm_w4a16_narrow_kernel<true>, dim3(grid), dim3(kBf16Threads), 0, s, x, ldx, wc,
                         ws, wz, M, N, K, ep.bias, ep.y, ep.ldy, tiles_m, tn);
    else
      hipLaunchKernelGGL(gemm_w4a16_narrow_kernel<false>, dim3(grid), dim3(kBf16Threads), 0, s, x, ldx, wc,
                         ws, wz, M, N, K, ep.bias, ep.y, ep.ldy, tiles_m, tn);
    return hipGetLastError();
  }
  int full, grid;
  bf16_tile_split(tiles_m * tiles_n, &full, &grid);
  if (ep.out_f32)
    hipLaunchKernelGGL(gemm_w4a16_kernel8<true>, dim3(grid), dim3(kW4Threads8), 0, s, x, ldx, wc, ws,
                       wz, M, N, K, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
  else
    hipLaunchKernelGGL(gemm_w4a16_kernel8<false>, dim3(grid), dim3(kW4Threads8), 0, s, x, ldx, wc, ws,
                       wz, M, N, K, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
  return hipGetLastError();
}

}  // namespace q4
