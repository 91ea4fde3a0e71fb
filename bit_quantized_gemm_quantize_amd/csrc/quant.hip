// Activation quantizer (MXFP4 / NVFP4) fused with the low-rank down-projection,
// and the offline weight packers.
//
// Activation pass (one read of X).  Without the low-rank term, MXFP4 and NVFP4 take
// one thread per 32-element block instead (mx_rows_kernel, shared with MXFP8).  With
// it:
//   * a workgroup owns up to 32 rows (as many as spread M evenly over the CUs) and
//     all of K; its 16 waves stride over K in pairs of 32-element blocks, so a lane
//     (row l%32, half l/32) owns one whole block per step: 64 contiguous bytes of X
//     in, 16 bytes of codes and its scale out.  The block maximum therefore needs
//     no cross-lane exchange.
//   * the same 64 bytes are the bf16 MFMA operand of t = X L1: the 32 block
//     elements feed four 32x32x16 steps (K order permuted identically for X and L1,
//     which a sum over K allows); L1^T rows are read 16 bytes at a time.
//   * per-wave partial t tiles are summed through LDS in a fixed order, so t is
//     deterministic.
#include <algorithm>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

constexpr int kQWaves = 16;
constexpr int kQRows = 32;
constexpr float kNvTensorDiv = 2688.0f;   // 6 (largest E2M1) * 448 (largest E4M3)

// ---------------------------------------------------------------------------- NVFP4 helpers
// E4M3FN code of a non-negative fp32 value, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  v = fminf(v, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}
__device__ __forceinline__ float nv_tensor_scale(float amax_t) {
  return amax_t > 0.0f ? amax_t / kNvTensorDiv : 1.0f;
}

// x / den in fp32 (IEEE division, round to nearest even) for the two bf16 values of
// a dword, then E2M1 codes into byte SEL of r.  den = s_b * s_t, or 0 when the
// block scale is 0: every code is then a signed zero.
template <int SEL>
__device__ __forceinline__ uint32_t nv_encode_pair(uint32_t r, uint32_t pair, float den) {
  const float x0 = bf16_lo(pair), x1 = bf16_hi(pair);
  const float v0 = den > 0.0f ? x0 / den : __builtin_copysignf(0.0f, x0);
  const float v1 = den > 0.0f ? x1 / den : __builtin_copysignf(0.0f, x1);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v0, v1, 1.0f, SEL);
}

// Encode 16 bf16 values (8 dwords) of one NVFP4 block.
__device__ __forceinline__ void nv_encode16(const uint32_t* w, float den, uint32_t* out2) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    uint32_t r = 0;
    r = nv_encode_pair<0>(r, w[4 * d + 0], den);
    r = nv_encode_pair<1>(r, w[4 * d + 1], den);
    r = nv_encode_pair<2>(r, w[4 * d + 2], den);
    r = nv_encode_pair<3>(r, w[4 * d + 3], den);
    out2[d] = r;
  }
}

// One NVFP4 pair of blocks (32 values): two scale bytes and 16 bytes of codes.
__device__ __forceinline__ uint32_t nv_encode32(const uint32_t* w, float s_t, float d6, u32x4* codes) {
  uint32_t sc = 0;
  uint32_t c[4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float amax = __uint_as_float(bf16_amax_bits<8>(w + 8 * b) << 16);
    uint32_t code = e4m3_code(amax / d6);
    float den = e4m3_value(code) * s_t;
    nv_encode16(w + 8 * b, den, c + 2 * b);
    sc |= code << (8 * b);
  }
  *codes = u32x4{c[0], c[1], c[2], c[3]};
  return sc;
}

// ---------------------------------------------------------------------------- smoothed MXFP4
// floor(log2 v) of a positive fp32 magnitude given as its 31-bit pattern.
// Normal: exponent field - 127; subnormal m * 2**-149: floor(log2 m) - 149.
__device__ __forceinline__ int f32_floor_log2(uint32_t mag) {
  const uint32_t e = mag >> 23;
  if (e != 0) return (int)e - 127;
  return (31 - __builtin_clz(mag & 0x7FFFFFu)) - 149;
}

// One MXFP4 block of the smoothed activation v_j = fp32(x_j * inv_j) (fp32 multiply,
// round to nearest even): shared exponent E = floor(log2 max|v|) - 2, clamped to
// [-127, 127] (-127 for a zero block), and the codes of v * 2**-E, each product exact
// (a power of two; a result too small for fp32 encodes to a signed zero either way),
// rounded to E2M1 by the converter with a unit scale.  w: the block's 16 dwords of
// bf16 pairs; inv: its 32 factors.  Returns E.
__device__ __forceinline__ int mx_encode_smoothed(const uint32_t* w, const float* __restrict__ inv,
                                                  u32x4* codes) {
  float v[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const u32x4 f = ld16(inv + 4 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * q + j;
      const uint32_t pair = w[e >> 1];
      const float x = (e & 1) ? bf16_hi(pair) : bf16_lo(pair);
      v[e] = x * __uint_as_float(f[j]);
    }
  }
  uint32_t amax = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = max(amax, __float_as_uint(v[e]) & 0x7FFFFFFFu);
  int E = amax == 0 ? -127 : f32_floor_log2(amax) - 2;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  const float down = exp2i(-E);
  uint32_t c[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 0] * down, v[8 * d + 1] * down, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 2] * down, v[8 * d + 3] * down, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 4] * down, v[8 * d + 5] * down, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 6] * down, v[8 * d + 7] * down, 1.0f, 3);
    c[d] = r;
  }
  *codes = u32x4{c[0], c[1], c[2], c[3]};
  return E;
}

// ---------------------------------------------------------------------------- per block
// One thread per (row, 32-element block) of a strided bf16 matrix, consecutive
// threads on consecutive blocks of a row (contiguous loads and stores).
//   MXFP8: E = floor(log2 amax) - 8 (emax of E4M3FN) clamped to [-127, 127], codes
//   E4M3_RNE(x * 2**-E) saturated at +-448 (the product is exact in fp32; the clamp
//   comes before the converter, which rounds to nearest even), 32 code bytes, one
//   scale byte E + 127.
//   MXFP4 and NVFP4 (the activation pass without the low-rank term): the encodes of
//   the row-per-lane pass (one MX block and its scale byte, or two NVFP4 blocks of 16
//   and their two E4M3 scale bytes), 16 code bytes.
constexpr int kBlkMXFP4 = 0, kBlkNVFP4 = 1, kBlkMXFP8 = 2;
template <int KIND>
__device__ __forceinline__ void mx_block(const uint16_t* __restrict__ x, int64_t K, int64_t sr, int64_t sk,
                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                         int64_t nblk, int64_t q, float s_t, float d6) {
  const int64_t r = q / nblk, b = q % nblk;
  const uint16_t* src = x + r * sr + b * 32 * sk;
  uint32_t w[16];
  if (sk == 1 && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = ld16(src + 8 * c);
      w[4 * c] = v[0]; w[4 * c + 1] = v[1]; w[4 * c + 2] = v[2]; w[4 * c + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = (uint32_t)src[2 * j * sk] | ((uint32_t)src[(2 * j + 1) * sk] << 16);
  }
  if (KIND == kBlkNVFP4) {
    u32x4 c;
    const uint32_t sc = nv_encode32(w, s_t, d6, &c);
    st16(codes + r * (K >> 1) + b * 16, c);
    *reinterpret_cast<uint16_t*>(scales + r * (2 * nblk) + 2 * b) = (uint16_t)sc;
    return;
  }
  const uint32_t amax = bf16_amax_bits<16>(w);
  if (KIND == kBlkMXFP4) {
    const int E = mx_block_exponent(amax);
    const float sc = exp2i(E);
    st16(codes + r * (K >> 1) + b * 16, u32x4{fp4_encode8_pow2(w, sc), fp4_encode8_pow2(w + 4, sc),
                                               fp4_encode8_pow2(w + 8, sc), fp4_encode8_pow2(w + 12, sc)});
    scales[r * nblk + b] = (uint8_t)(E + 127);
    return;
  }
  int E = amax == 0 ? -127 : bf16_floor_log2(amax) - 8;
  E = E < -127 ? -127 : (E > 127 ? 127 : E);
  const float down = exp2i(-E);
  uint32_t out[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * d + j;
      const float xv = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
      v[j] = fminf(fmaxf(xv * down, -448.0f), 448.0f);
    }
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
    out[d] = (uint32_t)word;
  }
  uint8_t* dst = codes + r * K + b * 32;
  st16(dst, u32x4{out[0], out[1], out[2], out[3]});
  st16(dst + 16, u32x4{out[4], out[5], out[6], out[7]});
  scales[r * nblk + b] = (uint8_t)(E + 127);
}

// amax_t: NVFP4's tensor amax (the tensor scale is derived from it), else unused.
template <int KIND>
__global__ __launch_bounds__(256) void mx_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t K, int64_t sr, int64_t sk,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales,
                                                      const float* __restrict__ amax_t) {
  float s_t = 1.0f, d6 = 6.0f;
  if (KIND == kBlkNVFP4) {
    s_t = nv_tensor_scale(*amax_t);
    d6 = 6.0f * s_t;
  }
  const int64_t nblk = K >> 5, work = rows * nblk;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < work; q += (int64_t)gridDim.x * blockDim.x)
    mx_block<KIND>(x, K, sr, sk, codes, scales, nblk, q, s_t, d6);
}

// Launch of mx_rows_kernel: one thread per block, the grid capped (the threads
// then stride over the blocks).
template <int KIND>
static hipError_t queue_mx_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                                uint8_t* codes, uint8_t* scales, hipStream_t s,
                                const float* amax_t = nullptr) {
  const int64_t work = rows * (K >> 5);
  if (work == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, int64_t(1) << 20);
  hipLaunchKernelGGL(mx_rows_kernel<KIND>, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, K, sr, sk, codes,
                     scales, amax_t);
  return hipGetLastError();
}

hipError_t launch_mxfp8_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  return queue_mx_rows<kBlkMXFP8>(x, rows, K, sr, sk, codes, scales, s);
}

// ---------------------------------------------------------------------------- activation pass
// One pair of 32-element blocks per lane half: the 64 bytes of X of block `blk` of
// `row` (zeros past M or K).
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t row, int64_t ldx,
                                           int64_t blk, bool ok, uint32_t* w) {
  if (ok) {
    const uint16_t* src = x + row * ldx + blk * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = ld16(src + 8 * q);
      w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) w[q] = 0;
  }
}

// A workgroup owns `rows` (<= 32) consecutive rows and all of K; rows is chosen
// so the workgroups spread evenly over the CUs (lanes past it idle).  Each of the 16
// waves takes every 16th pair of blocks, keeping the X bytes of three pairs in
// flight per lane.
template <int FMT, int R, bool SMOOTH = false>
__global__ __launch_bounds__(kQWaves * 64) void quant_act_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int rows,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ amax_t,
    const uint16_t* __restrict__ l1t, float* __restrict__ t, const float* __restrict__ inv_s) {
  __shared__ float red[R > 0 ? kQWaves * 32 * 32 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * rows;
  const int64_t row = m0 + i;
  const bool row_ok = i < rows && row < M;
  const int64_t nblk = K >> 5;
  const int64_t npair = (nblk + 1) >> 1;
  const int64_t sbytes = FMT == 0 ? nblk : 2 * nblk;   // scale bytes per row

  float s_t = 1.0f, d6 = 6.0f;
  if (FMT == 1) {
    s_t = nv_tensor_scale(*amax_t);
    d6 = 6.0f * s_t;
  }
  v16f acc = {};

  auto load = [&](int64_t p, uint32_t* w) {
    load_block(x, row, ldx, 2 * p + h, row_ok && p < npair && 2 * p + h < nblk, w);
  };
  auto step = [&](int64_t p, uint32_t* w) {
    if (p >= npair) return;
    const int64_t blk = 2 * p + h;
    const bool blk_ok = blk < nblk;
    if (row_ok && blk_ok) {
      u32x4 c;
      if (FMT == 0 && SMOOTH) {
        const int E = mx_encode_smoothed(w, inv_s + blk * 32, &c);
        scales[row * sbytes + blk] = (uint8_t)(E + 127);
      } else if (FMT == 0) {
        const int E = mx_block_exponent(bf16_amax_bits<16>(w));
        const float sc = exp2i(E);
        c = u32x4{fp4_encode8_pow2(w, sc), fp4_encode8_pow2(w + 4, sc),
                  fp4_encode8_pow2(w + 8, sc), fp4_encode8_pow2(w + 12, sc)};
        scales[row * sbytes + blk] = (uint8_t)(E + 127);
      } else {
        const uint32_t sc = nv_encode32(w, s_t, d6, &c);
        *reinterpret_cast<uint16_t*>(scales + row * sbytes + 2 * blk) = (uint16_t)sc;
      }
      st16(codes + row * (K >> 1) + blk * 16, c);
    }
    if (R > 0) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a = u32x4{w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]};
        u32x4 b = u32x4{0, 0, 0, 0};
        if (i < R && blk_ok) b = ld16(l1t + (int64_t)i * K + blk * 32 + 8 * s);
        acc = mfma_bf16_32x32x16(a, b, acc);
      }
    }
    load(p + 3 * kQWaves, w);                 // refill this buffer three steps ahead
  };
  uint32_t w0[16], w1[16], w2[16];
  const int64_t p0 = wave;
  load(p0, w0);
  load(p0 + kQWaves, w1);
  load(p0 + 2 * kQWaves, w2);
  for (int64_t p = p0; p < npair; p += 3 * kQWaves) {
    step(p, w0);
    step(p + kQWaves, w1);
    step(p + 2 * kQWaves, w2);
  }

  if (R > 0) {
    // acc: rows = x rows (8*(v/4) + 4*h + v%4), column = t column (lane % 32)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave * 1024 + acc_row(v, lane) * 32 + i] = acc[v];
    __syncthreads();
    constexpr int kR = R > 0 ? R : 1;
    for (int idx = threadIdx.x; idx < 32 * R; idx += kQWaves * 64) {
      const int rr = idx / kR, cc = idx % kR;
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kQWaves; ++wv) sum += red[wv * 1024 + rr * 32 + cc];
      if (rr < rows && m0 + rr < M) t[(m0 + rr) * R + cc] = sum;
    }
  }
}

// ---------------------------------------------------------------------------- tensor amax
__global__ void clear_f32_kernel(float* p) { *p = 0.0f; }

__global__ void nv_finalize_kernel(float* p) { *p = nv_tensor_scale(*p); }

// Largest |x| over a strided [rows, cols] bf16 matrix (element (r, c) at
// x[r * sr + c * sc]), reduced per workgroup (wave shuffles, then LDS) and then
// folded into *amax with one integer atomic max on the fp32 bit pattern per
// workgroup (valid for non-negative values).
constexpr int kAmaxBlocks = 1024;
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t sr, int64_t sc,
                                                   float* amax) {
  __shared__ uint32_t part[4];
  uint32_t m = 0;
  const int64_t total = rows * cols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (sc == 1 && (cols & 31) == 0 && (sr & 7) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    // 64 bytes per thread per step, two steps (eight 16-byte loads) in flight
    const int64_t per_row = cols >> 5, nq = rows * per_row;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += 2 * stride) {
      u32x4 v[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t qu = q + u * stride;
        const int64_t r = qu / per_row, c = qu % per_row;
        const uint16_t* src = x + r * sr + c * 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[u][j] = qu < nq ? ld16(src + 8 * j) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, bf16_amax_bits<4>(reinterpret_cast<const uint32_t*>(&v[u][j])));
    }
  } else {
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += stride) {
      const int64_t r = q / cols, c = q % cols;
      m = max(m, (uint32_t)(x[r * sr + c * sc] & 0x7FFFu));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(part[0], part[1]), max(part[2], part[3]));
    if (m != 0) atomicMax(reinterpret_cast<unsigned int*>(amax), m << 16);
  }
}

static hipError_t queue_tensor_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t sr,
                                    int64_t sc, float* amax, hipStream_t s) {
  hipLaunchKernelGGL(clear_f32_kernel, dim3(1), dim3(1), 0, s, amax);
  const int64_t work = (rows * cols + 31) / 32;
  int64_t blocks = (work + 255) / 256;
  if (blocks > kAmaxBlocks) blocks = kAmaxBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols, sr, sc, amax);
  return hipGetLastError();
}

template <int FMT, int R, bool SMOOTH = false>
static void queue_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                        uint8_t* scales, const float* amax, const uint16_t* l1t, float* t,
                        hipStream_t s, const float* inv_s = nullptr) {
  // rows per workgroup: the fewest rounds of workgroups over the CUs with at most 32
  // rows each (M = 4608 on 256 CUs: 18 rows, one workgroup per CU)
  int cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
  }
  int64_t waves = 1;
  while ((M + cus * waves - 1) / (cus * waves) > kQRows) ++waves;
  const int rows = (int)std::max<int64_t>(1, (M + cus * waves - 1) / (cus * waves));
  const unsigned grid = (unsigned)((M + rows - 1) / rows);
  hipLaunchKernelGGL((quant_act_kernel<FMT, R, SMOOTH>), dim3(grid), dim3(kQWaves * 64), 0, s, x, M, K, ldx,
                     rows, codes, scales, amax, l1t, t, inv_s);
}

hipError_t launch_quantize_act(int fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               const uint16_t* l1t, int r, float* t, hipStream_t s,
                               const float* inv_s) {
  if (fmt == 0 && inv_s != nullptr) {
    if (r == 0) queue_quant<0, 0, true>(x, M, K, ldx, codes, scales, nullptr, l1t, t, s, inv_s);
    else if (r == 16) queue_quant<0, 16, true>(x, M, K, ldx, codes, scales, nullptr, l1t, t, s, inv_s);
    else queue_quant<0, 32, true>(x, M, K, ldx, codes, scales, nullptr, l1t, t, s, inv_s);
    return hipGetLastError();
  }
  if (fmt == 1) {
    hipError_t e = queue_tensor_amax(x, M, K, ldx, 1, tensor_scale, s);
    if (e != hipSuccess) return e;
  }
  if (fmt == 0) {
    // without the low-rank term, one thread per block: the row-per-lane layout only
    // serves the MFMA of t = X L1
    if (r == 0) {
      const hipError_t e = queue_mx_rows<kBlkMXFP4>(x, M, K, ldx, 1, codes, scales, s);
      if (e != hipSuccess) return e;
    }
    else if (r == 16) queue_quant<0, 16>(x, M, K, ldx, codes, scales, nullptr, l1t, t, s);
    else queue_quant<0, 32>(x, M, K, ldx, codes, scales, nullptr, l1t, t, s);
  } else {
    if (r == 0) {
      const hipError_t e = queue_mx_rows<kBlkNVFP4>(x, M, K, ldx, 1, codes, scales, s, tensor_scale);
      if (e != hipSuccess) return e;
    } else if (r == 16) queue_quant<1, 16>(x, M, K, ldx, codes, scales, tensor_scale, l1t, t, s);
    else queue_quant<1, 32>(x, M, K, ldx, codes, scales, tensor_scale, l1t, t, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(nv_finalize_kernel, dim3(1), dim3(1), 0, s, tensor_scale);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- int4 symmetric
// Signed int4, symmetric, one fp32 scale per row: scale = max(amax / 7, 1e-8) and
// q = clamp(rint(x / scale), -8, 7), every step in fp32 (IEEE division, round half
// to even).  One wave per row of a strided bf16 matrix (element (r, k) at
// x[r * sr + k * sk]); a contiguous row of up to 4096 elements is read once into
// registers, others in two passes (the second from the cache).  Codes
// are two's-complement nibbles, the even k in the low nibble.
__global__ __launch_bounds__(256) void int4_sym_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t K, int64_t sr, int64_t sk,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                     // the whole wave
  const uint16_t* row = x + r * sr;
  const bool contig = sk == 1 && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const int64_t chunks = K >> 3;             // 8 elements (16 bytes of bf16) each
  auto load8 = [&](int64_t c, uint32_t* w) {
    if (contig) {
      const u32x4 v = ld16(row + 8 * c);
      w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)row[(8 * c + 2 * j) * sk] | ((uint32_t)row[(8 * c + 2 * j + 1) * sk] << 16);
    }
  };
  auto wave_scale = [&](uint32_t m) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    const float scale = fmaxf(__uint_as_float(m << 16) / 7.0f, 1e-8f);
    if (lane == 0) scales[r] = scale;
    return scale;
  };
  uint8_t* out = codes + r * (K >> 1);
  auto encode8 = [&](int64_t c, const uint32_t* w, float scale) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
      const float q = fminf(fmaxf(__builtin_rintf(v / scale), -8.0f), 7.0f);
      packed |= ((uint32_t)(int)q & 0xFu) << (4 * j);
    }
    *reinterpret_cast<uint32_t*>(out + 4 * c) = packed;
  };
  constexpr int kRegChunks = 8;              // rows up to 64 * 8 chunks stay in registers
  if (contig && chunks <= 64 * kRegChunks) {
    // one read of the row: every chunk's load in flight at once
    uint32_t w[kRegChunks][4];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i) {
      const int64_t c = lane + 64 * i;
      if (c < chunks) load8(c, w[i]);
      else w[i][0] = w[i][1] = w[i][2] = w[i][3] = 0;
    }
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i) m = max(m, bf16_amax_bits<4>(w[i]));
    const float scale = wave_scale(m);
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i)
      if (lane + 64 * i < chunks) encode8(lane + 64 * i, w[i], scale);
    return;
  }
  uint32_t m = 0;
  for (int64_t c = lane; c < chunks; c += 64) {
    uint32_t w[4];
    load8(c, w);
    m = max(m, bf16_amax_bits<4>(w));
  }
  const float scale = wave_scale(m);
  for (int64_t c = lane; c < chunks; c += 64) {
    uint32_t w[4];
    load8(c, w);
    encode8(c, w, scale);
  }
}

hipError_t launch_int4_sym_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                                uint8_t* codes, float* scales, hipStream_t s) {
  hipLaunchKernelGGL(int4_sym_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, x, rows,
                     K, sr, sk, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- weight packers
// One thread per (output column n, K group); consecutive threads take consecutive
// n, so a [K, N] row-major weight is read coalesced and a [N, K] one row-wise.
__device__ __forceinline__ void load_strided(const uint16_t* w, int64_t k0, int64_t n, int64_t sk,
                                             int64_t sn, int count, uint32_t* out) {
  for (int j = 0; j < count; j += 2) {
    uint32_t lo = w[(k0 + j) * sk + n * sn];
    uint32_t hi = w[(k0 + j + 1) * sk + n * sn];
    out[j >> 1] = lo | (hi << 16);
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                       int64_t N, int64_t sk, int64_t sn,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       const float* __restrict__ amax_t) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nblk = K >> 5;
  if (q >= N * nblk) return;
  const int64_t n = q % N, blk = q / N;
  uint32_t v[16];
  load_strided(w, blk * 32, n, sk, sn, 32, v);
  u32x4 c;
  if (FMT == 0) {
    const int E = mx_block_exponent(bf16_amax_bits<16>(v));
    const float sc = exp2i(E);
    c = u32x4{fp4_encode8_pow2(v, sc), fp4_encode8_pow2(v + 4, sc), fp4_encode8_pow2(v + 8, sc),
              fp4_encode8_pow2(v + 12, sc)};
    scales[n * nblk + blk] = (uint8_t)(E + 127);
  } else {
    const float s_t = nv_tensor_scale(*amax_t);
    const uint32_t sc = nv_encode32(v, s_t, 6.0f * s_t, &c);
    scales[n * 2 * nblk + 2 * blk] = (uint8_t)(sc & 0xFF);
    scales[n * 2 * nblk + 2 * blk + 1] = (uint8_t)(sc >> 8);
  }
  st16(codes + n * (K >> 1) + blk * 16, c);
}

// Asymmetric int4, group 64: s = bf16(fp32(hi - lo) / 15) (1 if 0),
// z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15).  v holds the
// 64 bf16 values of group g of column n (element 2j in the low half of v[j]).
__device__ __forceinline__ void int4_encode_group(const uint32_t* v, int64_t n, int64_t g, int64_t K,
                                                  uint8_t* __restrict__ codes,
                                                  uint16_t* __restrict__ scales,
                                                  uint16_t* __restrict__ zeros) {
  const int64_t ngrp = K >> 6;
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float a = bf16_lo(v[j]), b = bf16_hi(v[j]);
    lo = fminf(lo, fminf(a, b));
    hi = fmaxf(hi, fmaxf(a, b));
  }
  const uint32_t sbits = f32_to_bf16_rne((hi - lo) / 15.0f);
  float s = __uint_as_float(sbits << 16);
  uint32_t sstore = sbits;
  if (s == 0.0f) { s = 1.0f; sstore = 0x3F80u; }
  const float z = fminf(fmaxf(rintf(-lo / s), 0.0f), 15.0f);
  uint32_t out[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pair = v[4 * d + j];
      const float q0 = fminf(fmaxf(rintf(bf16_lo(pair) / s) + z, 0.0f), 15.0f);
      const float q1 = fminf(fmaxf(rintf(bf16_hi(pair) / s) + z, 0.0f), 15.0f);
      r |= ((uint32_t)q0 | ((uint32_t)q1 << 4)) << (8 * j);
    }
    out[d] = r;
  }
  uint8_t* dst = codes + n * (K >> 1) + g * 32;
  st16(dst, u32x4{out[0], out[1], out[2], out[3]});
  st16(dst + 16, u32x4{out[4], out[5], out[6], out[7]});
  scales[n * ngrp + g] = (uint16_t)sstore;
  zeros[n * ngrp + g] = (uint16_t)f32_to_bf16_rne(z + 0.0f);   // never -0
}

// Any strides: one thread per (column n, group); consecutive threads take
// consecutive n, so a [K, N] row-major weight is read coalesced.
__global__ __launch_bounds__(256) void pack_int4_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                        int64_t N, int64_t sk, int64_t sn,
                                                        uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ zeros) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ngrp = K >> 6;
  if (q >= N * ngrp) return;
  const int64_t n = q % N, g = q / N;
  uint32_t v[32];
  load_strided(w, g * 64, n, sk, sn, 64, v);
  int4_encode_group(v, n, g, K, codes, scales, zeros);
}

// K-contiguous weight ([N, K], nn.Linear layout): one thread per (n, group),
// consecutive threads along K, 128 contiguous bytes per thread in 16-byte loads.
__global__ __launch_bounds__(256) void pack_int4_rows_kernel(const uint16_t* __restrict__ w,
                                                             int64_t K, int64_t N, int64_t sn,
                                                             uint8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ scales,
                                                             uint16_t* __restrict__ zeros) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ngrp = K >> 6;
  if (q >= N * ngrp) return;
  const int64_t n = q / ngrp, g = q % ngrp;
  const uint16_t* src = w + n * sn + g * 64;
  uint32_t v[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4 x = ld16(src + 8 * j);
    v[4 * j] = x[0]; v[4 * j + 1] = x[1]; v[4 * j + 2] = x[2]; v[4 * j + 3] = x[3];
  }
  int4_encode_group(v, n, g, K, codes, scales, zeros);
}

hipError_t launch_pack_weights(int fmt, const uint16_t* w, int64_t K, int64_t N, int64_t sk,
                               int64_t sn, uint8_t* codes, void* scales, uint16_t* zeros,
                               float* tensor_scale, hipStream_t s) {
  // K-contiguous rows with 16-byte alignment: the rows of W^T are quantized exactly
  // like activation rows (same blocks along K, same encoders), with vector loads
  const bool rows = sk == 1 && sn % 8 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
  if (rows && fmt != 2)
    return launch_quantize_act(fmt, w, N, K, sn, codes, static_cast<uint8_t*>(scales), tensor_scale,
                               nullptr, 0, nullptr, s);
  if (rows) {
    const int64_t work = N * (K >> 6);
    hipLaunchKernelGGL(pack_int4_rows_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, w,
                       K, N, sn, codes, static_cast<uint16_t*>(scales), zeros);
    return hipGetLastError();
  }
  if (fmt == 2) {
    const int64_t work = N * (K >> 6);
    hipLaunchKernelGGL(pack_int4_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, w, K,
                       N, sk, sn, codes, static_cast<uint16_t*>(scales), zeros);
    return hipGetLastError();
  }
  const int64_t work = N * (K >> 5);
  const unsigned grid = (unsigned)((work + 255) / 256);
  if (fmt == 0) {
    hipLaunchKernelGGL(pack_fp4_kernel<0>, dim3(grid), dim3(256), 0, s, w, K, N, sk, sn, codes,
                       static_cast<uint8_t*>(scales), nullptr);
    return hipGetLastError();
  }
  // logical [K, N]: rows k (stride sk), columns n (stride sn)
  hipError_t e = queue_tensor_amax(w, K, N, sk, sn, tensor_scale, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_fp4_kernel<1>, dim3(grid), dim3(256), 0, s, w, K, N, sk, sn, codes,
                     static_cast<uint8_t*>(scales), tensor_scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nv_finalize_kernel, dim3(1), dim3(1), 0, s, tensor_scale);
  return hipGetLastError();
}

}  // namespace q4
