// Activation quantizer (MXFP4 / NVFP4) fused with the low-rank down-projection,
// and the offline weight packers.
//
// Activation pass, one read of X per encode:
//   * MXFP4 without the low-rank term: one thread per 32-element block
//     (mx_rows_kernel, shared with MXFP8 and the weight packer).
//   * with the low-rank term t = X L1 (or SmoothQuant factors): quant_act_kernel,
//     a workgroup's rows of X (and of L1^T, and the factors) copied chunk by chunk
//     straight into a ring of LDS stages, each block encoded by one lane from LDS,
//     and t formed from the same LDS tiles on the bf16 MFMA.
//   * NVFP4: a tensor-amax launch that leaves per-workgroup partial maxima in a
//     small scratch array, then the encode launch (16-element blocks).
#include <algorithm>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

// partial maxima of the NVFP4 tensor-amax launch: the scratch it needs, 4 KB
constexpr int kNvPartials = kNvScratchWords;
constexpr int kQRows = 32;
constexpr float kNvTensorDiv = 2688.0f;   // 6 (largest E2M1) * 448 (largest E4M3)
constexpr int64_t kNvEncodeGroups = 2048;

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

// The correctly rounded quotient x / den from y = RN(1/den) (Markstein: with y the
// correctly rounded reciprocal and q = RN(x y) within an ulp of x / den, the
// residual r = x - den q is exact in one fma and RN(q + r y) is RN(x / den); den,
// y and the quotients that decide a code are normal fp32 numbers here).
__device__ __forceinline__ float nv_quotient(float x, float den, float y) {
  const float q = x * y;
  const float r = __builtin_fmaf(-den, q, x);
  return __builtin_fmaf(r, y, q);
}
template <int SEL>
__device__ __forceinline__ uint32_t nv_encode_pair_rcp(uint32_t r, uint32_t pair, float den, float y) {
  const float v0 = nv_quotient(bf16_lo(pair), den, y), v1 = nv_quotient(bf16_hi(pair), den, y);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v0, v1, 1.0f, SEL);
}

// Encode 16 bf16 values (8 dwords) of one NVFP4 block: x / den for each, rounded
// to E2M1.  With den in [2^-100, 2^100] the quotients go through the reciprocal
// (one IEEE division per block); otherwise, and for den = 0 (signed zero codes),
// through the IEEE division per element.
__device__ __forceinline__ void nv_encode16(const uint32_t* w, float den, uint32_t* out2) {
  if (den >= 0x1p-100f && den <= 0x1p100f) {
    const float y = 1.0f / den;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      uint32_t r = 0;
      r = nv_encode_pair_rcp<0>(r, w[4 * d + 0], den, y);
      r = nv_encode_pair_rcp<1>(r, w[4 * d + 1], den, y);
      r = nv_encode_pair_rcp<2>(r, w[4 * d + 2], den, y);
      r = nv_encode_pair_rcp<3>(r, w[4 * d + 3], den, y);
      out2[d] = r;
    }
    return;
  }
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

// Per-code reciprocals of an NVFP4 encode launch, filled by threads 0..127 of each
// workgroup: for a block scale of E4M3 code c the encoder divides by
// den_c = fp32(value(c) * s_t); where den_c lies in [2^-100, 2^100], rcp[c] holds
// RN(1/den_c) (one IEEE division per code and workgroup instead of one per block), and
// 0 marks the codes whose blocks divide element by element (den_c = 0 gives signed
// zero codes, as in nv_encode16).
__device__ __forceinline__ void nv_fill_rcp(float* rcp, float s_t) {
  if (threadIdx.x < 128) {
    const float den = e4m3_value(threadIdx.x) * s_t;
    rcp[threadIdx.x] = (den >= 0x1p-100f && den <= 0x1p100f) ? 1.0f / den : 0.0f;
  }
}

// nv_encode32 with the block scale's quotient amax / d6 through y6 = RN(1/d6) when
// y6 > 0 (d6 in [2^-80, 2^100]: every quotient that decides a nonzero code, at least
// 2^-10, is then a normal number and so is the correction's residual), and the
// elements' quotients through rcp.  Same codes as nv_encode32.
__device__ __forceinline__ uint32_t nv_encode32_rcp(const uint32_t* w, float s_t, float d6, float y6,
                                                    const float* rcp, u32x4* codes) {
  uint32_t sc = 0;
  uint32_t c[4];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float amax = __uint_as_float(bf16_amax_bits<8>(w + 8 * b) << 16);
    const uint32_t code = e4m3_code(y6 > 0.0f ? nv_quotient(amax, d6, y6) : amax / d6);
    const float den = e4m3_value(code) * s_t;
    const float y = rcp[code];
    const uint32_t* v = w + 8 * b;
    if (y != 0.0f) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint32_t r = 0;
        r = nv_encode_pair_rcp<0>(r, v[4 * d + 0], den, y);
        r = nv_encode_pair_rcp<1>(r, v[4 * d + 1], den, y);
        r = nv_encode_pair_rcp<2>(r, v[4 * d + 2], den, y);
        r = nv_encode_pair_rcp<3>(r, v[4 * d + 3], den, y);
        c[2 * b + d] = r;
      }
    } else {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        uint32_t r = 0;
        r = nv_encode_pair<0>(r, v[4 * d + 0], den);
        r = nv_encode_pair<1>(r, v[4 * d + 1], den);
        r = nv_encode_pair<2>(r, v[4 * d + 2], den);
        r = nv_encode_pair<3>(r, v[4 * d + 3], den);
        c[2 * b + d] = r;
      }
    }
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
// mx_block (q4_device.h): one thread per (row, 32-element block).
template <int KIND>
__global__ __launch_bounds__(256) void mx_rows_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t K, int64_t sr, int64_t sk,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t nblk = K >> 5, work = rows * nblk;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < work; q += (int64_t)gridDim.x * blockDim.x)
    mx_block<KIND>(x, K, sr, sk, codes, scales, nblk, q);
}

// Launch of mx_rows_kernel: one thread per block, the grid capped (the threads
// then stride over the blocks).
template <int KIND>
static hipError_t queue_mx_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                                uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t work = rows * (K >> 5);
  if (work == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, int64_t(1) << 20);
  hipLaunchKernelGGL(mx_rows_kernel<KIND>, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, K, sr, sk, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_mxfp8_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  return queue_mx_rows<kBlkMXFP8>(x, rows, K, sr, sk, codes, scales, s);
}

// ---------------------------------------------------------------------------- NVFP4 tensor amax
// NVFP4 needs the tensor's largest magnitude before any block can be encoded, so
// its pass is two launches: nv_amax_kernel reduces |x| per workgroup and stores
// the partial maxima (fp32 bit patterns, an order-preserving integer for
// non-negative values) in a scratch array of at most kNvPartials words; every
// workgroup of the encode launch reduces that array itself, in the same order,
// so each derives the same s_t, and workgroup 0 stores s_t.  No atomics, no
// clearing, no single-thread launch.

// Largest of the n partial maxima, reduced by the whole workgroup (256 threads).
__device__ __forceinline__ uint32_t reduce_partials(const uint32_t* __restrict__ partials, int n,
                                                    uint32_t* lds4) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += 256) m = max(m, partials[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(lds4[0], lds4[1]), max(lds4[2], lds4[3]));
  __syncthreads();
  return m;
}

// Partial max of |x| over a strided [rows, cols] bf16 matrix (element (r, c) at
// x[r * sr + c * sc]); workgroup b stores its maximum's bits in partials[b].
// Rows of 16-byte aligned, contiguous chunks are read 16 bytes at a time, four
// loads in flight per thread.
__global__ __launch_bounds__(256) void nv_amax_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t sr, int64_t sc,
                                                      uint32_t* __restrict__ partials) {
  __shared__ uint32_t part[4];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sc == 1 && (cols & 7) == 0 && (sr & 7) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    const int64_t per_row = cols >> 3, nq = rows * per_row;      // 16-byte chunks
    const bool flat = sr == cols;
    for (int64_t q = tid; q < nq; q += 4 * stride) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t qu = q + u * stride;
        const int64_t off = flat ? qu * 8 : (qu / per_row) * sr + (qu % per_row) * 8;
        v[u] = qu < nq ? ld16(x + off) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) m = max(m, bf16_amax_bits<4>(reinterpret_cast<const uint32_t*>(&v[u])));
    }
  } else {
    for (int64_t q = tid; q < rows * cols; q += stride) {
      const int64_t r = q / cols, c = q % cols;
      m = max(m, (uint32_t)(x[r * sr + c * sc] & 0x7FFFu));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = max(max(part[0], part[1]), max(part[2], part[3])) << 16;
}

// Grid of the amax launch: at most kNvPartials workgroups.
static int nv_amax_grid(int64_t elems) {
  const int64_t want = (elems / 8 + 1023) / 1024;              // about four chunks per thread
  return (int)std::max<int64_t>(1, std::min<int64_t>(kNvPartials, want));
}

static hipError_t queue_nv_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t sr, int64_t sc,
                                uint32_t* partials, int grid, hipStream_t s) {
  hipLaunchKernelGGL(nv_amax_kernel, dim3(grid), dim3(256), 0, s, x, rows, cols, sr, sc, partials);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- NVFP4 encode
// One 16-element block per thread and step (two steps in flight), consecutive
// threads on consecutive blocks of a row: 32 bytes of X in, 8 bytes of codes and
// one E4M3 scale byte out.  Any K that is a multiple of 16.  x is [rows, K] with
// row stride ldx (a multiple of 8, 16-byte aligned base).
__device__ __forceinline__ void nv_block16(const uint16_t* __restrict__ x, int64_t K, int64_t ldx,
                                           int64_t nb, int64_t q, float s_t, float d6,
                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                           const u32x4& lo, const u32x4& hi) {
  const int64_t r = q / nb, b = q % nb;
  const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  const float amax = __uint_as_float(bf16_amax_bits<8>(w) << 16);
  const uint32_t code = e4m3_code(amax / d6);
  uint32_t c[2];
  nv_encode16(w, e4m3_value(code) * s_t, c);
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2*>(codes + r * (K >> 1) + b * 8) = u32x2{c[0], c[1]};
  scales[r * nb + b] = (uint8_t)code;
}

__global__ __launch_bounds__(256) void nv_encode_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t K, int64_t ldx, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        const uint32_t* __restrict__ partials, int nparts,
                                                        float* __restrict__ tensor_scale) {
  __shared__ uint32_t lds4[4];
  __shared__ float rcp[128];
  const int64_t nb = K >> 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if ((nb & 1) == 0) {
    // a pair of blocks per thread and step: 64 bytes of X in, 16 code bytes and 2
    // scale bytes out; the next step's loads are issued before the current step is
    // encoded, and the first step's before the tensor scale is reduced
    const int64_t np = nb >> 1, work = rows * np;
    auto load = [&](int64_t q, uint32_t* w) {
      if (q < work) {
        const uint16_t* src = x + (q / np) * ldx + (q % np) * 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 v = ld16(src + 8 * c);
          w[4 * c] = v[0]; w[4 * c + 1] = v[1]; w[4 * c + 2] = v[2]; w[4 * c + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = 0;
      }
    };
    int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t w[16];
    load(q, w);
    const float s_t = nv_tensor_scale(__uint_as_float(reduce_partials(partials, nparts, lds4)));
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
    const float d6 = 6.0f * s_t;
    const float y6 = (d6 >= 0x1p-80f && d6 <= 0x1p100f) ? 1.0f / d6 : 0.0f;
    nv_fill_rcp(rcp, s_t);
    __syncthreads();
    for (; q < work; q += stride) {
      uint32_t wn[16];
      load(q + stride, wn);
      u32x4 c;
      const uint32_t sc = nv_encode32_rcp(w, s_t, d6, y6, rcp, &c);
      const int64_t r = q / np, p = q % np;
      st16(codes + r * (K >> 1) + p * 16, c);
      *reinterpret_cast<uint16_t*>(scales + r * nb + 2 * p) = (uint16_t)sc;
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = wn[j];
    }
    return;
  }
  const float s_t = nv_tensor_scale(__uint_as_float(reduce_partials(partials, nparts, lds4)));
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  const float d6 = 6.0f * s_t;
  const int64_t work = rows * nb;
  auto src = [&](int64_t q) { return x + (q / nb) * ldx + (q % nb) * 16; };
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < work; q += 2 * stride) {
    const int64_t q1 = q + stride;
    const uint16_t* p0 = src(q);
    const u32x4 a0 = ld16(p0), a1 = ld16(p0 + 8);
    u32x4 b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
    if (q1 < work) {
      const uint16_t* p1 = src(q1);
      b0 = ld16(p1);
      b1 = ld16(p1 + 8);
    }
    nv_block16(x, K, ldx, nb, q, s_t, d6, codes, scales, a0, a1);
    if (q1 < work) nv_block16(x, K, ldx, nb, q1, s_t, d6, codes, scales, b0, b1);
  }
}

static hipError_t queue_nv_encode(const uint16_t* x, int64_t rows, int64_t K, int64_t ldx, uint8_t* codes,
                                  uint8_t* scales, uint32_t* partials, int nparts, float* tensor_scale,
                                  hipStream_t s) {
  // one thread per pair of blocks (even block count) or per two blocks, at most
  // kNvEncodeGroups workgroups (eight per CU, all resident): each reduces the amax
  // partials once, then strides over the pairs
  const int64_t work = rows * (K >> 5) + (((K >> 4) & 1) ? rows : 0);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, kNvEncodeGroups));
  hipLaunchKernelGGL(nv_encode_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, K, ldx, codes, scales,
                     partials, nparts, tensor_scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- fused pass with t = X L1
// A workgroup owns `rows` (<= 32) consecutive rows and walks K in chunks of 256
// elements.  Each chunk of its rows of X and of L1^T (r rows) goes straight into
// LDS, one contiguous KB per wave instruction (two rows of 512 bytes; the 16-byte
// chunks XOR-swizzled by row & 15 so that the MFMA's column reads of 32 rows hit 16
// distinct bank groups per pass).  From LDS, one lane per (row, 32-element block)
// encodes the block, and wave w runs the MFMAs of K steps 2w, 2w+1 of the chunk
// (32 x 32 x 16 bf16: rows of X against the rows of L1^T), accumulating its own
// partial t, reduced across the waves at the end.  A ring of four stages, one
// barrier per chunk: the loads of chunks c+1..c+3 are in flight while chunk c is
// worked on (one chunk of 18 rows is only 9 KB, so a single chunk ahead would
// leave too few bytes in flight per CU to cover HBM latency: 15.3 us at 4608 x 3072
// with two stages, 11.5 us with four).  Every wave issues the same number of loads
// per chunk (rows past the workgroup's read zeros; with smoothing wave 0 issues one
// more, the chunk's factors), so the wait for chunk c is a fixed count of younger
// loads.
constexpr int kFKC = 256;                    // K elements per chunk
constexpr int kFWaves = 8;
constexpr int kFRowBytes = kFKC * 2;         // 512
constexpr int kFOp = 32 * kFRowBytes;        // one operand's rows of a chunk
constexpr int kFDepth = 4;                   // ring stages
constexpr int kFXLoads = 32 / 2 / kFWaves;   // X load instructions per wave per chunk

template <int FMT, int R, bool SMOOTH = false>
__global__ __launch_bounds__(kFWaves * 64) void quant_act_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int rows,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const uint32_t* __restrict__ partials,
    int nparts, float* __restrict__ tensor_scale, const uint16_t* __restrict__ l1t, float* __restrict__ t,
    const float* __restrict__ inv_s) {
  // a stage: X, then L1^T, then (smoothing) the chunk's 256 factors, which wave 0
  // loads with one more instruction (factors read from global memory inside the
  // loop would make the compiler's waits for them drain the whole ring)
  constexpr int kFactOff = (R > 0 ? 2 : 1) * kFOp;
  constexpr int kStage = kFactOff + (SMOOTH ? kFKC * 4 : 0);
  constexpr int kLoads = kFXLoads + R / 2 / kFWaves;        // per wave per chunk (wave 0: + SMOOTH)
  static_assert(R % (2 * kFWaves) == 0, "L1^T rows split evenly over the waves");
  static_assert(kFDepth * kStage >= kFWaves * 32 * 32 * 4, "t partials fit the ring");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFDepth * kStage];
  __shared__ uint32_t lds4[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.x * rows;
  const int nr = (int)min<int64_t>(rows, M - m0);
  const int64_t nblk = K >> 5;
  const int64_t sbytes = FMT == 0 ? nblk : 2 * nblk;   // scale bytes per row
  const int nchunk = (int)((K + kFKC - 1) / kFKC);

  float s_t = 1.0f, d6 = 6.0f;
  if constexpr (FMT == 1) {
    // the tensor scale from the amax launch's partial maxima (the first 256 threads
    // reduce them); workgroup 0 stores it
    uint32_t m = 0;
    if (threadIdx.x < 256) {
      for (int q = threadIdx.x; q < nparts; q += 256) m = max(m, partials[q]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
      if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = m;
    }
    __syncthreads();
    s_t = nv_tensor_scale(__uint_as_float(max(max(lds4[0], lds4[1]), max(lds4[2], lds4[3]))));
    d6 = 6.0f * s_t;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  }

  // buffer views: the workgroup's rows of X (through the last row's K), and L1^T
  const auto rx = make_rsrc(x + m0 * ldx, (uint32_t)(((int64_t)(nr - 1) * ldx + K) * 2));
  const auto rl = make_rsrc(l1t, (uint32_t)(R > 0 ? (int64_t)R * K * 2 : 0));
  const auto rf = make_rsrc(inv_s, (uint32_t)(SMOOTH ? K * 4 : 0));
  const uint32_t ldb = (uint32_t)(ldx * 2), kb2 = (uint32_t)(K * 2);

  // chunk c into stage st: instruction j covers rows 2j, 2j+1 (lane l: row 2j + l/32,
  // LDS slot l % 32, which holds the row's 16-byte chunk (l % 32) ^ (row & 15)).
  // Rows past nr of X read past the view (zeros); bytes past K within a row are
  // never used (blocks and K steps past K are skipped).
  auto load_chunk = [&](int c, int st) {
    uint8_t* base = lds + st * kStage;
    const int p = lane & 31;
#pragma unroll
    for (int jj = 0; jj < kFXLoads; ++jj) {
      const int j = wave + jj * kFWaves;
      const int rr = 2 * j + (lane >> 5);
      const uint32_t off = rr < nr ? (uint32_t)rr * ldb + (uint32_t)(c * kFKC + 8 * (p ^ (rr & 15))) * 2 : kOOB;
      dma_ld16(rx, base + j * 1024, off);
    }
    if constexpr (R > 0) {
#pragma unroll
      for (int jj = 0; jj < R / 2 / kFWaves; ++jj) {
        const int j = wave + jj * kFWaves;
        const int rr = 2 * j + (lane >> 5);
        dma_ld16(rl, base + kFOp + j * 1024, (uint32_t)rr * kb2 + (uint32_t)(c * kFKC + 8 * (p ^ (rr & 15))) * 2);
      }
    }
    if constexpr (SMOOTH) {
      // lane l: factors 4 l .. 4 l + 3 of the chunk (past K: zeros, never used)
      if (wave == 0) dma_ld16(rf, base + kFactOff, (uint32_t)(c * kFKC + 4 * lane) * 4);
    }
  };

  v16f acc = {};
  auto process_chunk = [&](int c, int st) {
    const uint8_t* base = lds + st * kStage;
    // encodes: one lane per (row, block of the chunk)
    for (int item = threadIdx.x; item < nr * 8; item += kFWaves * 64) {
      const int rr = item >> 3, b = item & 7;
      const int64_t blk = (int64_t)c * 8 + b;
      if (blk >= nblk) continue;
      uint32_t w[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = ld16(base + rr * kFRowBytes + (((4 * b + q) ^ (rr & 15)) << 4));
        w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
      }
      const int64_t row = m0 + rr;
      u32x4 cw;
      if (FMT == 0 && SMOOTH) {
        const int E = mx_encode_smoothed(w, reinterpret_cast<const float*>(base + kFactOff) + 32 * b, &cw);
        scales[row * sbytes + blk] = (uint8_t)(E + 127);
      } else if (FMT == 0) {
        const int E = mx_block_exponent(bf16_amax_bits<16>(w));
        const float sc = exp2i(E);
        cw = u32x4{fp4_encode8_pow2(w, sc), fp4_encode8_pow2(w + 4, sc),
                   fp4_encode8_pow2(w + 8, sc), fp4_encode8_pow2(w + 12, sc)};
        scales[row * sbytes + blk] = (uint8_t)(E + 127);
      } else {
        const uint32_t sc = nv_encode32(w, s_t, d6, &cw);
        *reinterpret_cast<uint16_t*>(scales + row * sbytes + 2 * blk) = (uint16_t)sc;
      }
      st16(codes + row * (K >> 1) + blk * 16, cw);
    }
    if constexpr (R > 0) {
      // K steps 2 wave, 2 wave + 1 of the chunk: lane half h holds elements 8h..8h+7
      // of the step, i.e. chunk 2s + h of the row
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const int s = 2 * wave + ss;
        if ((int64_t)c * kFKC + 16 * s >= K) break;
        const int slot = (2 * s + h) ^ (i & 15);
        const u32x4 a = ld16(base + i * kFRowBytes + (slot << 4));
        const u32x4 b = ld16(base + kFOp + i * kFRowBytes + (slot << 4));
        acc = mfma_bf16_32x32x16(a, b, acc);
      }
    }
  };

  for (int c = 0; c < kFDepth - 1 && c < nchunk; ++c) load_chunk(c, c);
  for (int c = 0; c < nchunk; ++c) {
    // chunk c has landed for every wave (loads complete in issue order, so it is
    // done once at most the younger chunks' loads are pending), and every wave is
    // done with chunk c-1, whose stage the next load reuses
    const int younger = min(kFDepth - 2, nchunk - 1 - c);
    if (SMOOTH && wave == 0) {
      if (younger >= 2) wait_vmcnt<2 * (kLoads + 1)>();
      else if (younger == 1) wait_vmcnt<kLoads + 1>();
      else wait_vmem();
    } else {
      if (younger >= 2) wait_vmcnt<2 * kLoads>();
      else if (younger == 1) wait_vmcnt<kLoads>();
      else wait_vmem();
    }
    barrier_after_wait();
    if (c + kFDepth - 1 < nchunk) load_chunk(c + kFDepth - 1, (c + kFDepth - 1) % kFDepth);
    process_chunk(c, c % kFDepth);
  }

  if constexpr (R > 0) {
    // the ring is free once every wave is past its last chunk
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
    // acc: rows = x rows (8*(v/4) + 4*h + v%4), column = t column (lane % 32)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave * 1024 + acc_row(v, lane) * 32 + i] = acc[v];
    __syncthreads();
    constexpr int kR = R > 0 ? R : 1;
    for (int idx = threadIdx.x; idx < 32 * R; idx += kFWaves * 64) {
      const int rr = idx / kR, cc = idx % kR;
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kFWaves; ++wv) sum += red[wv * 1024 + rr * 32 + cc];
      if (rr < nr) t[(m0 + rr) * R + cc] = sum;
    }
  }
}

template <int FMT, int R, bool SMOOTH = false>
static void queue_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                        uint8_t* scales, const uint32_t* partials, int nparts, float* tensor_scale,
                        const uint16_t* l1t, float* t, hipStream_t s, const float* inv_s = nullptr) {
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
  hipLaunchKernelGGL((quant_act_kernel<FMT, R, SMOOTH>), dim3(grid), dim3(kFWaves * 64), 0, s, x, M, K, ldx,
                     rows, codes, scales, partials, nparts, tensor_scale, l1t, t, inv_s);
}

hipError_t launch_quantize_act(int fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               const uint16_t* l1t, int r, float* t, hipStream_t s,
                               uint32_t* nv_scratch, const float* inv_s) {
  if (fmt == 0 && inv_s != nullptr) {
    if (r == 0) queue_quant<0, 0, true>(x, M, K, ldx, codes, scales, nullptr, 0, nullptr, l1t, t, s, inv_s);
    else if (r == 16) queue_quant<0, 16, true>(x, M, K, ldx, codes, scales, nullptr, 0, nullptr, l1t, t, s, inv_s);
    else queue_quant<0, 32, true>(x, M, K, ldx, codes, scales, nullptr, 0, nullptr, l1t, t, s, inv_s);
    return hipGetLastError();
  }
  if (fmt == 0) {
    // without the low-rank term, one thread per block (no lane idles, every load
    // instruction covers a contiguous 4 KB)
    if (r == 0) return queue_mx_rows<kBlkMXFP4>(x, M, K, ldx, 1, codes, scales, s);
    if (r == 16) queue_quant<0, 16>(x, M, K, ldx, codes, scales, nullptr, 0, nullptr, l1t, t, s);
    else queue_quant<0, 32>(x, M, K, ldx, codes, scales, nullptr, 0, nullptr, l1t, t, s);
    return hipGetLastError();
  }
  // NVFP4: partial maxima into the scratch, then the encode launch
  const int parts = nv_amax_grid(M * K);
  const hipError_t e = queue_nv_amax(x, M, K, ldx, 1, nv_scratch, parts, s);
  if (e != hipSuccess) return e;
  if (r == 0) return queue_nv_encode(x, M, K, ldx, codes, scales, nv_scratch, parts, tensor_scale, s);
  if (r == 16) queue_quant<1, 16>(x, M, K, ldx, codes, scales, nv_scratch, parts, tensor_scale, l1t, t, s);
  else queue_quant<1, 32>(x, M, K, ldx, codes, scales, nv_scratch, parts, tensor_scale, l1t, t, s);
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
  // x / scale is the IEEE quotient either way: through the row's reciprocal
  // (nv_quotient) for scale in [2^-100, 2^100], else by division
  auto encode8 = [&](int64_t c, const uint32_t* w, float scale, float y) {
    uint32_t packed = 0;
    if (scale >= 0x1p-100f && scale <= 0x1p100f) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
        const float q = fminf(fmaxf(__builtin_rintf(nv_quotient(v, scale, y)), -8.0f), 7.0f);
        packed |= ((uint32_t)(int)q & 0xFu) << (4 * j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
        const float q = fminf(fmaxf(__builtin_rintf(v / scale), -8.0f), 7.0f);
        packed |= ((uint32_t)(int)q & 0xFu) << (4 * j);
      }
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
    const float scale = wave_scale(m), y = 1.0f / scale;
#pragma unroll
    for (int i = 0; i < kRegChunks; ++i)
      if (lane + 64 * i < chunks) encode8(lane + 64 * i, w[i], scale, y);
    return;
  }
  uint32_t m = 0;
  for (int64_t c = lane; c < chunks; c += 64) {
    uint32_t w[4];
    load8(c, w);
    m = max(m, bf16_amax_bits<4>(w));
  }
  const float scale = wave_scale(m), y = 1.0f / scale;
  for (int64_t c = lane; c < chunks; c += 64) {
    uint32_t w[4];
    load8(c, w);
    encode8(c, w, scale, y);
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

// MXFP4: one thread per (column n, 32-element block).  NVFP4: one thread per
// (column n, 16-element block), the tensor scale from the partial maxima of the
// amax launch (reduced by every workgroup; workgroup 0 stores s_t).
template <int FMT>
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                       int64_t N, int64_t sk, int64_t sn,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       const uint32_t* __restrict__ partials, int nparts,
                                                       float* __restrict__ tensor_scale) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (FMT == 0) {
    const int64_t nblk = K >> 5;
    if (q >= N * nblk) return;
    const int64_t n = q % N, blk = q / N;
    uint32_t v[16];
    load_strided(w, blk * 32, n, sk, sn, 32, v);
    const int E = mx_block_exponent(bf16_amax_bits<16>(v));
    const float sc = exp2i(E);
    st16(codes + n * (K >> 1) + blk * 16, u32x4{fp4_encode8_pow2(v, sc), fp4_encode8_pow2(v + 4, sc),
                                                 fp4_encode8_pow2(v + 8, sc), fp4_encode8_pow2(v + 12, sc)});
    scales[n * nblk + blk] = (uint8_t)(E + 127);
    return;
  }
  __shared__ uint32_t lds4[4];
  const float s_t = nv_tensor_scale(__uint_as_float(reduce_partials(partials, nparts, lds4)));
  if (blockIdx.x == 0 && threadIdx.x == 0) *tensor_scale = s_t;
  const int64_t nb = K >> 4;
  if (q >= N * nb) return;
  const int64_t n = q % N, blk = q / N;
  uint32_t v[8];
  load_strided(w, blk * 16, n, sk, sn, 16, v);
  const uint32_t code = e4m3_code(__uint_as_float(bf16_amax_bits<8>(v) << 16) / (6.0f * s_t));
  uint32_t c[2];
  nv_encode16(v, e4m3_value(code) * s_t, c);
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2*>(codes + n * (K >> 1) + blk * 8) = u32x2{c[0], c[1]};
  scales[n * nb + blk] = (uint8_t)code;
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
  // w / s is the IEEE quotient either way: through the group's reciprocal
  // (nv_quotient) for s in [2^-100, 2^100], else by division
  const bool rcp = s >= 0x1p-100f && s <= 0x1p100f;
  const float y = 1.0f / s;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t pair = v[4 * d + j];
      const float a = bf16_lo(pair), b = bf16_hi(pair);
      const float qa = rcp ? nv_quotient(a, s, y) : a / s;
      const float qb = rcp ? nv_quotient(b, s, y) : b / s;
      const float q0 = fminf(fmaxf(rintf(qa) + z, 0.0f), 15.0f);
      const float q1 = fminf(fmaxf(rintf(qb) + z, 0.0f), 15.0f);
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
                               float* tensor_scale, hipStream_t s, uint32_t* nv_scratch) {
  // K-contiguous rows with 16-byte alignment: the rows of W^T are quantized exactly
  // like activation rows (same blocks along K, same encoders), with vector loads
  const bool rows = sk == 1 && sn % 8 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0;
  if (rows && fmt != 2)
    return launch_quantize_act(fmt, w, N, K, sn, codes, static_cast<uint8_t*>(scales), tensor_scale,
                               nullptr, 0, nullptr, s, nv_scratch);
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
  if (fmt == 0) {
    const int64_t work = N * (K >> 5);
    hipLaunchKernelGGL(pack_fp4_kernel<0>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, s, w, K, N,
                       sk, sn, codes, static_cast<uint8_t*>(scales), nullptr, 0, nullptr);
    return hipGetLastError();
  }
  // NVFP4, logical [K, N]: rows k (stride sk), columns n (stride sn)
  const int parts = nv_amax_grid(K * N);
  const hipError_t e = queue_nv_amax(w, K, N, sk, sn, nv_scratch, parts, s);
  if (e != hipSuccess) return e;
  const int64_t work = N * (K >> 4);
  hipLaunchKernelGGL(pack_fp4_kernel<1>, dim3((unsigned)std::max<int64_t>(1, (work + 255) / 256)), dim3(256),
                     0, s, w, K, N, sk, sn, codes, static_cast<uint8_t*>(scales), nv_scratch, parts,
                     tensor_scale);
  return hipGetLastError();
}

}  // namespace q4
