// Epilogue shared by the GEMM kernels.  The main loop leaves a wave with an F x 4
// grid of 32x32 fp32 accumulators (F = 4 or 2 weight sub-tiles) laid out as
// D[n][m] (MFMA A operand = weight rows n, B operand = activation rows m), so lane
// l holds output row m = l%32 of each tile and, per register group v/4, four
// consecutive output columns n.
//
// The low-rank up-projection t L2 runs as bf16 MFMAs on the same accumulators,
// with t split into bf16 hi + lo (before the K loop or after it); the store adds
// the bias and writes bf16 or fp32.
#pragma once

#include <type_traits>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

// t = hi + lo for a pair of fp32 values, hi and lo bf16 pairs (packed, element 0
// in the low half).  The hardware conversion rounds to nearest even; v - hi is
// exact in fp32, so hi + lo carries 16 significant bits of t.
__device__ __forceinline__ void split_bf16_pair(float v0, float v1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, v2bf{(__bf16)v0, (__bf16)v1});
  const float r0 = v0 - __uint_as_float(hi << 16);
  const float r1 = v1 - __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(uint32_t, v2bf{(__bf16)r0, (__bf16)r1});
}

// acc[f][g]: f = weight (n) sub-tile, g = activation (m) sub-tile, 32 x 32 each.
// n_base / m_base: first n / m of the wave's (32 F) x 128 region.
template <int R, int F>
__device__ __forceinline__ void lowrank_accumulate(v16f (&acc)[F][4], int64_t n_base, int64_t m_base,
                                                 int64_t M, int64_t N, const float* __restrict__ t,
                                                 const uint16_t* __restrict__ l2t, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < R / 16; ++ks) {
    u32x4 thi[4], tlo[4], l2f[F];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t m = m_base + 32 * g + r32;
      thi[g] = u32x4{0, 0, 0, 0};
      tlo[g] = u32x4{0, 0, 0, 0};
      if (m < M) {
        const float* src = t + m * R + 16 * ks + 8 * h;
        const u32x4 a = ld16(src), b = ld16(src + 4);
        const uint32_t tv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t hi, lo;
          split_bf16_pair(__uint_as_float(tv[2 * d]), __uint_as_float(tv[2 * d + 1]), hi, lo);
          thi[g][d] = hi;
          tlo[g][d] = lo;
        }
      }
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int64_t n = n_base + 32 * f + r32;
      l2f[f] = (n < N) ? ld16(l2t + n * R + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[f][g] = mfma_bf16_32x32x16(l2f[f], thi[g], acc[f][g]);
        acc[f][g] = mfma_bf16_32x32x16(l2f[f], tlo[g], acc[f][g]);
      }
  }
}

// The same t L2 term with both operands already in LDS: lds_t holds the tile's t
// rows (fp32, 4R bytes each, row m_local at m_local * 4R), lds_l2 its L2^T rows
// (bf16, 2R bytes each), both with their 16-byte chunks swizzled by lds_swz.
// m_loc / n_loc: first row of the wave's region within the tile (multiples of 16).
template <int R, int F>
__device__ __forceinline__ void lowrank_accumulate_lds(v16f (&acc)[F][4], const uint8_t* lds_t,
                                                       const uint8_t* lds_l2, int m_loc, int n_loc,
                                                       int lane) {
  constexpr int kCT = 4 * R / 16, kCL = 2 * R / 16;     // 16-byte chunks per row
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < R / 16; ++ks) {
    u32x4 thi[4], tlo[4], l2f[F];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = m_loc + 32 * g + r32, c = 4 * ks + 2 * h;   // chunks c, c + 1: t[16 ks + 8 h ..]
      const uint8_t* src = lds_t + row * (4 * R);
      const u32x4 a = ld16(src + ((c ^ lds_swz<kCT>(row)) << 4)),
                  b = ld16(src + (((c + 1) ^ lds_swz<kCT>(row)) << 4));
      const uint32_t tv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t hi, lo;
        split_bf16_pair(__uint_as_float(tv[2 * d]), __uint_as_float(tv[2 * d + 1]), hi, lo);
        thi[g][d] = hi;
        tlo[g][d] = lo;
      }
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int row = n_loc + 32 * f + r32, c = 2 * ks + h;       // L2^T[16 ks + 8 h ..]
      l2f[f] = ld16(lds_l2 + row * (2 * R) + ((c ^ lds_swz<kCL>(row)) << 4));
    }
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[f][g] = mfma_bf16_32x32x16(l2f[f], thi[g], acc[f][g]);
        acc[f][g] = mfma_bf16_32x32x16(l2f[f], tlo[g], acc[f][g]);
      }
  }
}

// A 16-byte store marked non-temporal: the output is not read again by this
// kernel, so it should not displace the operands in the caches.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Output staging through LDS: each wave writes a 128-row slab of its 128 x (32 F)
// output region into LDS, ROW_BYTES wide at most (rows padded by 16 bytes), then
// reads it back so that every store instruction writes whole 128-byte row segments
// (8 rows of 128 bytes, or 4 of 256).  Direct stores from the MFMA layout would
// write 8- or 16-byte pieces of 32 different rows per instruction.
template <bool OUT_F32, int F, int ROW_BYTES>
struct EpilogueShape {
  static constexpr int kElem = OUT_F32 ? 4 : 2;
  static constexpr int kFPerPassMax = ROW_BYTES / (32 * kElem);          // 32-column blocks
  // the largest count of sub-tiles per pass that fits the row and divides F
  static constexpr int per_pass() {
    int d = F < kFPerPassMax ? F : kFPerPassMax;
    while (F % d != 0) --d;
    return d;
  }
  static constexpr int kFPerPass = per_pass();
  static constexpr int kPasses = F / kFPerPass;
  static_assert(kPasses * kFPerPass == F, "every sub-tile is staged");
  static constexpr int kRowBytes = 32 * kFPerPass * kElem;
  static constexpr int kStageRowBytes = kRowBytes + 16;
  static constexpr int kStageWaveBytes = 128 * kStageRowBytes;
};
// the 4-wave bf16 GEMMs' staging (128-byte rows): what their operand LDS must hold
constexpr int kStageWaveBytes = EpilogueShape<false, 4, 128>::kStageWaveBytes;   // 18432
constexpr int kEpilogueLdsBytes = 4 * EpilogueShape<true, 4, 128>::kStageWaveBytes;

// One staging pass: the accumulators of weight sub-tiles pass * kFPerPass ..
// + kFPerPass - 1, scaled (SCALED) and with the bias added (BIAS), into this wave's
// LDS rows: row m_local = 32 g + lane%32 (G activation sub-tiles of 32 rows),
// columns 32 f' + 8 vq + 4 h .. +3.
template <bool OUT_F32, int F, int ROW_BYTES, bool SCALED, bool BIAS, int G = 4>
__device__ __forceinline__ void epilogue_stage_pass(v16f (&acc)[F][G], int pass, int64_t n_base,
                                                    int64_t N, const uint16_t* __restrict__ bias,
                                                    int lane, uint8_t* stage, float scale) {
  using S = EpilogueShape<OUT_F32, F, ROW_BYTES>;
  const int r32 = lane & 31, h = lane >> 5;
  constexpr int kElem = S::kElem;
#pragma unroll
  for (int fp = 0; fp < S::kFPerPass; ++fp) {
    const int f = pass * S::kFPerPass + fp;
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      // bias of the 4 consecutive columns this lane holds in register group vq
      const int64_t n = n_base + 32 * f + 8 * vq + 4 * h;
      float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (BIAS && bias != nullptr) {           // the fp32 path adds zeros without a bias
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n + j < N) b[j] = __uint_as_float((uint32_t)bias[n + j] << 16);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        uint8_t* dst = stage + (32 * g + r32) * S::kStageRowBytes + (32 * fp + 8 * vq + 4 * h) * kElem;
        float a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = acc[f][g][4 * vq + j];
          if (SCALED) a[j] = BIAS ? __builtin_fmaf(a[j], scale, b[j]) : a[j] * scale;
          else if (BIAS) a[j] += b[j];
        }
        if (OUT_F32) {
          *reinterpret_cast<v4f*>(dst) = v4f{a[0], a[1], a[2], a[3]};
        } else {
          const v2bf p0 = {(__bf16)a[0], (__bf16)a[1]};
          const v2bf p1 = {(__bf16)a[2], (__bf16)a[3]};
          typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
        }
      }
    }
  }
}

// y = scale * acc + bias (SCALED), or acc + bias, for a wave region of 32 G rows.
// The bias is added, and the scale applied, pass by pass, so only the accumulators
// being staged are moved out of the matrix registers; without a bias the add is
// skipped.
template <bool OUT_F32, int F, int ROW_BYTES = 128, bool SCALED = false, int G = 4>
__device__ __forceinline__ void epilogue_store(v16f (&acc)[F][G], int64_t n_base, int64_t m_base,
                                               int64_t M, int64_t N,
                                               const uint16_t* __restrict__ bias, void* y,
                                               int64_t ldy, int lane, uint8_t* stage,
                                               float scale = 1.0f) {
  using S = EpilogueShape<OUT_F32, F, ROW_BYTES>;
  constexpr int kElem = S::kElem;
  constexpr int kColsPerPass = 32 * S::kFPerPass;
  constexpr int kStageRow = S::kStageRowBytes;
  constexpr int kLanesPerRow = S::kRowBytes / 16;
  constexpr int kRowsPerStore = 64 / kLanesPerRow;
  constexpr int kPer16 = 16 / kElem;             // elements per 16-byte store
#pragma unroll
  for (int pass = 0; pass < S::kPasses; ++pass) {
    if (pass > 0) {
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): previous pass read back
      __builtin_amdgcn_wave_barrier();
    }
    // fp32 output keeps one path (a second copy of the pass made the compiler spill);
    // it reads the bias only when there is one
    if (OUT_F32 || bias)
      epilogue_stage_pass<OUT_F32, F, ROW_BYTES, SCALED, true, G>(acc, pass, n_base, N, bias, lane, stage, scale);
    else
      epilogue_stage_pass<OUT_F32, F, ROW_BYTES, SCALED, false, G>(acc, pass, n_base, N, bias, lane, stage, scale);
    __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    // LDS -> global: kLanesPerRow lanes per row (16 bytes each), whole row segments
    const int col_bytes = (lane % kLanesPerRow) * 16;
    const int64_t n = n_base + pass * kColsPerPass + col_bytes / kElem;
#pragma unroll 4
    for (int it = 0; it < 32 * G / kRowsPerStore; ++it) {
      const int ml = kRowsPerStore * it + lane / kLanesPerRow;
      const int64_t m = m_base + ml;
      const u32x4 v = ld16(stage + ml * kStageRow + col_bytes);
      if (m < M) {
        uint8_t* dst = static_cast<uint8_t*>(y) + (m * ldy + n) * kElem;
        if (n + kPer16 <= N) {
          st16_stream(dst, v);
        } else if (n < N) {
          const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
          for (int j = 0; j < kPer16 && n + j < N; ++j) {
            if (OUT_F32) reinterpret_cast<uint32_t*>(dst)[j] = w[j];
            else reinterpret_cast<uint16_t*>(dst)[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
          }
        }
      }
    }
  }
}

// bf16 output of a wave's 128 x 32F region staged in one pass and held in
// registers until it is stored: out[i] holds the 16 bytes of store i (row
// kRowsPerStore i + lane / kLanesPerRow, bytes 16 (lane % kLanesPerRow) ..).  This
// lets a kernel free its LDS (and queue other loads) before the stores go out.
template <int F>
struct RegEpilogue {
  using S = EpilogueShape<false, F, 64 * F>;
  static_assert(S::kPasses == 1, "one staging pass");
  static constexpr int kLanesPerRow = S::kRowBytes / 16;
  static constexpr int kRowsPerStore = 64 / kLanesPerRow;
  static constexpr int kStores = 128 / kRowsPerStore;
};

template <int F>
__device__ __forceinline__ void epilogue_stage_to_regs(v16f (&acc)[F][4], int64_t n_base, int64_t N,
                                                       const uint16_t* __restrict__ bias, int lane,
                                                       uint8_t* stage,
                                                       u32x4 (&out)[RegEpilogue<F>::kStores]) {
  using E = RegEpilogue<F>;
  if (bias)
    epilogue_stage_pass<false, F, 64 * F, false, true>(acc, 0, n_base, N, bias, lane, stage, 1.0f);
  else
    epilogue_stage_pass<false, F, 64 * F, false, false>(acc, 0, n_base, N, bias, lane, stage, 1.0f);
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  const int col_bytes = (lane % E::kLanesPerRow) * 16;
#pragma unroll
  for (int it = 0; it < E::kStores; ++it)
    out[it] = ld16(stage + (E::kRowsPerStore * it + lane / E::kLanesPerRow) * E::S::kStageRowBytes + col_bytes);
}

// The stores of epilogue_stage_to_regs' registers, for a region wholly inside the
// output (no masks).
template <int F>
__device__ __forceinline__ void epilogue_store_regs(const u32x4 (&out)[RegEpilogue<F>::kStores],
                                                    int64_t n_base, int64_t m_base, void* y,
                                                    int64_t ldy, int lane) {
  using E = RegEpilogue<F>;
  const int64_t n = n_base + (lane % E::kLanesPerRow) * 8;
  uint16_t* base = static_cast<uint16_t*>(y) + (m_base + lane / E::kLanesPerRow) * ldy + n;
#pragma unroll
  for (int it = 0; it < E::kStores; ++it)
    st16_stream(base + (int64_t)E::kRowsPerStore * it * ldy, out[it]);
}

// MXFP4 output for the next layer: the bf16 output of a wave's 128 x 32F region is
// staged in one pass (as epilogue_stage_to_regs) and, instead of (or besides) being
// stored, each row's 32-column blocks are quantized exactly as quantize_act
// quantizes a bf16 activation: shared exponent E = floor(log2 amax) - 2 of the block's
// bf16 values, codes RNE_E2M1(y * 2**-E).  A lane reads 8 columns; the 4 lanes of a
// block exchange their maxima with DPP quad permutes.  Codes go to qc [M, N/2] (row
// stride ldc bytes, low nibble = even column), scale bytes to qs [M, N/32] (stride
// lds), the bf16 values to y when y is not null.  N is a multiple of 32, so a block
// is either wholly inside the output or wholly outside.
template <int F>
__device__ __forceinline__ void epilogue_store_mxfp4(v16f (&acc)[F][4], int64_t n_base, int64_t m_base,
                                                     int64_t M, int64_t N,
                                                     const uint16_t* __restrict__ bias, uint16_t* y,
                                                     int64_t ldy, uint8_t* qc, int64_t ldc, uint8_t* qs,
                                                     int64_t lds, int lane, uint8_t* stage) {
  using E = RegEpilogue<F>;
  if (bias)
    epilogue_stage_pass<false, F, 64 * F, false, true>(acc, 0, n_base, N, bias, lane, stage, 1.0f);
  else
    epilogue_stage_pass<false, F, 64 * F, false, false>(acc, 0, n_base, N, bias, lane, stage, 1.0f);
  __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): this wave's LDS writes done
  __builtin_amdgcn_wave_barrier();
  const int chunk = lane % E::kLanesPerRow;     // 8 columns: chunk / 4 is the block
  const int64_t n = n_base + chunk * 8;
#pragma unroll 4
  for (int it = 0; it < E::kStores; ++it) {
    const int ml = E::kRowsPerStore * it + lane / E::kLanesPerRow;
    const int64_t m = m_base + ml;
    const u32x4 v = ld16(stage + ml * E::S::kStageRowBytes + chunk * 16);
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
    uint32_t amax = bf16_amax_bits<4>(w);
    amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, false));  // lane ^ 1
    amax = max(amax, (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, false));  // lane ^ 2
    const int ex = mx_block_exponent(amax);
    const uint32_t codes = fp4_encode8_pow2(w, exp2i(ex));
    if (m < M && n < N) {
      *reinterpret_cast<uint32_t*>(qc + m * ldc + (n >> 1)) = codes;
      if ((chunk & 3) == 0) qs[m * lds + (n >> 5)] = (uint8_t)(ex + 127);
      if (y != nullptr) st16(y + m * ldy + n, v);
    }
  }
}

}  // namespace q4
