// INT4 x INT4 GEMM, symmetric with one fp32 scale per row of each operand (the
// per-channel quantizer of the SVDQuant Guide's "Step 1"), on the INT8 MFMA:
// gfx950 has no 4-bit integer matrix instruction, so the nibbles are widened to
// int8 between the LDS read and the MFMA ("Quantization for the impatient": a
// 4-bit format pays off only where the hardware multiplies it natively).
//
// Y[m, n] = fp32(fp32(sum_k qa[m,k] qb[n,k]) * sa[m]) * sb[n] (+ bias).  The sum is
// exact in int32 (|q| <= 7, so |sum| <= 49 K), and its conversion to fp32 is exact
// for K <= 2^18.
//
// Tiling as the MXFP4 GEMM: 256 x 256 output tile per workgroup of 4 waves, wave
// (wm, wn) owning 128 x 128 as 4 x 4 tiles of v_mfma_i32_32x32x32_i8 with int32
// accumulators in the matrix registers; K-tiles of 256 codes (128 bytes per row)
// loaded straight into two LDS stages with 16-byte chunks XOR-swizzled by row.  The
// tiles that do not fill a last round over the CUs run as two 128-row halves.
// Lane half h reads K blocks 4h + s (16 bytes, 32 codes) in step s; the 32 codes
// feed two MFMAs of 16 int8 each.  Both operands are widened with the same
// permutation (even nibbles, then odd), which a sum over K allows.
#include <type_traits>

#include "q4_epilogue.h"

namespace q4 {

namespace {

constexpr int kI4BM = 256, kI4BN = 256, kI4KT = 256, kI4KTB = kI4KT / 2;
// 8 waves, two per SIMD: wave (wm, wn) = (w % 2, w / 2) owns 128 x 32 F (F = 2 in a
// whole tile, 128 int32 accumulators per lane), so one wave's nibble widening issues
// while the SIMD's other wave runs MFMAs.  The code also builds with 4 waves of
// 128 x 128 (F = 4).
constexpr int kI4Waves = 8, kI4Threads = 64 * kI4Waves;
constexpr int kI4FFull = 512 / (32 * kI4Waves), kI4FHalf = kI4FFull / 2;   // weight sub-tiles per wave
constexpr int kI4OperandLds = 2 * 2 * kI4BM * kI4KTB;               // [operand][stage]
constexpr int kI4StageLds = kI4Waves * EpilogueShape<true, kI4FFull, 128>::kStageWaveBytes;
constexpr int kI4Lds = kI4StageLds > kI4OperandLds ? kI4StageLds : kI4OperandLds;
static_assert(kI4Waves * EpilogueShape<false, kI4FFull, 128>::kStageWaveBytes <= kI4Lds,
              "the epilogue stages each wave's output in the operand LDS");

// 8 packed signed nibbles -> 8 int8: the even nibbles in lo, the odd ones in hi.
// Per byte, t = v ^ 8 maps the nibble v to 8 + v (v < 8) or v - 8; adding 0x78 and
// flipping bit 7 gives v or v - 16 as int8, with no carry between bytes.
__device__ __forceinline__ void i4_widen(uint32_t d, uint32_t& lo, uint32_t& hi) {
  lo = (((d & 0x0F0F0F0Fu) ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
  hi = ((((d >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// A 16-byte fragment (32 codes) -> the two int8 MFMA operands it feeds.
__device__ __forceinline__ void i4_operands(u32x4 f, v4i& op0, v4i& op1) {
  uint32_t a, b, c, d;
  i4_widen(f[0], a, b);
  i4_widen(f[1], c, d);
  op0 = v4i{(int)a, (int)b, (int)c, (int)d};
  i4_widen(f[2], a, b);
  i4_widen(f[3], c, d);
  op1 = v4i{(int)a, (int)b, (int)c, (int)d};
}

// One output tile of 256 activation rows x 64 F weight rows at (m0, n0): F weight
// sub-tiles of 32 rows per wave (4 in a whole tile, 2 in a half).
template <bool OUT_F32, int F>
__device__ __forceinline__ void i4_tile(uint8_t* lds_raw, const uint8_t* __restrict__ ac,
                                        const float* __restrict__ as, const uint8_t* __restrict__ bc,
                                        const float* __restrict__ bs, int64_t M, int64_t N, int64_t K,
                                        const uint16_t* __restrict__ bias, void* __restrict__ y,
                                        int64_t ldy, int64_t m0, int64_t n0) {
  constexpr int kTN = 32 * F * (kI4Waves / 2), kRowsB = kTN / kI4Waves;   // weight rows: per tile, per wave
  constexpr int kRowsA = kI4BM / kI4Waves;                               // activation rows per wave
  auto& lds = *reinterpret_cast<uint8_t(*)[2][2][kI4BM * kI4KTB]>(lds_raw);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t kbytes = (uint32_t)(K >> 1), nblk = (uint32_t)(K >> 5);
  const int nkt = (int)((K + kI4KT - 1) / kI4KT);
  const uint32_t rows_a = rows_in(kI4BM, M, m0), rows_b = rows_in(kTN, N, n0);
  const auto rc_a = make_rsrc(ac + m0 * kbytes, rows_a * kbytes);
  const auto rc_b = make_rsrc(bc + n0 * kbytes, rows_b * kbytes);

  // K-tile kt -> stage: each wave moves kRowsA activation and kRowsB weight rows, 8 rows
  // of 128 bytes per instruction (lane i: row i / 8, stored chunk i % 8 holding
  // global chunk (i % 8) ^ lds_swz<8>(row)); rows and blocks past the matrix read as zero
  const int lr = lane >> 3, lp = lane & 7;
  auto load_ktile = [&](int kt, int stage) {
    // row = 16 q + 8 (j % 2) + lr: its swizzle lds_swz<8>(row) is 4 (j % 2) + lr / 2
    uint32_t koff[2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const uint32_t blk = (uint32_t)kt * 8 + (lp ^ (4 * jp + (lr >> 1)));
      koff[jp] = blk < nblk ? blk * 16 : kOOB;
    }
#pragma unroll
    for (int j = 0; j < kRowsA / 8; ++j) {
      const uint32_t row = kRowsA * wave + 8 * j + lr;
      buf_ld16_lds(rc_a, &lds[0][stage][(kRowsA * wave + 8 * j) * kI4KTB], row * kbytes + koff[j & 1]);
    }
#pragma unroll
    for (int j = 0; j < kRowsB / 8; ++j) {
      const uint32_t row = kRowsB * wave + 8 * j + lr;
      buf_ld16_lds(rc_b, &lds[1][stage][(kRowsB * wave + 8 * j) * kI4KTB], row * kbytes + koff[j & 1]);
    }
  };
  // raw 16-byte fragments (32 codes), double-buffered across MFMA steps; widened to
  // int8 right before their MFMAs
  u32x4 fa[2][4], fb[2][F];
  auto read_frags = [&](int buf, int stage, int s) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = wm * 128 + 32 * g + r32;
      fa[buf][g] = ld16(&lds[0][stage][row * kI4KTB + (((4 * h + s) ^ lds_swz<8>(row)) << 4)]);
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int row = wn * 32 * F + 32 * f + r32;
      fb[buf][f] = ld16(&lds[1][stage][row * kI4KTB + (((4 * h + s) ^ lds_swz<8>(row)) << 4)]);
    }
  };

  v16i acc[F][4];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = v16i{};
  auto mma = [&](int buf) {
    v4i a0[4], a1[4], b0[F], b1[F];
#pragma unroll
    for (int g = 0; g < 4; ++g) i4_operands(fa[buf][g], a0[g], a1[g]);
#pragma unroll
    for (int f = 0; f < F; ++f) i4_operands(fb[buf][f], b0[f], b1[f]);
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        acc[f][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b0[f], a0[g], acc[f][g], 0, 0, 0);
        acc[f][g] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b1[f], a1[g], acc[f][g], 0, 0, 0);
      }
  };

  // Pipeline: K-tiles kt and kt+1 sit in the two stages.  Each MFMA step runs while
  // the fragments of the next are read; in step 3 every wave first waits for K-tile
  // kt+1 (loaded a whole K-tile earlier) and passes the barrier, which frees stage
  // kt % 2 for the loads of K-tile kt+2 and lets step 0 of K-tile kt+1 be read.
  // Loads past K read zeros and are never used.
  load_ktile(0, 0);
  load_ktile(1, 1);
  wait_vmem();
  __syncthreads();
  read_frags(0, 0, 0);
  auto ktile = [&](auto stage_c, int kt) {
    constexpr int st = decltype(stage_c)::value;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      read_frags((s + 1) & 1, st, s + 1);
      mma(s & 1);
    }
    wait_vmem();                                 // K-tile kt+1 has landed
    __syncthreads();                             // and every read of stage st is done
    load_ktile(kt + 2, st);
    read_frags(0, st ^ 1, 0);
    mma(1);
  };
  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    ktile(std::integral_constant<int, 0>{}, kt);
    ktile(std::integral_constant<int, 1>{}, kt + 1);
  }
  if (kt < nkt) ktile(std::integral_constant<int, 0>{}, kt);
  wait_vmem();                                   // the loads past K have landed
  __syncthreads();                               // before the epilogue reuses the LDS

  // scales: acc[f][g] register j is row m = m_base + 32 g + lane % 32, column
  // n = n_base + 32 f + 8 (j / 4) + 4 h + j % 4.  Indices past the matrix are clamped
  // (those results are never stored), so the loads need no branches.
  const int64_t n_base = n0 + wn * 32 * F, m_base = m0 + wm * 128;
  v16f accf[F][4];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float sb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t n = n_base + 32 * f + 8 * (j >> 2) + 4 * h + (j & 3);
      sb[j] = bs[n < N ? n : N - 1];
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t m = m_base + 32 * g + r32;
      const float sa = as[m < M ? m : M - 1];
#pragma unroll
      for (int j = 0; j < 16; ++j) accf[f][g][j] = (float)acc[f][g][j] * sa * sb[j];
    }
  }
  epilogue_store<OUT_F32, F, 128>(accf, n_base, m_base, M, N, bias, y, ldy, lane,
                                  lds_raw + wave * EpilogueShape<OUT_F32, F, 128>::kStageWaveBytes);
}

// Workgroup b -> a whole tile or, for b < 2 (tiles - full), a half of a leftover
// tile (weight rows 128 h .. +127), with the XCD-aware order of tile_of.
template <bool OUT_F32>
__global__ __launch_bounds__(kI4Threads) void gemm_i4_kernel(
    const uint8_t* __restrict__ ac, const float* __restrict__ as, const uint8_t* __restrict__ bc,
    const float* __restrict__ bs, int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n, int full) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kI4Lds];
  int vt, half, tm, tn;
  const bool is_half = tile_unit(blockIdx.x, tiles_m * tiles_n, full, &vt, &half);
  tile_of(vt, tiles_m, tiles_n, 4, &tm, &tn);
  const int64_t m0 = (int64_t)tm * kI4BM, n0 = (int64_t)tn * kI4BN + (is_half ? 128 * half : 0);
  if (n0 >= N) return;                                   // a half past the last weight row
  if (is_half)
    i4_tile<OUT_F32, kI4FHalf>(lds_raw, ac, as, bc, bs, M, N, K, bias, y, ldy, m0, n0);
  else
    i4_tile<OUT_F32, kI4FFull>(lds_raw, ac, as, bc, bs, M, N, K, bias, y, ldy, m0, n0);
}

}  // namespace

hipError_t launch_gemm_i4(const uint8_t* ac, const float* as, const uint8_t* bc, const float* bs,
                          int64_t M, int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kI4BM - 1) / kI4BM), tiles_n = (int)((N + kI4BN - 1) / kI4BN);
  const int tiles = tiles_m * tiles_n;
  // leftover tiles of the last round over the CUs (one workgroup per CU) run as halves
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
  }
  const int rem = tiles % cus;
  const int full = (tiles > cus && rem > 0 && 2 * rem <= cus) ? tiles - rem : tiles;
  const unsigned grid = (unsigned)(full + 2 * (tiles - full));
  if (ep.out_f32)
    hipLaunchKernelGGL((gemm_i4_kernel<true>), dim3(grid), dim3(kI4Threads), 0, s, ac, as, bc, bs, M, N, K,
                       ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
  else
    hipLaunchKernelGGL((gemm_i4_kernel<false>), dim3(grid), dim3(kI4Threads), 0, s, ac, as, bc, bs, M, N, K,
                       ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
  return hipGetLastError();
}

}  // namespace q4
