// MXFP4 x MXFP4 GEMM on the CDNA4 block-scaled MFMA, low-rank branch and bias
// fused into the epilogue.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), 128 x 128 per
// wave as 4 x 4 MFMA tiles of v_mfma_scale_f32_32x32x64_f8f6f4 (FP4 x FP4, one
// E8M0 scale per 32 K elements per row, applied by the MFMA itself).  K advances in
// tiles of 256 elements (128 bytes per row; 8 scale bytes per row).
//
// K order inside a K-tile: lane half h (= lane/32) of every fragment owns the
// contiguous blocks 4h .. 4h+3 of the tile, and MFMA step s (0..3) consumes block
// 4h + s from every lane.  A and B use the same assignment, so each MFMA sums
// products of matching K indices; its scale for the step is byte s of the lane's
// 4-byte scale word (the op_sel index), one aligned dword load per fragment.
//
// LDS: the two operand tiles (256 rows x 128 bytes each) are stored with 16-byte
// chunks XOR-swizzled by row (chunk c of row r at c ^ (r & 7)), so both the
// row-contiguous global->LDS writes and the 16-byte fragment reads are free of
// bank conflicts.  The next K-tile is fetched from global into registers while
// the current one is multiplied: two LDS stages, one barrier per K-tile, and the
// global loads for tile kt+2 in flight while tile kt is multiplied.
#include "q4_epilogue.h"

namespace q4 {

constexpr int kBM = 256, kBN = 256;
constexpr int kKT = 256;          // K elements per K-tile
constexpr int kKTB = kKT / 2;     // bytes per row per K-tile
constexpr int kThreads = 256;
constexpr int kGroupM = 4;

template <int R, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int64_t M, int64_t N, int64_t K, const float* __restrict__ t,
    const uint16_t* __restrict__ l2t, const uint16_t* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int tiles_m, int tiles_n) {
  // two stages x (activation tile, weight tile), 256 rows x 128 bytes each
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBM * kKTB];

  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, kGroupM, &tm, &tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;       // wave's n half, m half
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kbytes = K >> 1, nblk = K >> 5;
  const int nkt = (int)((K + kKT - 1) / kKT);

  // global -> LDS mapping: 16-byte chunk (row, c) with c = tid & 7, rows tid/8 + 32 j
  const int lrow = tid >> 3, lc = tid & 7;
  u32x4 ra[8], rb[8];
  uint32_t sa_next[4], sb_next[4];
  auto gload = [&](int kt) {
    const int64_t blk = (int64_t)kt * 8 + lc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = lrow + 32 * j;
      ra[j] = (m0 + row < M && blk < nblk) ? ld16(ac + (m0 + row) * kbytes + blk * 16) : u32x4{0, 0, 0, 0};
      rb[j] = (n0 + row < N && blk < nblk) ? ld16(bc + (n0 + row) * kbytes + blk * 16) : u32x4{0, 0, 0, 0};
    }
    // scale words: bytes for blocks 8kt + 4h .. 8kt + 4h + 3 of the lane's fragment rows
    const int64_t blk0 = (int64_t)kt * 8 + 4 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t m = m0 + wx * 128 + 32 * g + r32;
      sa_next[g] = (m < M && blk0 < nblk) ? *reinterpret_cast<const uint32_t*>(as + m * nblk + blk0) : 0x7F7F7F7Fu;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t n = n0 + wy * 128 + 32 * f + r32;
      sb_next[f] = (n < N && blk0 < nblk) ? *reinterpret_cast<const uint32_t*>(bs + n * nblk + blk0) : 0x7F7F7F7Fu;
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = lrow + 32 * j;
      const int off = row * kKTB + ((lc ^ (row & 7)) << 4);
      st16(&lds[stage][0][off], ra[j]);
      st16(&lds[stage][1][off], rb[j]);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = v16f{};

  uint32_t sa[4], sb[4];
  if (nkt > 0) {
    gload(0);
    lstore(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) { sa[g] = sa_next[g]; sb[g] = sb_next[g]; }
    if (nkt > 1) gload(1);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nkt) {
      lstore(stage ^ 1);                 // tile kt+1 (its loads were issued one iteration ago)
    }
    uint32_t sa_cur[4], sb_cur[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) { sa_cur[g] = sa[g]; sb_cur[g] = sb[g]; sa[g] = sa_next[g]; sb[g] = sb_next[g]; }
    if (kt + 2 < nkt) gload(kt + 2);
    const uint8_t* la = lds[stage][0];
    const uint8_t* lb = lds[stage][1];

#define Q4_MX_STEP(S)                                                                  \
  {                                                                                    \
    u32x4 pa[4], pb[4];                                                                \
    _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                    \
      const int row = wx * 128 + 32 * g + r32;                                         \
      pa[g] = ld16(la + row * kKTB + (((4 * h + (S)) ^ (row & 7)) << 4));              \
    }                                                                                  \
    _Pragma("unroll") for (int f = 0; f < 4; ++f) {                                    \
      const int row = wy * 128 + 32 * f + r32;                                         \
      pb[f] = ld16(lb + row * kKTB + (((4 * h + (S)) ^ (row & 7)) << 4));              \
    }                                                                                  \
    _Pragma("unroll") for (int f = 0; f < 4; ++f)                                      \
      _Pragma("unroll") for (int g = 0; g < 4; ++g)                                    \
        acc[f][g] = mfma_fp4_32x32x64<S, S>(pb[f], pa[g], acc[f][g], (int)sb_cur[f], (int)sa_cur[g]); \
  }
    Q4_MX_STEP(0)
    Q4_MX_STEP(1)
    Q4_MX_STEP(2)
    Q4_MX_STEP(3)
#undef Q4_MX_STEP
    __syncthreads();
  }

  const int64_t n_base = n0 + wy * 128, m_base = m0 + wx * 128;
  if (R > 0) epilogue_lowrank<R>(acc, n_base, m_base, M, N, t, l2t, lane);
  epilogue_store<OUT_F32>(acc, n_base, m_base, M, N, bias, y, ldy, lane);
}

template <int R, bool F32>
static void queue(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                  int64_t M, int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_mx_kernel<R, F32>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, s, ac, as,
                     bc, bs, M, N, K, ep.t, ep.l2t, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n);
}

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K,
                          const EpilogueArgs& ep, hipStream_t s) {
  if (ep.out_f32) {
    if (ep.r == 0) queue<0, true>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, true>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, true>(ac, as, bc, bs, M, N, K, ep, s);
  } else {
    if (ep.r == 0) queue<0, false>(ac, as, bc, bs, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, false>(ac, as, bc, bs, M, N, K, ep, s);
    else queue<32, false>(ac, as, bc, bs, M, N, K, ep, s);
  }
  return hipGetLastError();
}

}  // namespace q4
