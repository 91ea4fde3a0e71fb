// MXFP8 x MXFP8 GEMM (E4M3 elements, one E8M0 scale per 32 K elements per row) on
// the same CDNA4 block-scaled MFMA as the MXFP4 GEMM, with format code 0 (FP8
// E4M3) on both operands: the 8-bit member of the OCP MX family the pages set
// beside MXFP4 ("Quantization for the impatient", formats table).  One
// v_mfma_scale_f32_32x32x64_f8f6f4 takes twice the cycles of its FP4 form, and
// each operand is twice the bytes, so this GEMM has half the FP4 peak.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves, wave (wm, wn) owning
// 128 x 128 as 4 x 4 MFMA tiles with fp32 accumulators in the matrix registers.
// K advances in tiles of 128 elements (128 bytes per row, 4 scale bytes per row),
// loaded straight into two LDS stages with the 16-byte chunks XOR-swizzled by row
// (chunk c of row r at c ^ lds_swz<8>(r), for the 64-bank LDS).  An MFMA step consumes 64 K elements, and
// with 8-bit operands the instruction splits each 32-element block over the two
// lane halves (measured on gfx950: lane half h holds K [16h, 16h+16) of the step
// in its first 16 bytes and K [32+16h, 32+16h+16) in its last 16, and block b is
// scaled by the scale operand of lane half b).  So in step s lane half h reads
// chunks 4s + h and 4s + 2 + h and supplies the scale of block 2s + h: its scale
// dword for the K-tile (blocks 0..3 of the tile for its row) is shifted right by
// 8 h, so byte 2s of it is that scale, and op_sel 2s picks it.
//
// Tail: as in the MXFP4 GEMM, the tiles that do not fill a last round over the CUs
// run as two halves of 128 weight rows each (wave tiles 128 x 64), dispatched first.
#include <type_traits>

#include "q4_epilogue.h"

namespace q4 {

namespace {

constexpr int kX8BM = 256, kX8BN = 256, kX8KT = 128, kX8KTB = kX8KT;
constexpr int kX8Waves = 4, kX8Threads = 64 * kX8Waves;
constexpr int kX8Lds = 2 * 2 * kX8BM * kX8KTB;                      // [operand][stage]
constexpr int kFmtFP8 = 0;                                          // f8f6f4 operand code for E4M3
static_assert(kX8Waves * EpilogueShape<true, 4, 128>::kStageWaveBytes <= kX8Lds &&
                  kX8Waves * EpilogueShape<false, 4, 128>::kStageWaveBytes <= kX8Lds,
              "the epilogue stages each wave's output in the operand LDS");

// The MFMAs of step S (0 or 1) of a K-tile: the weight fragment is the MFMA's first
// operand, so accumulator register j of lane l holds column n = acc_row(j, l) and
// row m = l % 32 of the 32 x 32 result, the layout the epilogue takes.  F weight
// sub-tiles of 32 rows per wave: 4 in a whole tile, 2 in a half.
template <int S, int F>
__device__ __forceinline__ void mx8_step(v16f (&acc)[F][4], const v8i (&a)[4], const v8i (&b)[F],
                                         const uint32_t (&sa)[4], const uint32_t (&sb)[F]) {
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      acc[f][g] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[f], a[g], acc[f][g], kFmtFP8, kFmtFP8,
                                                                  2 * S, (int)sb[f], 2 * S, (int)sa[g]);
}

// One output tile: 256 activation rows x 64 F weight rows at (m0, n0).
template <bool OUT_F32, int F>
__device__ __forceinline__ void mx8_tile(
    uint8_t* lds_raw, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, int64_t M, int64_t N, int64_t K,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int64_t m0, int64_t n0) {
  constexpr int kTN = 64 * F, kRowsB = kTN / kX8Waves;     // weight rows: per tile, per wave
  auto& lds = *reinterpret_cast<uint8_t(*)[2][2][kX8BM * kX8KTB]>(lds_raw);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave >> 1, wm = wave & 1;
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t kbytes = (uint32_t)K, nblk = (uint32_t)(K >> 5), nchunk = (uint32_t)(K >> 4);
  const int nkt = (int)(K / kX8KT);
  const uint32_t rows_a = rows_in(kX8BM, M, m0), rows_b = rows_in(kTN, N, n0);
  const auto rc_a = make_rsrc(ac + m0 * kbytes, rows_a * kbytes);
  const auto rc_b = make_rsrc(bc + n0 * kbytes, rows_b * kbytes);
  const auto rs_a = make_rsrc(as + m0 * nblk, rows_a * nblk);
  const auto rs_b = make_rsrc(bs + n0 * nblk, rows_b * nblk);

  // K-tile kt -> stage: each wave moves 64 activation and kRowsB weight rows, 8 rows
  // of 128 bytes per instruction (lane i: row i / 8, stored chunk i % 8 holding
  // global chunk (i % 8) ^ lds_swz<8>(row)); rows past the matrix read as zero
  const int lr = lane >> 3, lp = lane & 7;
  auto load_ktile = [&](int kt, int stage) {
    // row = 16 q + 8 (j % 2) + lr: its swizzle lds_swz<8>(row) is 4 (j % 2) + lr / 2
    uint32_t koff[2];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const uint32_t chunk = (uint32_t)kt * 8 + (lp ^ (4 * jp + (lr >> 1)));
      koff[jp] = chunk < nchunk ? chunk * 16 : kOOB;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t row = 64 * wave + 8 * j + lr;
      buf_ld16_lds(rc_a, &lds[0][stage][(64 * wave + 8 * j) * kX8KTB], row * kbytes + koff[j & 1]);
    }
#pragma unroll
    for (int j = 0; j < kRowsB / 8; ++j) {
      const uint32_t row = kRowsB * wave + 8 * j + lr;
      buf_ld16_lds(rc_b, &lds[1][stage][(kRowsB * wave + 8 * j) * kX8KTB], row * kbytes + koff[j & 1]);
    }
  };
  // the lane's scale dwords of K-tile kt (rows past the matrix, and K-tiles past K,
  // read whatever the view holds there or zero: never used)
  auto load_scales = [&](int kt, uint32_t* da, uint32_t* db) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      da[g] = buf_ld4(rs_a, (uint32_t)(wm * 128 + 32 * g + r32) * nblk + 4 * kt);
#pragma unroll
    for (int f = 0; f < F; ++f)
      db[f] = buf_ld4(rs_b, (uint32_t)(wn * 32 * F + 32 * f + r32) * nblk + 4 * kt);
  };
  // fragment registers, double-buffered across MFMA steps
  v8i fa[2][4], fb[2][F];
  auto frag = [&](int op, int stage, int row, int s) {
    const uint8_t* base = &lds[op][stage][row * kX8KTB];
    const int c = 4 * s + h;
    const u32x4 lo = ld16(base + ((c ^ lds_swz<8>(row)) << 4)), hi = ld16(base + (((c + 2) ^ lds_swz<8>(row)) << 4));
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto read_frags = [&](int buf, int stage, int s) {
#pragma unroll
    for (int g = 0; g < 4; ++g) fa[buf][g] = frag(0, stage, wm * 128 + 32 * g + r32, s);
#pragma unroll
    for (int f = 0; f < F; ++f) fb[buf][f] = frag(1, stage, wn * 32 * F + 32 * f + r32, s);
  };

  v16f acc[F][4];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = v16f{};

  // Pipeline: K-tiles kt and kt+1 sit in the two stages; the scale dwords of even
  // and odd K-tiles in two register sets.  In K-tile kt, step 0 runs while the
  // fragments of step 1 are read; then every wave waits for K-tile kt+1 (loaded a
  // whole K-tile earlier) and passes the barrier, which frees stage kt % 2 for the
  // loads of K-tile kt+2; step 1 runs while the fragments of K-tile kt+1's step 0
  // are read.  The scale loads for kt+2 go out after step 1 (issued earlier, they
  // would keep a third register set live through it).  Loads past K read zeros
  // (codes) and are never used.
  uint32_t sx_a[4], sx_b[F], sy_a[4], sy_b[F];
  load_ktile(0, 0);
  load_scales(0, sx_a, sx_b);
  load_ktile(1, 1);
  load_scales(1, sy_a, sy_b);
  wait_vmem();
  __syncthreads();
  read_frags(0, 0, 0);
  auto ktile = [&](auto stage_c, int kt, uint32_t* sr_a, uint32_t* sr_b) {
    constexpr int st = decltype(stage_c)::value;
    // step 0's fragments were read during the last K-tile's step 1: waiting for them
    // here keeps the 16 reads below from counting against them (the LDS counter
    // holds at most 15)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    uint32_t ca[4], cb[F];
#pragma unroll
    for (int i = 0; i < 4; ++i) ca[i] = sr_a[i] >> (8 * h);
#pragma unroll
    for (int i = 0; i < F; ++i) cb[i] = sr_b[i] >> (8 * h);
    read_frags(1, st, 1);
    mx8_step<0, F>(acc, fa[0], fb[0], ca, cb);
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 2 * F, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * F, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem();                                 // K-tile kt+1 and its scales have landed
    __syncthreads();                             // and every read of stage st is done
    load_ktile(kt + 2, st);
    read_frags(0, st ^ 1, 0);
    mx8_step<1, F>(acc, fa[1], fb[1], ca, cb);
    __builtin_amdgcn_sched_group_barrier(0x020, 8 + F, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 2 * F, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * F, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_scales(kt + 2, sr_a, sr_b);
  };
  int kt = 0;
  for (; kt + 1 < nkt; kt += 2) {
    ktile(std::integral_constant<int, 0>{}, kt, sx_a, sx_b);
    ktile(std::integral_constant<int, 1>{}, kt + 1, sy_a, sy_b);
  }
  if (kt < nkt) ktile(std::integral_constant<int, 0>{}, kt, sx_a, sx_b);
  wait_vmem();                                   // the loads past K have landed
  __syncthreads();                               // before the epilogue reuses the LDS

  const int64_t n_base = n0 + wn * 32 * F, m_base = m0 + wm * 128;
  epilogue_store<OUT_F32, F, 128>(acc, n_base, m_base, M, N, bias, y, ldy, lane,
                                  lds_raw + wave * EpilogueShape<OUT_F32, F, 128>::kStageWaveBytes);
}

// Workgroup b -> a whole tile or, for b < 2 (tiles - full), a half of a leftover
// tile (weight rows 128 h .. +127), with the XCD-aware order of tile_of.
template <bool OUT_F32>
__global__ __launch_bounds__(kX8Threads) void gemm_mx8_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ bias,
    void* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n, int full) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kX8Lds];
  int vt, half, tm, tn;
  const bool is_half = tile_unit(blockIdx.x, tiles_m * tiles_n, full, &vt, &half);
  tile_of(vt, tiles_m, tiles_n, 4, &tm, &tn);
  const int64_t m0 = (int64_t)tm * kX8BM, n0 = (int64_t)tn * kX8BN + (is_half ? 128 * half : 0);
  if (n0 >= N) return;                                   // a half past the last weight row
  if (is_half)
    mx8_tile<OUT_F32, 2>(lds_raw, ac, as, bc, bs, M, N, K, bias, y, ldy, m0, n0);
  else
    mx8_tile<OUT_F32, 4>(lds_raw, ac, as, bc, bs, M, N, K, bias, y, ldy, m0, n0);
}

}  // namespace

hipError_t launch_gemm_mx8(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                           int64_t M, int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kX8BM - 1) / kX8BM), tiles_n = (int)((N + kX8BN - 1) / kX8BN);
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
    hipLaunchKernelGGL((gemm_mx8_kernel<true>), dim3(grid), dim3(kX8Threads), 0, s, ac, as, bc, bs, M, N, K,
                       ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
  else
    hipLaunchKernelGGL((gemm_mx8_kernel<false>), dim3(grid), dim3(kX8Threads), 0, s, ac, as, bc, bs, M, N, K,
                       ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
  return hipGetLastError();
}

}  // namespace q4
