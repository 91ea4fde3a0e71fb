// NVFP4-style GEMM, exact: every operand value e2m1 * s_b (two significant bits
// times the four of an E4M3 scale) fits bf16 exactly, so each K-tile is dequantized
// to bf16 in LDS and multiplied on the bf16 MFMA; the two fp32 tensor scales
// multiply the fp32 result in the epilogue.  The block-scaled FP4 MFMA cannot take
// this format directly: its scales are powers of two per 32 elements, while an
// NVFP4 block scale carries mantissa bits and covers 16 elements.
#include "gemm_bf16_core.h"

namespace q4 {

// Two E2M1 codes (byte B of a dword) times the block scale -> a bf16 pair.  The
// products are exact bf16 values, so keeping the upper halves is exact; one byte
// permute (bytes 2, 3 of lo, then of hi) packs them.
template <int B>
__device__ __forceinline__ uint32_t nv_dequant_pair(uint32_t codes, float s) {
  const v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, B);
  const uint32_t lo = __float_as_uint(v[0] * s), hi = __float_as_uint(v[1] * s);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// 32 E2M1 codes (one 16-byte chunk) times their two block scales -> 4 chunks of bf16.
__device__ __forceinline__ void nv_dequant_chunk(u32x4 codes, uint32_t sc2, u32x4* out4) {
  const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)(sc2 & 0xFFu), 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)((sc2 >> 8) & 0xFFu), 0);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float s = d < 2 ? s0 : s1;
    out4[d] = u32x4{nv_dequant_pair<0>(codes[d], s), nv_dequant_pair<1>(codes[d], s),
                    nv_dequant_pair<2>(codes[d], s), nv_dequant_pair<3>(codes[d], s)};
  }
}

// Per K-tile (64 K) and operand: 256 (weights: TN) rows x 2 chunks of 32 codes;
// thread tid owns chunk c = tid & 1 of rows tid/2 and tid/2 + 128, with the two
// E4M3 scale bytes of each chunk.  Reads past M / N / K return zeros (buffer range
// checks).
template <int TN>
struct NvLoader {
  static constexpr int kValuPerStore = 192;   // VALU ops of one store part (about)
  static constexpr int kRegLoads = 4 + 2 * (TN / 128);   // VMEM instructions of issue_regs
  static constexpr bool kLateStores = true;   // heavy conversion: see bf16_ktile_late
  __amdgpu_buffer_rsrc_t rca, rsa, rcb, rsb;
  uint32_t kb, sbytes, nchunk;
  int tid;
  u32x4 ca[2], cb[2];
  uint32_t sa[2], sb[2];

  __device__ __forceinline__ void init(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                                       const uint8_t* bs, int64_t M, int64_t N, int64_t K,
                                       int64_t m0, int64_t n0, int t) {
    kb = (uint32_t)(K >> 1); sbytes = (uint32_t)(K >> 4); nchunk = (uint32_t)(K >> 5);
    const uint32_t ra = rows_in(kBf16BM, M, m0), rb = rows_in(TN, N, n0);
    rca = make_rsrc(ac + m0 * kb, ra * kb);
    rcb = make_rsrc(bc + n0 * kb, rb * kb);
    rsa = make_rsrc(as + m0 * sbytes, ra * sbytes);
    rsb = make_rsrc(bs + n0 * sbytes, rb * sbytes);
    tid = t;
  }
  __device__ __forceinline__ void issue_lds(int, uint8_t*, uint8_t*) {}   // all through registers
  __device__ __forceinline__ void issue_regs(int kt) {
    const uint32_t chunk = (uint32_t)kt * 2 + (tid & 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t row = (tid >> 1) + 128 * j;
      const uint32_t co = in_range_or_oob(row * kb + chunk * 16, chunk, nchunk);
      const uint32_t so = in_range_or_oob(row * sbytes + chunk * 2, chunk, nchunk);
      ca[j] = buf_ld16(rca, co);
      sa[j] = __builtin_amdgcn_raw_buffer_load_b16(rsa, (int)so, 0, 0);
      if (j < TN / 128) {
        cb[j] = buf_ld16(rcb, co);
        sb[j] = __builtin_amdgcn_raw_buffer_load_b16(rsb, (int)so, 0, 0);
      }
    }
  }
  // half P: both operands' chunks of row group P
  template <int P>
  __device__ __forceinline__ void store(uint8_t* la, uint8_t* lb) {
    // row (tid >> 1) + 128 P: row & 7 does not depend on P
    const int c = tid & 1, r = tid >> 1;
    const int off = r * kBf16RowBytes + P * 128 * kBf16RowBytes;
    u32x4 o[4];
    nv_dequant_chunk(ca[P], sa[P], o);
#pragma unroll
    for (int d = 0; d < 4; ++d) st16(la + off + (((4 * c + d) ^ (r & 7)) << 4), o[d]);
    if (P < TN / 128) {
      nv_dequant_chunk(cb[P], sb[P], o);
#pragma unroll
      for (int d = 0; d < 4; ++d) st16(lb + off + (((4 * c + d) ^ (r & 7)) << 4), o[d]);
    }
  }
};

// One output tile of 256 activation rows x 64 F weight rows at (m0, n0).
template <int R, bool OUT_F32, int F>
__device__ __forceinline__ void nv_tile(
    uint8_t* lds, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const float* __restrict__ ats, const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
    const float* __restrict__ bts, int64_t M, int64_t N, int64_t K, const float* __restrict__ t,
    const uint16_t* __restrict__ l2t, const uint16_t* __restrict__ bias, void* __restrict__ y,
    int64_t ldy, int64_t m0, int64_t n0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wy = wave >> 1, wx = wave & 1;
  NvLoader<64 * F> ld;
  ld.init(ac, as, bc, bs, M, N, K, m0, n0, tid);
  v16f acc[F][4];
  bf16_mainloop(acc, ld, K, lds, wx, wy, lane);

  // the tensor scales multiply the 4-bit product only, before the low-rank term
  const float scale = ats[0] * bts[0];
  const int64_t n_base = n0 + wy * 32 * F, m_base = m0 + wx * 128;
  if (R > 0) {
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[f][g] = acc[f][g] * scale;
    lowrank_accumulate<R>(acc, n_base, m_base, M, N, t, l2t, lane);
  }
  __syncthreads();                           // all waves are done reading operand tiles
  epilogue_store<OUT_F32, F, 128, true>(acc, n_base, m_base, M, N, bias, y, ldy, lane,
                                        lds + wave * EpilogueShape<OUT_F32, F, 128>::kStageWaveBytes,
                                        R > 0 ? 1.0f : scale);
}

// Whole 256 x 256 tiles and halves (256 x 128) of the leftover ones: see tile_unit.
template <int R, bool OUT_F32>
__global__ __launch_bounds__(kBf16Threads, 1) void gemm_nv_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ t, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy, int tiles_m, int tiles_n,
    int full) {
  static_assert(kEpilogueLdsBytes <= kBf16MainLds, "the epilogue stages its output in the operand LDS");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBf16MainLds];
  int vt, half, tm, tn;
  const bool is_half = tile_unit(blockIdx.x, tiles_m * tiles_n, full, &vt, &half);
  tile_of(vt, tiles_m, tiles_n, kBf16GroupM, &tm, &tn);
  if (!is_half) {
    nv_tile<R, OUT_F32, 4>(lds, ac, as, ats, bc, bs, bts, M, N, K, t, l2t, bias, y, ldy,
                           (int64_t)tm * kBf16BM, (int64_t)tn * kBf16BN);
  } else {
    if ((int64_t)tn * 256 + 128 * half >= N) return;       // half past the last weight row
    nv_tile<R, OUT_F32, 2>(lds, ac, as, ats, bc, bs, bts, M, N, K, t, l2t, bias, y, ldy,
                           (int64_t)tm * kBf16BM, (int64_t)tn * kBf16BN + 128 * half);
  }
}

template <int R, bool F32>
static void queue(const uint8_t* ac, const uint8_t* as, const float* ats, const uint8_t* bc,
                  const uint8_t* bs, const float* bts, int64_t M, int64_t N, int64_t K,
                  const EpilogueArgs& ep, hipStream_t s) {
  const int tiles_m = (int)((M + kBf16BM - 1) / kBf16BM), tiles_n = (int)((N + kBf16BN - 1) / kBf16BN);
  int full, grid;
  bf16_tile_split(tiles_m * tiles_n, &full, &grid);
  hipLaunchKernelGGL((gemm_nv_kernel<R, F32>), dim3(grid), dim3(kBf16Threads), 0, s, ac, as, ats, bc,
                     bs, bts, M, N, K, ep.t, ep.l2t, ep.bias, ep.y, ep.ldy, tiles_m, tiles_n, full);
}

hipError_t launch_gemm_nv(const uint8_t* ac, const uint8_t* as, const float* ats,
                          const uint8_t* bc, const uint8_t* bs, const float* bts, int64_t M,
                          int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  if (ep.out_f32) {
    if (ep.r == 0) queue<0, true>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, true>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else queue<32, true>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
  } else {
    if (ep.r == 0) queue<0, false>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else if (ep.r == 16) queue<16, false>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else queue<32, false>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
  }
  return hipGetLastError();
}

}  // namespace q4
