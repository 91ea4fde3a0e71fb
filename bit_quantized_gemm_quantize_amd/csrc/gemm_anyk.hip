// The W4A4 GEMM for any K the block formats allow: MXFP4 with K a multiple of 32,
// NVFP4 with K a multiple of 16.  The tiled kernels step K in units of 128 or more
// (their scale loads are aligned words of 4 or 16 scale bytes); this one serves the
// other K, with the same arithmetic, the same epilogue and the same tolerance.
//
// Tiling: 256 x 128 output tile per workgroup of 4 waves; wave (wm, wn) owns
// m in [128 wm, +128) and n in [64 wn, +64) as 2 x 4 tiles of 32 x 32, the
// accumulators laid out as in the tiled kernels (MFMA A operand = weight rows, B
// operand = activation rows).  Operands go straight from global memory into the
// registers of the MFMA layout, one K step ahead; rows past M or N and blocks past K
// read as zero through the buffer range checks.
//   MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 per 64 K elements; lane half h takes
//   block 2 s + h of step s with its E8M0 byte.
//   NVFP4: each 16-element block is dequantized exactly to bf16 (as in gemm_nv) and
//   multiplied on v_mfma_f32_32x32x16_bf16; the fp32 tensor scales multiply the
//   4-bit product in the epilogue, before the low-rank term.
#include "q4_epilogue.h"

namespace q4 {

constexpr int kAkBM = 256, kAkBN = 128, kAkF = 2;

template <int FMT, int R, bool OUT_F32>
__global__ __launch_bounds__(256) void gemm_anyk_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ t, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, void* __restrict__ y, int64_t ldy) {
  using S = EpilogueShape<OUT_F32, kAkF, 128>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * S::kStageWaveBytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t m_base = (int64_t)blockIdx.y * kAkBM + 128 * wm;
  const int64_t n_base = (int64_t)blockIdx.x * kAkBN + 64 * wn;
  const uint32_t kb = (uint32_t)(K >> 1);
  const uint32_t sbytes = (uint32_t)(FMT == 0 ? K >> 5 : K >> 4);   // scale bytes per row
  const uint32_t ra_rows = rows_in(128, M, m_base), rb_rows = rows_in(64, N, n_base);
  const auto rca = make_rsrc(ac + m_base * kb, ra_rows * kb);
  const auto rsa = make_rsrc(as + m_base * sbytes, ra_rows * sbytes);
  const auto rcb = make_rsrc(bc + n_base * kb, rb_rows * kb);
  const auto rsb = make_rsrc(bs + n_base * sbytes, rb_rows * sbytes);

  v16f acc[kAkF][4];
#pragma unroll
  for (int f = 0; f < kAkF; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[f][g] = v16f{};

  if constexpr (FMT == 0) {
    // step s: lane half h holds block 2 s + h (16 code bytes, one scale byte)
    const uint32_t nblk = sbytes;
    const int64_t nsteps = (nblk + 1) >> 1;
    struct Ops {
      u32x4 a[4], b[kAkF];
      uint32_t sa[4], sb[kAkF];
    };
    auto load = [&](int64_t s, Ops& o) {
      const uint32_t blk = (uint32_t)(2 * s + h);
      const bool kin = s < nsteps && blk < nblk;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t row = 32 * g + r32;
        o.a[g] = buf_ld16(rca, kin ? row * kb + blk * 16 : kOOB);
        o.sa[g] = __builtin_amdgcn_raw_buffer_load_b8(rsa, (int)(kin ? row * nblk + blk : kOOB), 0, 0);
      }
#pragma unroll
      for (int f = 0; f < kAkF; ++f) {
        const uint32_t row = 32 * f + r32;
        o.b[f] = buf_ld16(rcb, kin ? row * kb + blk * 16 : kOOB);
        o.sb[f] = __builtin_amdgcn_raw_buffer_load_b8(rsb, (int)(kin ? row * nblk + blk : kOOB), 0, 0);
      }
    };
    auto mma = [&](const Ops& o) {
#pragma unroll
      for (int f = 0; f < kAkF; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          acc[f][g] = mfma_fp4_32x32x64<0, 0>(o.b[f], o.a[g], acc[f][g], (int)o.sb[f], (int)o.sa[g]);
    };
    Ops o0, o1;
    load(0, o0);
    for (int64_t s = 0; s < nsteps; s += 2) {
      load(s + 1, o1);
      mma(o0);
      load(s + 2, o0);
      if (s + 1 < nsteps) mma(o1);
    }
  } else {
    // step s (16 K): lane half h holds elements 8 h .. 8 h + 7 of block s (4 code
    // bytes), dequantized with the block's E4M3 scale
    const int64_t nsteps = K >> 4;
    struct Ops {
      uint32_t a[4], b[kAkF], sa[4], sb[kAkF];
    };
    auto load = [&](int64_t s, Ops& o) {
      const bool kin = s < nsteps;
      const uint32_t co = (uint32_t)(8 * s + 4 * h), so = (uint32_t)s;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t row = 32 * g + r32;
        o.a[g] = buf_ld4(rca, kin ? row * kb + co : kOOB);
        o.sa[g] = __builtin_amdgcn_raw_buffer_load_b8(rsa, (int)(kin ? row * sbytes + so : kOOB), 0, 0);
      }
#pragma unroll
      for (int f = 0; f < kAkF; ++f) {
        const uint32_t row = 32 * f + r32;
        o.b[f] = buf_ld4(rcb, kin ? row * kb + co : kOOB);
        o.sb[f] = __builtin_amdgcn_raw_buffer_load_b8(rsb, (int)(kin ? row * sbytes + so : kOOB), 0, 0);
      }
    };
    auto deq = [](uint32_t codes, uint32_t sc) {
      const float s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
      return u32x4{nv_dequant_pair<0>(codes, s), nv_dequant_pair<1>(codes, s), nv_dequant_pair<2>(codes, s),
                   nv_dequant_pair<3>(codes, s)};
    };
    auto mma = [&](const Ops& o) {
      u32x4 a[4], b[kAkF];
#pragma unroll
      for (int g = 0; g < 4; ++g) a[g] = deq(o.a[g], o.sa[g]);
#pragma unroll
      for (int f = 0; f < kAkF; ++f) b[f] = deq(o.b[f], o.sb[f]);
#pragma unroll
      for (int f = 0; f < kAkF; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = mfma_bf16_32x32x16(b[f], a[g], acc[f][g]);
    };
    Ops o0, o1;
    load(0, o0);
    for (int64_t s = 0; s < nsteps; s += 2) {
      load(s + 1, o1);
      mma(o0);
      load(s + 2, o0);
      if (s + 1 < nsteps) mma(o1);
    }
  }

  float scale = 1.0f;
  if constexpr (FMT == 1) {
    // the tensor scales multiply the 4-bit product only, before the low-rank term
    scale = ats[0] * bts[0];
    if (R > 0) {
#pragma unroll
      for (int f = 0; f < kAkF; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[f][g] = acc[f][g] * scale;
      scale = 1.0f;
    }
  }
  if constexpr (R > 0) lowrank_accumulate<R>(acc, n_base, m_base, M, N, t, l2t, lane);
  epilogue_store<OUT_F32, kAkF, 128, FMT == 1>(acc, n_base, m_base, M, N, bias, y, ldy, lane,
                                               lds + wave * S::kStageWaveBytes, scale);
}

template <int FMT, int R, bool F32>
static void queue(const uint8_t* ac, const uint8_t* as, const float* ats, const uint8_t* bc,
                  const uint8_t* bs, const float* bts, int64_t M, int64_t N, int64_t K,
                  const EpilogueArgs& ep, hipStream_t s) {
  const dim3 grid((unsigned)((N + kAkBN - 1) / kAkBN), (unsigned)((M + kAkBM - 1) / kAkBM));
  hipLaunchKernelGGL((gemm_anyk_kernel<FMT, R, F32>), grid, dim3(256), 0, s, ac, as, ats, bc, bs, bts, M, N,
                     K, ep.t, ep.l2t, ep.bias, ep.y, ep.ldy);
}

template <int FMT>
static void queue_fmt(const uint8_t* ac, const uint8_t* as, const float* ats, const uint8_t* bc,
                      const uint8_t* bs, const float* bts, int64_t M, int64_t N, int64_t K,
                      const EpilogueArgs& ep, hipStream_t s) {
  if (ep.out_f32) {
    if (ep.r == 0) queue<FMT, 0, true>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else if (ep.r == 16) queue<FMT, 16, true>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else queue<FMT, 32, true>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
  } else {
    if (ep.r == 0) queue<FMT, 0, false>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else if (ep.r == 16) queue<FMT, 16, false>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
    else queue<FMT, 32, false>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
  }
}

hipError_t launch_gemm_anyk(int fmt, const uint8_t* ac, const uint8_t* as, const float* ats,
                            const uint8_t* bc, const uint8_t* bs, const float* bts, int64_t M,
                            int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s) {
  if (fmt == 0) queue_fmt<0>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
  else queue_fmt<1>(ac, as, ats, bc, bs, bts, M, N, K, ep, s);
  return hipGetLastError();
}

}  // namespace q4
