// FP8 attention of the DiT block (NVIDIA Technical Blog summary, second optimization
// layer: attention quantized to FP8).  Q, K and V arrive as the QKV projection
// writes them (bf16, token-major, head h in columns h*128 .. +128) and are
// quantized to MXFP8 (E4M3 elements, one E8M0 scale per 32): Q and K along
// head_dim, V along the keys, transposed.  The attention kernel then runs both
// products on the block-scaled MFMA: per query, base-2 logits t = c log2(e) s, the
// probabilities 2**(t - M) for an integer shift M at or above the logits, MXFP8
// along the keys per 32-key chunk (P^), and O = P^ V^ / sum P^.  Because MX
// quantization commutes with powers of two, any such M gives the same P^ up to
// 2**M, so the kernel walks the keys in blocks of 64 with a running integer M and
// folds the shift between blocks into the E8M0 scales it hands the MFMA: no
// rescaling of O between blocks.
//
// Layouts (bytes):
//   Q, K codes [tokens, heads*128], scales [tokens, heads*4] (the MXFP8 row layout);
//   V codes [batch, heads*128, seq64] (row h*128+d: channel d of head h over the
//   keys, zero past seq; seq64 = seq rounded up to 64), V scales
//   [batch, heads, seq64/64, 256]: for key block kb, byte c*128 + (d%32)*4 + d/32
//   holds the E8M0 scale of channel d over keys 64 kb + 32 c .. +31.
//
// Kernel: a workgroup of 4 waves takes 128 queries of one (batch, head); each
// wave 32 queries.  Per key block each wave computes S^T = K Q^T as two 32 x 32
// tiles (A = K rows, B = Q rows, K-dim = head_dim in two steps of 64), so a lane
// owns one query and 32 of the block's keys: the row maximum needs one exchange
// between the lane halves.  MFMA row i of score tile t holds key
// 32 t + 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3), which puts in lane half h the
// keys 16 h .. 16 h + 15 (tile 0) and 32 + 16 h .. (tile 1): exactly the bytes the
// 8-bit MFMA wants in lane half h of its B operand for a 64-element K step.  So the
// probabilities, encoded to E4M3 in place, are the B operand of O^T = V^T P^T with
// no trip through LDS; lane half h supplies the scale of key chunk h (= tile h).
// The sum of P^ comes from one more MFMA against a tile of ones.  K blocks (64 keys
// x 128 bytes) and V^T blocks (128 channels x 64 bytes) are loaded straight into
// two LDS stages, 16-byte chunks XOR-swizzled per row so the fragment reads spread
// over the 64 banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

namespace {

constexpr int kHD = 128;                     // head_dim
constexpr int kKB = 64;                      // keys per block
constexpr int kAWaves = 4;
constexpr int kAThreads = 64 * kAWaves;
constexpr int kQW = 32;                      // queries per wave
constexpr int kQB = kQW * kAWaves;           // queries per workgroup
constexpr int kKBytes = kKB * kHD;           // K codes of a block
constexpr int kVBytes = kHD * kKB;           // V^T codes of a block
constexpr int kKsOff = kKBytes + kVBytes;    // K scale dwords (64 keys)
constexpr int kVsOff = kKsOff + 256;         // V scale bytes (256)
constexpr int kStage = kVsOff + 256;
constexpr int kAttnLds = 2 * kStage;
constexpr int kFmtE4M3 = 0;                  // f8f6f4 operand code for E4M3

// chunk swizzles of the K rows (128 bytes, 8 chunks) and V^T rows (64 bytes, 4
// chunks): chunk c of row r sits at position c ^ swz(r)
__device__ __forceinline__ int swz_k(int key) { return ((key >> 1) & 3) | (((key >> 4) & 1) << 2); }
__device__ __forceinline__ int swz_v(int d) { return (d >> 2) & 3; }
// the key of the block held by MFMA row i of score tile t
__device__ __forceinline__ int tile_key(int t, int i) {
  return 32 * t + 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

// max of x over the lane pair (l, l ^ 32).  The swap leaves x of one lane of the
// pair in each of its two results, so their max is the pair's.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// E8M0 exponent of a block whose largest magnitude is pmax (fp32, >= 0), for E4M3
// elements: floor(log2 pmax) - 8 clamped to [-127, 127]; -127 for 0 (and for
// fp32 subnormals, whose probabilities are below 2**-126).
__device__ __forceinline__ int mx8_exponent(float pmax) {
  const int ef = (int)((__float_as_uint(pmax) >> 23) & 0xFF);
  if (ef == 0) return -127;
  const int E = ef - 127 - 8;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

struct AttnView {
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  int seq, heads, seq64, nqb, total, per_xcd;
  float c2;              // softmax scale * log2(e)
  uint16_t* out;
  int64_t ldo;
};

__global__ __launch_bounds__(kAThreads, 2) void attn_fp8_kernel(AttnView a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kAttnLds];
  // consecutive work units (query blocks of one head) on one XCD share its L2
  const int w = blockIdx.x;
  const int unit = (w & 7) * a.per_xcd + (w >> 3);
  if (unit >= a.total) return;
  const int bh = unit / a.nqb, qb = unit % a.nqb;
  const int b = bh / a.heads, hd = bh % a.heads;
  const int q0 = qb * kQB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const uint32_t row_b = (uint32_t)a.heads * kHD;      // code bytes per token
  const uint32_t srow = (uint32_t)a.heads * 4;         // scale bytes per token
  const int64_t tok0 = (int64_t)b * a.seq;

  // buffer views: rows past the sequence (of this batch item) read as zero
  const int qrows = min(kQB, a.seq - q0);
  const auto rq = make_rsrc(a.qc + (tok0 + q0) * row_b + hd * kHD, (uint32_t)qrows * row_b - hd * kHD);
  const auto rqs = make_rsrc(a.qs + (tok0 + q0) * srow + hd * 4, (uint32_t)qrows * srow - hd * 4);
  const auto rk = make_rsrc(a.kc + tok0 * row_b + hd * kHD, (uint32_t)a.seq * row_b - hd * kHD);
  const auto rks = make_rsrc(a.ks + tok0 * srow + hd * 4, (uint32_t)a.seq * srow - hd * 4);
  const auto rv = make_rsrc(a.vc + (int64_t)bh * kHD * a.seq64, (uint32_t)kHD * a.seq64);
  const auto rvs = make_rsrc(a.vs + (int64_t)bh * (a.seq64 / kKB) * 256, (uint32_t)(a.seq64 / kKB) * 256);
  const int nkb = a.seq64 / kKB;

  // the loads of key block kb into stage st: wave w moves K rows 16w .. 16w+15 and
  // V^T rows 32w .. 32w+31; wave 0 the K scales, wave 1 the V scales
  auto load_block = [&](int kb, int st) {
    uint8_t* base = lds + st * kStage;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * wave + jj;
      const int r = 8 * j + (lane >> 3), p = lane & 7;
      dma_ld16(rk, base + 8 * j * 128, (uint32_t)(kb * kKB + r) * row_b + ((p ^ swz_k(r)) << 4));
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * wave + jj;
      const int d = 16 * j + (lane >> 2), p = lane & 3;
      dma_ld16(rv, base + kKBytes + 16 * j * 64, (uint32_t)d * a.seq64 + kb * kKB + ((p ^ swz_v(d)) << 4));
    }
    if (wave == 0) dma_ld4(rks, base + kKsOff, (uint32_t)(kb * kKB + lane) * srow);
    if (wave == 1) dma_ld4(rvs, base + kVsOff, (uint32_t)kb * 256 + 4 * lane);
  };

  load_block(0, 0);
  // this lane's query (row i of the wave's 32): its two 64-element head_dim steps,
  // lane half h holding chunks 4s + h and 4s + 2 + h, and its scale dword shifted so
  // that byte 2s is the scale of head_dim block 2s + h
  const uint32_t qrow = (uint32_t)(kQW * wave + i);
  v8i qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const u32x4 lo = buf_ld16(rq, qrow * row_b + ((4 * s + h) << 4));
    const u32x4 hi = buf_ld16(rq, qrow * row_b + ((4 * s + 2 + h) << 4));
    qf[s] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  const uint32_t qsc = buf_ld4(rqs, qrow * srow) >> (8 * h);

  // per-lane LDS offsets: K fragment chunks (rows of tile 1 are 32 keys = 4096
  // bytes further, with the same swizzle), V^T fragment chunks (d-tiles 2048 bytes
  // apart, same swizzle), the K scale dword of the lane's key, the V scale dword
  const int key0 = tile_key(0, i);
  uint32_t koff[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) koff[s][hf] = key0 * 128 + (((4 * s + 2 * hf + h) ^ swz_k(key0)) << 4);
  uint32_t voff[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) voff[hf] = kKBytes + i * 64 + (((2 * hf + h) ^ swz_v(i)) << 4);

  // O^T and l = sum of the quantized probabilities, both relative to 2**mref: the
  // exponent shift of the first block (kept until a far larger maximum comes)
  v16f o[4], lt = v16f{};
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = v16f{};
  float mcur = -__builtin_inff(), mref = -__builtin_inff();
  const int rem = a.seq - (nkb - 1) * kKB;          // keys of the last block
  // the A operand of the l tile: every element E4M3 1.0 (0x38), scale 2**0
  const v8i ones = v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                       0x38383838, 0x38383838, 0x38383838, 0x38383838};

  auto block = [&](int kb, auto mask_c) {
    constexpr bool kMask = decltype(mask_c)::value;
    const int st = kb & 1;
    // block kb has landed (this wave's part), and every wave is done with block kb-1
    wait_vmem();
    barrier_after_wait();
    if (kb + 1 < nkb) load_block(kb + 1, st ^ 1);
    const uint8_t* sb = lds + st * kStage;

    // ---- scores: S^T tiles t = 0, 1 (rows: keys, columns: the wave's queries)
    const uint32_t ks0 = *reinterpret_cast<const uint32_t*>(sb + kKsOff + 4 * key0) >> (8 * h);
    const uint32_t ks1 = *reinterpret_cast<const uint32_t*>(sb + kKsOff + 4 * (key0 + 32)) >> (8 * h);
    v16f s0 = v16f{}, s1 = v16f{};
    // head_dim step S (0, 1): the scale bytes 2S of the shifted dwords
#define Q4_ATTN_SCORE_STEP(S)                                                                                  \
    {                                                                                                          \
      const u32x4 a0 = ld16(sb + koff[S][0]), a1 = ld16(sb + koff[S][1]);                                      \
      const u32x4 b0 = ld16(sb + 4096 + koff[S][0]), b1 = ld16(sb + 4096 + koff[S][1]);                        \
      const v8i k0 = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]}; \
      const v8i k1 = v8i{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]}; \
      s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k0, qf[S], s0, kFmtE4M3, kFmtE4M3, 2 * S, (int)ks0,  \
                                                           2 * S, (int)qsc);                                   \
      s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k1, qf[S], s1, kFmtE4M3, kFmtE4M3, 2 * S, (int)ks1,  \
                                                           2 * S, (int)qsc);                                   \
    }
    Q4_ATTN_SCORE_STEP(0)
    Q4_ATTN_SCORE_STEP(1)
#undef Q4_ATTN_SCORE_STEP
    // The softmax below runs at raised issue priority: of the two waves sharing a
    // SIMD, the one in its VALU phase then issues first and the other's MFMAs fill
    // in behind it (measured 4-5% faster than equal priority; raising it around the
    // MFMA phases instead made no difference).
    __builtin_amdgcn_s_setprio(1);

    // ---- probabilities.  Element k of tile t is key 32 t + 16 h + k of the block;
    // tile t is 32-key chunk t.  Keys past the sequence (last block only) get -inf.
    if constexpr (kMask) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (16 * h + k >= rem) s0[k] = -__builtin_inff();
        if (32 + 16 * h + k >= rem) s1[k] = -__builtin_inff();
      }
    }
    float mx0 = s0[0], mx1 = s1[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) {
      mx0 = fmaxf(mx0, s0[k]);
      mx1 = fmaxf(mx1, s1[k]);
    }
    mx0 = pair_max(mx0);
    mx1 = pair_max(mx1);
    // the integer exponent shift M >= the base-2 logits seen so far (any integer
    // gives the same quantized weights up to a power of two, which the MFMA's
    // scale absorbs)
    mcur = fmaxf(mcur, __builtin_ceilf(fmaxf(mx0, mx1) * a.c2));
    if (mref == -__builtin_inff()) mref = mcur;
    if (__builtin_amdgcn_ballot_w64(mcur - mref > 100.0f)) {
      // keep the scale bytes below 255: move O and l to the new shift (exactly).
      // Rare: the empty asm keeps it a branch, not multiplies on every block.
      asm volatile("" ::: "memory");
      const float f = mcur - mref > 100.0f ? exp2i((int)(mref - mcur)) : 1.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[dt][k] *= f;
#pragma unroll
      for (int k = 0; k < 16; ++k) lt[k] *= f;
      mref = mcur - mref > 100.0f ? mcur : mref;
    }
    // the chunks' E8M0 exponents from their largest probabilities, and the codes:
    // p * 2**-E = 2**(c2 s - (M + E)) (M + E is an integer: one rounding, in the fma)
    const int e0 = mx8_exponent(__builtin_amdgcn_exp2f(__builtin_fmaf(mx0, a.c2, -mcur)));
    const int e1 = mx8_exponent(__builtin_amdgcn_exp2f(__builtin_fmaf(mx1, a.c2, -mcur)));
    const float sh0 = -(mcur + (float)e0), sh1 = -(mcur + (float)e1);
    uint32_t pw[8];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      float v0[4], v1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v0[j] = fminf(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[4 * wd + j], a.c2, sh0)), 448.0f);
        v1[j] = fminf(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[4 * wd + j], a.c2, sh1)), 448.0f);
      }
      int x0 = __builtin_amdgcn_cvt_pk_fp8_f32(v0[0], v0[1], 0, false);
      x0 = __builtin_amdgcn_cvt_pk_fp8_f32(v0[2], v0[3], x0, true);
      int x1 = __builtin_amdgcn_cvt_pk_fp8_f32(v1[0], v1[1], 0, false);
      x1 = __builtin_amdgcn_cvt_pk_fp8_f32(v1[2], v1[3], x1, true);
      pw[wd] = (uint32_t)x0;
      pw[4 + wd] = (uint32_t)x1;
    }
    const v8i pf = v8i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    // lane half h supplies the scale of chunk h, relative to 2**mref
    const int psc = (h ? e1 : e0) + (int)(mcur - mref) + 127;

    __builtin_amdgcn_s_setprio(0);
    // ---- O^T += V^T P^T (four 32-channel tiles) and l += sum P^ (the ones tile)
    const uint32_t vsc = *reinterpret_cast<const uint32_t*>(sb + kVsOff + 4 * (32 * h + i));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const u32x4 a0 = ld16(sb + voff[0] + dt * 2048), a1 = ld16(sb + voff[1] + dt * 2048);
      const v8i vf = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      switch (dt) {   // the byte of the scale dword is an immediate
        case 0: o[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[0], kFmtE4M3, kFmtE4M3, 0, (int)vsc, 0, psc); break;
        case 1: o[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[1], kFmtE4M3, kFmtE4M3, 1, (int)vsc, 0, psc); break;
        case 2: o[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[2], kFmtE4M3, kFmtE4M3, 2, (int)vsc, 0, psc); break;
        default: o[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, o[3], kFmtE4M3, kFmtE4M3, 3, (int)vsc, 0, psc); break;
      }
    }
    lt = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lt, kFmtE4M3, kFmtE4M3, 0, 127, 0, psc);
  };

  for (int kb = 0; kb + 1 < nkb; ++kb) block(kb, std::false_type{});
  if (rem < kKB) block(nkb - 1, std::true_type{});
  else block(nkb - 1, std::false_type{});

  // ---- O / l in bf16: lane (i, h) holds channels 32 dt + 8 q + 4 h + r of query i
  const int query = q0 + kQW * wave + i;
  if (query >= a.seq) return;
  const float inv = 1.0f / lt[0];
  uint16_t* dst = a.out + (tok0 + query) * a.ldo + hd * kHD;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = f32_to_bf16_rne(o[dt][4 * q] * inv) | (f32_to_bf16_rne(o[dt][4 * q + 1] * inv) << 16);
      const uint32_t hi = f32_to_bf16_rne(o[dt][4 * q + 2] * inv) | (f32_to_bf16_rne(o[dt][4 * q + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * q + 4 * h) = make_uint2(lo, hi);
    }
}

// V [tokens, ldv] bf16 -> V^T MXFP8 codes and scales in the layouts above.  A
// workgroup takes 4 chunks of 32 keys of one (batch, head); wave w chunk w; lane
// channels 2 lane, 2 lane + 1 (one dword per key: 256 contiguous bytes per key
// row across the wave).
__device__ __forceinline__ void quant_v_group(int vb, const uint16_t* __restrict__ v, int64_t ldv, int seq,
                                              int heads, int seq64, int groups_per_bh,
                                              uint8_t* __restrict__ vc, uint8_t* __restrict__ vs) {
  const int g = vb % groups_per_bh, bh = vb / groups_per_bh;
  const int b = bh / heads, hd = bh % heads;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = 4 * g + wave;                    // 32-key chunk of this (b, head)
  if (chunk * 32 >= seq64) return;
  const uint16_t* src = v + ((int64_t)b * seq + chunk * 32) * ldv + hd * kHD + 2 * lane;
  uint32_t w[32];
#pragma unroll
  for (int r = 0; r < 32; ++r)
    w[r] = (chunk * 32 + r < seq) ? *reinterpret_cast<const uint32_t*>(src + (int64_t)r * ldv) : 0u;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int d = 2 * lane + half;
    uint32_t amax = 0;
#pragma unroll
    for (int r = 0; r < 32; ++r) amax = max(amax, (half ? (w[r] >> 16) : w[r]) & 0x7FFFu);
    int E = amax == 0 ? -127 : bf16_floor_log2(amax) - 8;
    E = E < -127 ? -127 : (E > 127 ? 127 : E);
    const float down = exp2i(-E);
    uint32_t out[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wd = w[4 * q + j];
        x[j] = fminf(fmaxf((half ? bf16_hi(wd) : bf16_lo(wd)) * down, -448.0f), 448.0f);
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], word, true);
      out[q] = (uint32_t)word;
    }
    uint8_t* dst = vc + ((int64_t)bh * kHD + d) * seq64 + chunk * 32;
    st16(dst, u32x4{out[0], out[1], out[2], out[3]});
    st16(dst + 16, u32x4{out[4], out[5], out[6], out[7]});
    vs[((int64_t)bh * (seq64 / kKB) + chunk / 2) * 256 + (chunk & 1) * 128 + (d & 31) * 4 + (d >> 5)] =
        (uint8_t)(E + 127);
  }
}

// The three quantizations in one launch: workgroups [0, nqk) take Q's and then K's
// 32-element row blocks, one per thread (mx_block), the rest V's groups of 32-key
// chunks (quant_v_group).  One launch instead of three saves two launch gaps and
// two tails.
__global__ __launch_bounds__(256) void attn_quant_kernel(const uint16_t* __restrict__ q, int64_t ldq,
                                                         const uint16_t* __restrict__ k, int64_t ldk,
                                                         const uint16_t* __restrict__ v, int64_t ldv,
                                                         int64_t tokens, int64_t width, int seq, int heads,
                                                         int seq64, int groups, int nqk, uint8_t* __restrict__ qc,
                                                         uint8_t* __restrict__ qs, uint8_t* __restrict__ kc,
                                                         uint8_t* __restrict__ ks, uint8_t* __restrict__ vc,
                                                         uint8_t* __restrict__ vs) {
  if ((int)blockIdx.x >= nqk) {
    quant_v_group((int)blockIdx.x - nqk, v, ldv, seq, heads, seq64, groups, vc, vs);
    return;
  }
  const int64_t nblk = width >> 5, work = tokens * nblk;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < work) mx_block<kBlkMXFP8>(q, width, ldq, 1, qc, qs, nblk, i);
  else if (i < 2 * work) mx_block<kBlkMXFP8>(k, width, ldk, 1, kc, ks, nblk, i - work);
}

}  // namespace

hipError_t launch_attn_quantize(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk,
                                const uint16_t* v, int64_t ldv, int64_t batch, int64_t seq, int64_t heads,
                                uint8_t* qc, uint8_t* qs, uint8_t* kc, uint8_t* ks, uint8_t* vc,
                                uint8_t* vs, hipStream_t s) {
  const int64_t tokens = batch * seq, width = heads * kHD;
  const int64_t seq64 = (seq + kKB - 1) / kKB * kKB;
  const int64_t groups = (seq64 / 32 + 3) / 4;
  const int64_t nqk = (2 * tokens * (width >> 5) + 255) / 256;       // Q and K blocks, 256 per workgroup
  const int64_t grid = nqk + batch * heads * groups;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s, q, ldq, k, ldk, v, ldv, tokens, width,
                     (int)seq, (int)heads, (int)seq64, (int)groups, (int)nqk, qc, qs, kc, ks, vc, vs);
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                           const uint8_t* vc, const uint8_t* vs, int64_t batch, int64_t seq, int64_t heads,
                           float softmax_scale, uint16_t* out, int64_t ldo, hipStream_t s) {
  AttnView a;
  a.qc = qc; a.qs = qs; a.kc = kc; a.ks = ks; a.vc = vc; a.vs = vs;
  a.seq = (int)seq;
  a.heads = (int)heads;
  a.seq64 = (int)((seq + kKB - 1) / kKB * kKB);
  a.nqb = (int)((seq + kQB - 1) / kQB);
  a.total = (int)(batch * heads * a.nqb);
  a.per_xcd = (a.total + 7) / 8;
  a.c2 = (float)((double)softmax_scale * 1.4426950408889634);
  a.out = out;
  a.ldo = ldo;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3((unsigned)(8 * a.per_xcd)), dim3(kAThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace q4
