// Host-side launchers behind the C ABI (internal to libq4lin).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// Words of device scratch the NVFP4 tensor-amax launch needs (its partial maxima).
constexpr int kNvScratchWords = 1024;

// Activation quantizer (+ t = X L1 when r > 0).  fmt 0 = MXFP4, 1 = NVFP4.
// NVFP4 queues the tensor-amax launch (partial maxima into nv_scratch, at least
// kNvScratchWords words) and the encode launch; nv_scratch is unused otherwise.
// inv_s (MXFP4, r > 0 only): the smoothing factors' reciprocals.
hipError_t launch_quantize_act(int fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               const uint16_t* l1t, int r, float* t, hipStream_t s,
                               uint32_t* nv_scratch, const float* inv_s = nullptr);

// Weight packer over a strided logical [K, N] bf16 matrix.  fmt 0/1/2 (NVFP4 uses
// nv_scratch as launch_quantize_act does).
hipError_t launch_pack_weights(int fmt, const uint16_t* w, int64_t K, int64_t N, int64_t sk,
                               int64_t sn, uint8_t* codes, void* scales, uint16_t* zeros,
                               float* tensor_scale, hipStream_t s, uint32_t* nv_scratch);

struct EpilogueArgs {
  const float* t;         // [M, r] fp32 or nullptr
  const uint16_t* l2t;    // [N, r] bf16 or nullptr
  int r;                  // 0, 16, 32
  const uint16_t* bias;   // [N] bf16 or nullptr
  void* y;
  int64_t ldy;
  int out_f32;            // 0: bf16, 1: fp32
  // MXFP4 output for the next layer (MXFP4 GEMM only): codes [M, N/2] and scale
  // bytes [M, N/32], row strides in bytes; qc == nullptr: none (y is then required)
  uint8_t* qc = nullptr;
  int64_t ldc = 0;
  uint8_t* qs = nullptr;
  int64_t lds = 0;
  // SwiGLU epilogue (MXFP4 GEMM only): y is bf16 [M, N/2], silu(gate) * up of the
  // weight rows' gate/up groups of 2 x 32
  int swiglu = 0;
  // QKV split + RoPE (MXFP4 GEMM only): y receives Q, yk K and yv V (bf16 [M, N/3]
  // each, row stride ldy); cs: float [M, head_dim/2, 2] (cos, sin) or nullptr
  int qkv = 0;
  uint16_t* yk = nullptr;
  uint16_t* yv = nullptr;
  const float* cs = nullptr;
  int head_dim = 0;
};

hipError_t launch_int4_sym_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                                uint8_t* codes, float* scales, hipStream_t s);

hipError_t launch_mxfp8_rows(const uint16_t* x, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                             uint8_t* codes, uint8_t* scales, hipStream_t s);

hipError_t launch_gemm_mx8(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                           int64_t M, int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s);

hipError_t launch_gemm_i4(const uint8_t* ac, const float* as, const uint8_t* bc, const float* bs,
                          int64_t M, int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s);

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K,
                          const EpilogueArgs& ep, hipStream_t s);

hipError_t launch_gemm_nv(const uint8_t* ac, const uint8_t* as, const float* ats,
                          const uint8_t* bc, const uint8_t* bs, const float* bts, int64_t M,
                          int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s);

hipError_t launch_gemm_w4a16(const uint16_t* x, int64_t ldx, const uint8_t* wc,
                             const uint16_t* ws, const uint16_t* wz, int64_t M, int64_t N,
                             int64_t K, const EpilogueArgs& ep, hipStream_t s);

// The W4A4 GEMM for any K the formats allow (MXFP4: K % 32 == 0, NVFP4: K % 16 ==
// 0), used when K is not a multiple of the tiled kernels' 128.  fmt 0 or 1.
hipError_t launch_gemm_anyk(int fmt, const uint8_t* ac, const uint8_t* as, const float* ats,
                            const uint8_t* bc, const uint8_t* bs, const float* bts, int64_t M,
                            int64_t N, int64_t K, const EpilogueArgs& ep, hipStream_t s);

// FP8 attention (head_dim 128): the MXFP8 quantization of Q, K (rows) and V
// (transposed, along the keys), and the attention kernel.  Layouts as declared in
// q4lin.h.
hipError_t launch_attn_quantize(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk,
                                const uint16_t* v, int64_t ldv, int64_t batch, int64_t seq, int64_t heads,
                                uint8_t* qc, uint8_t* qs, uint8_t* kc, uint8_t* ks, uint8_t* vc,
                                uint8_t* vs, hipStream_t s);
hipError_t launch_attn_fp8(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                           const uint8_t* vc, const uint8_t* vs, int64_t batch, int64_t seq, int64_t heads,
                           float softmax_scale, uint16_t* out, int64_t ldo, hipStream_t s);

}  // namespace q4
