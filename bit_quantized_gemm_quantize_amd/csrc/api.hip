// The C ABI of libq4lin (declared in include/q4lin.h): argument checks on the
// host, then the launches, queued on the caller's stream.  No synchronization;
// the only allocation is the NVFP4 scratch below.
#include "q4lin.h"

#include <map>
#include <mutex>
#include <utility>

#include "q4_internal.h"

// Scratch of quantize_act_noalloc: the NVFP4 partial maxima in a static device
// array, q4::kNvScratchWords words (4 KB) on every GPU the library runs on, held
// until the process ends.  In host code `scratch` names a host-side stand-in, not
// the device memory: only the address static_scratch() looks up is passed on.
static __device__ __align__(256) uint32_t scratch[q4::kNvScratchWords];

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

q4_status launched(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_LAUNCH; }

bool rank_ok(int32_t r) { return r == 0 || r == 16 || r == 32; }

// Size limits of the kernels' 32-bit tile addressing and grid sizes.
constexpr int64_t kMaxRows = int64_t(1) << 30;   // M, N
constexpr int64_t kMaxK = int64_t(1) << 22;      // K, and ldx of the W4A16 activations
constexpr int64_t kMaxLdx = int64_t(1) << 26;    // ldx of the quantizer's activations
// FP8 attention: the code tensors (batch * seq * heads * 128 bytes) stay below 2^31,
// the reach of the kernels' 32-bit buffer offsets
constexpr int64_t kMaxAttnElems = int64_t(1) << 31;

// The NVFP4 tensor-amax scratch (q4::kNvScratchWords words): one buffer per
// (device, stream), allocated on the first NVFP4 quantization queued on that
// stream and kept until the process ends.  Work queued on one stream runs in
// order, so no two calls use one buffer at the same time; calls on different
// streams get different buffers.  Null if the allocation fails.
uint32_t* nv_stream_scratch(void* stream) {
  static std::mutex mu;
  static std::map<std::pair<int, void*>, uint32_t*> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, stream);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  void* p = nullptr;
  if (hipMalloc(&p, sizeof(uint32_t) * q4::kNvScratchWords) != hipSuccess) return nullptr;
  cache.emplace(key, static_cast<uint32_t*>(p));
  return static_cast<uint32_t*>(p);
}

// The array's device address on the current device, looked up once per device
// (with that device current) on its first call there.  Null if the lookup fails.
uint32_t* static_scratch() {
  static std::mutex mu;
  static std::map<int, uint32_t*> addr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = addr.find(dev);
  if (it != addr.end()) return it->second;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  addr.emplace(dev, static_cast<uint32_t*>(p));
  return static_cast<uint32_t*>(p);
}

// K granularity of the W4A4 GEMMs: the block of MXFP4 (32) and NVFP4 (16); the
// INT4 and MXFP8 kernels step K in tiles of 128.
int64_t gemm_k_unit(q4_format fmt) { return fmt == Q4_MXFP4 ? 32 : (fmt == Q4_NVFP4 ? 16 : 128); }

// Checks shared by the two W4A4 entry points.
q4_status check_w4a4(q4_format fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                     const float* a_tscale, const uint8_t* b_codes, const uint8_t* b_scales,
                     const float* b_tscale, int64_t M, int64_t N, int64_t K, void* y, int64_t ldy,
                     q4_out out) {
  if (fmt != Q4_MXFP4 && fmt != Q4_NVFP4 && fmt != Q4_INT4_SYM && fmt != Q4_MXFP8) return Q4_ERR_FORMAT;
  if (out != Q4_OUT_BF16 && out != Q4_OUT_F32) return Q4_ERR_FORMAT;
  if (M < 0 || N < 0 || K < 0 || (K % gemm_k_unit(fmt)) != 0 || ldy < N) return Q4_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || K > kMaxK) return Q4_ERR_SHAPE;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !y) return Q4_ERR_NULL;
  if (fmt == Q4_NVFP4 && (!a_tscale || !b_tscale)) return Q4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(y, 16) || (ldy % 8) != 0)
    return Q4_ERR_ALIGN;
  if (fmt == Q4_NVFP4 && (!aligned(a_tscale, 4) || !aligned(b_tscale, 4))) return Q4_ERR_ALIGN;
  return Q4_OK;
}

// quantize_act and quantize_act_noalloc: the same checks and launches; they differ
// only in where the NVFP4 partial maxima live.
q4_status quantize_act_impl(q4_format fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* codes, uint8_t* scales, float* tensor_scale, const uint16_t* l1t,
                            int32_t r, float* t, void* stream, bool noalloc) {
  if (fmt != Q4_MXFP4 && fmt != Q4_NVFP4 && fmt != Q4_INT4_SYM && fmt != Q4_MXFP8) return Q4_ERR_FORMAT;
  if ((fmt == Q4_INT4_SYM || fmt == Q4_MXFP8) && r != 0) return Q4_ERR_FORMAT;
  // NVFP4 blocks are 16 wide; with the fused t the pass reads 32 at a time
  const int64_t unit = (fmt == Q4_NVFP4 && r == 0) ? 16 : 32;
  if (M < 0 || K < 0 || (K % unit) != 0 || ldx < K || !rank_ok(r)) return Q4_ERR_SHAPE;
  if (M > kMaxRows || K > kMaxK || ldx > kMaxLdx) return Q4_ERR_SHAPE;
  if (!x || !codes || !scales) return Q4_ERR_NULL;
  if (fmt == Q4_NVFP4 && !tensor_scale) return Q4_ERR_NULL;
  if (r > 0 && (!l1t || !t)) return Q4_ERR_NULL;
  if (!aligned(x, 16) || (ldx % 8) != 0 || !aligned(codes, 16) || !aligned(scales, 4))
    return Q4_ERR_ALIGN;
  if (fmt == Q4_NVFP4 && !aligned(tensor_scale, 4)) return Q4_ERR_ALIGN;
  if (r > 0 && (!aligned(l1t, 16) || !aligned(t, 16))) return Q4_ERR_ALIGN;
  if (M == 0) return Q4_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == Q4_INT4_SYM)
    return launched(q4::launch_int4_sym_rows(x, M, K, ldx, 1, codes, reinterpret_cast<float*>(scales), s));
  if (fmt == Q4_MXFP8) return launched(q4::launch_mxfp8_rows(x, M, K, ldx, 1, codes, scales, s));
  uint32_t* scr = nullptr;
  if (fmt == Q4_NVFP4) {
    // the amax launch never has more workgroups than the scratch has words, so
    // every size fits either scratch
    scr = noalloc ? static_scratch() : nv_stream_scratch(stream);
    if (scr == nullptr) return noalloc ? Q4_ERR_LAUNCH : Q4_ERR_ALLOC;
  }
  return launched(q4::launch_quantize_act((int)fmt, x, M, K, ldx, codes, scales, tensor_scale, l1t, (int)r,
                                          t, s, scr));
}

}  // namespace

extern "C" {

const char* q4_status_string(q4_status s) {
  switch (s) {
    case Q4_OK: return "Q4_OK";
    case Q4_ERR_NULL: return "Q4_ERR_NULL";
    case Q4_ERR_SHAPE: return "Q4_ERR_SHAPE";
    case Q4_ERR_ALIGN: return "Q4_ERR_ALIGN";
    case Q4_ERR_FORMAT: return "Q4_ERR_FORMAT";
    case Q4_ERR_LAUNCH: return "Q4_ERR_LAUNCH";
    case Q4_ERR_ALLOC: return "Q4_ERR_ALLOC";
  }
  return "unknown";
}

q4_status quantize_act(q4_format fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                       uint8_t* codes, uint8_t* scales, float* tensor_scale,
                       const uint16_t* l1t, int32_t r, float* t, void* stream) {
  return quantize_act_impl(fmt, x, M, K, ldx, codes, scales, tensor_scale, l1t, r, t, stream, false);
}

q4_status quantize_act_noalloc(q4_format fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* codes, uint8_t* scales, float* tensor_scale,
                               const uint16_t* l1t, int32_t r, float* t, void* stream) {
  return quantize_act_impl(fmt, x, M, K, ldx, codes, scales, tensor_scale, l1t, r, t, stream, true);
}

q4_status quantize_act_smooth(q4_format fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const float* inv_s, uint8_t* codes, uint8_t* scales,
                              const uint16_t* l1t, int32_t r, float* t, void* stream) {
  if (fmt != Q4_MXFP4) return Q4_ERR_FORMAT;
  if (M < 0 || K < 0 || (K % 32) != 0 || ldx < K || !rank_ok(r)) return Q4_ERR_SHAPE;
  if (M > kMaxRows || K > kMaxK || ldx > kMaxLdx) return Q4_ERR_SHAPE;
  if (!x || !inv_s || !codes || !scales) return Q4_ERR_NULL;
  if (r > 0 && (!l1t || !t)) return Q4_ERR_NULL;
  if (!aligned(x, 16) || (ldx % 8) != 0 || !aligned(codes, 16) || !aligned(scales, 4) ||
      !aligned(inv_s, 16))
    return Q4_ERR_ALIGN;
  if (r > 0 && (!aligned(l1t, 16) || !aligned(t, 16))) return Q4_ERR_ALIGN;
  if (M == 0) return Q4_OK;
  return launched(q4::launch_quantize_act((int)fmt, x, M, K, ldx, codes, scales, nullptr, l1t, (int)r,
                                          t, static_cast<hipStream_t>(stream), nullptr, inv_s));
}

q4_status pack_weights(q4_format fmt, const uint16_t* w, int64_t K, int64_t N, int64_t stride_k,
                       int64_t stride_n, uint8_t* codes, void* scales, uint16_t* zeros,
                       float* tensor_scale, void* stream) {
  if (fmt != Q4_MXFP4 && fmt != Q4_NVFP4 && fmt != Q4_INT4_G64 && fmt != Q4_INT4_SYM && fmt != Q4_MXFP8)
    return Q4_ERR_FORMAT;
  const int64_t blk = fmt == Q4_INT4_G64 ? 64 : (fmt == Q4_NVFP4 ? 16 : 32);
  if (K < 0 || N < 0 || (K % blk) != 0 || stride_k < 1 || stride_n < 1) return Q4_ERR_SHAPE;
  if (!w || !codes || !scales) return Q4_ERR_NULL;
  if (fmt == Q4_INT4_G64 && !zeros) return Q4_ERR_NULL;
  if (fmt == Q4_NVFP4 && !tensor_scale) return Q4_ERR_NULL;
  if (!aligned(w, 2) || !aligned(codes, 16) || !aligned(scales, 4)) return Q4_ERR_ALIGN;
  if (fmt == Q4_INT4_G64 && !aligned(zeros, 2)) return Q4_ERR_ALIGN;
  if (fmt == Q4_NVFP4 && !aligned(tensor_scale, 4)) return Q4_ERR_ALIGN;
  if (N == 0) return Q4_OK;
  if (fmt == Q4_INT4_SYM)
    return launched(q4::launch_int4_sym_rows(w, N, K, stride_n, stride_k, codes,
                                             static_cast<float*>(scales), static_cast<hipStream_t>(stream)));
  if (fmt == Q4_MXFP8)
    return launched(q4::launch_mxfp8_rows(w, N, K, stride_n, stride_k, codes, static_cast<uint8_t*>(scales),
                                          static_cast<hipStream_t>(stream)));
  uint32_t* scratch = nullptr;
  if (fmt == Q4_NVFP4 && (scratch = nv_stream_scratch(stream)) == nullptr) return Q4_ERR_ALLOC;
  return launched(q4::launch_pack_weights((int)fmt, w, K, N, stride_k, stride_n, codes, scales, zeros,
                                          tensor_scale, static_cast<hipStream_t>(stream), scratch));
}

q4_status gemm_w4a4(q4_format fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                    const float* a_tscale, const uint8_t* b_codes, const uint8_t* b_scales,
                    const float* b_tscale, int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                    void* y, int64_t ldy, q4_out out, void* stream) {
  q4_status st = check_w4a4(fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K,
                            y, ldy, out);
  if (st != Q4_OK) return st;
  if (M == 0 || N == 0) return Q4_OK;
  q4::EpilogueArgs ep{nullptr, nullptr, 0, bias, y, ldy, out == Q4_OUT_F32 ? 1 : 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == Q4_INT4_SYM)
    return launched(q4::launch_gemm_i4(a_codes, reinterpret_cast<const float*>(a_scales), b_codes,
                                       reinterpret_cast<const float*>(b_scales), M, N, K, ep, s));
  if (fmt == Q4_MXFP8) return launched(q4::launch_gemm_mx8(a_codes, a_scales, b_codes, b_scales, M, N, K, ep, s));
  if (K % 128 != 0)
    return launched(q4::launch_gemm_anyk((int)fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M,
                                         N, K, ep, s));
  if (fmt == Q4_MXFP4) return launched(q4::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, ep, s));
  return launched(q4::launch_gemm_nv(a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, ep, s));
}

q4_status gemm_w4a4_lowrank(q4_format fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                            const float* a_tscale, const uint8_t* b_codes, const uint8_t* b_scales,
                            const float* b_tscale, int64_t M, int64_t N, int64_t K, const float* t,
                            const uint16_t* l2t, int32_t r, const uint16_t* bias, void* y,
                            int64_t ldy, q4_out out, void* stream) {
  q4_status st = check_w4a4(fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K,
                            y, ldy, out);
  if (st != Q4_OK) return st;
  if (fmt == Q4_INT4_SYM || fmt == Q4_MXFP8) return Q4_ERR_FORMAT;
  if (!rank_ok(r)) return Q4_ERR_SHAPE;
  if (r > 0 && (!t || !l2t)) return Q4_ERR_NULL;
  if (r > 0 && (!aligned(t, 16) || !aligned(l2t, 16))) return Q4_ERR_ALIGN;
  if (M == 0 || N == 0) return Q4_OK;
  q4::EpilogueArgs ep{r > 0 ? t : nullptr, r > 0 ? l2t : nullptr, (int)r, bias, y, ldy,
                      out == Q4_OUT_F32 ? 1 : 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K % 128 != 0)
    return launched(q4::launch_gemm_anyk((int)fmt, a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M,
                                         N, K, ep, s));
  if (fmt == Q4_MXFP4) return launched(q4::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, ep, s));
  return launched(q4::launch_gemm_nv(a_codes, a_scales, a_tscale, b_codes, b_scales, b_tscale, M, N, K, ep, s));
}

q4_status gemm_w4a4_lowrank_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                   int64_t N, int64_t K, const float* t, const uint16_t* l2t,
                                   int32_t r, const uint16_t* bias, uint16_t* y, int64_t ldy,
                                   void* stream) {
  if (M < 0 || N < 0 || K < 0 || (K % 128) != 0 || (N % 64) != 0 || !rank_ok(r)) return Q4_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || K > kMaxK || ldy < N / 2) return Q4_ERR_SHAPE;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !y) return Q4_ERR_NULL;
  if (r > 0 && (!t || !l2t)) return Q4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(y, 16) || (ldy % 8) != 0)
    return Q4_ERR_ALIGN;
  if (r > 0 && (!aligned(t, 16) || !aligned(l2t, 16))) return Q4_ERR_ALIGN;
  if (M == 0 || N == 0) return Q4_OK;
  q4::EpilogueArgs ep{r > 0 ? t : nullptr, r > 0 ? l2t : nullptr, (int)r, bias, y, ldy, 0};
  ep.swiglu = 1;
  return launched(q4::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, ep,
                                     static_cast<hipStream_t>(stream)));
}

q4_status gemm_w4a4_lowrank_qkv_rope(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                     int64_t N, int64_t K, const float* t, const uint16_t* l2t,
                                     int32_t r, const uint16_t* bias, const float* cs,
                                     int32_t head_dim, uint16_t* yq, uint16_t* yk, uint16_t* yv,
                                     int64_t ldy, void* stream) {
  const int64_t D = N / 3;
  if (M < 0 || N < 0 || K < 0 || (K % 128) != 0 || (N % 384) != 0 || !rank_ok(r)) return Q4_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || K > kMaxK || ldy < D) return Q4_ERR_SHAPE;
  if (cs && (head_dim < 2 || head_dim > 65536 || (head_dim % 2) != 0 || (D % head_dim) != 0))
    return Q4_ERR_SHAPE;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !yq || !yk || !yv) return Q4_ERR_NULL;
  if (r > 0 && (!t || !l2t)) return Q4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(yq, 16) || !aligned(yk, 16) || !aligned(yv, 16) ||
      (ldy % 8) != 0)
    return Q4_ERR_ALIGN;
  if (cs && !aligned(cs, 8)) return Q4_ERR_ALIGN;
  if (r > 0 && (!aligned(t, 16) || !aligned(l2t, 16))) return Q4_ERR_ALIGN;
  if (M == 0 || N == 0) return Q4_OK;
  q4::EpilogueArgs ep{r > 0 ? t : nullptr, r > 0 ? l2t : nullptr, (int)r, bias, yq, ldy, 0};
  ep.qkv = 1;
  ep.yk = yk;
  ep.yv = yv;
  ep.cs = cs;
  ep.head_dim = cs ? (int)head_dim : 0;
  return launched(q4::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, ep,
                                     static_cast<hipStream_t>(stream)));
}

q4_status gemm_w4a4_lowrank_mxout(const uint8_t* a_codes, const uint8_t* a_scales,
                                  const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                  int64_t N, int64_t K, const float* t, const uint16_t* l2t,
                                  int32_t r, const uint16_t* bias, uint16_t* y, int64_t ldy,
                                  uint8_t* y_codes, int64_t ldc, uint8_t* y_scales, int64_t lds,
                                  void* stream) {
  if (M < 0 || N < 0 || K < 0 || (K % 128) != 0 || (N % 32) != 0 || !rank_ok(r)) return Q4_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || K > kMaxK) return Q4_ERR_SHAPE;
  if (ldc < N / 2 || lds < N / 32 || (y && ldy < N)) return Q4_ERR_SHAPE;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !y_codes || !y_scales) return Q4_ERR_NULL;
  if (r > 0 && (!t || !l2t)) return Q4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(y_codes, 4) || (ldc % 4) != 0)
    return Q4_ERR_ALIGN;
  if (y && (!aligned(y, 16) || (ldy % 8) != 0)) return Q4_ERR_ALIGN;
  if (r > 0 && (!aligned(t, 16) || !aligned(l2t, 16))) return Q4_ERR_ALIGN;
  if (M == 0 || N == 0) return Q4_OK;
  q4::EpilogueArgs ep{r > 0 ? t : nullptr, r > 0 ? l2t : nullptr, (int)r, bias, y, y ? ldy : 0, 0};
  ep.qc = y_codes;
  ep.ldc = ldc;
  ep.qs = y_scales;
  ep.lds = lds;
  return launched(q4::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, M, N, K, ep,
                                     static_cast<hipStream_t>(stream)));
}

q4_status gemm_w4a16(const uint16_t* x, int64_t ldx, const uint8_t* w_codes,
                     const uint16_t* w_scales, const uint16_t* w_zeros, int64_t M, int64_t N,
                     int64_t K, int32_t group, const uint16_t* bias, void* y, int64_t ldy,
                     q4_out out, void* stream) {
  if (out != Q4_OUT_BF16 && out != Q4_OUT_F32) return Q4_ERR_FORMAT;
  if (group != 64) return Q4_ERR_SHAPE;
  if (M < 0 || N < 0 || K < 0 || (K % 64) != 0 || ldx < K || ldy < N) return Q4_ERR_SHAPE;
  if (M > kMaxRows || N > kMaxRows || K > kMaxK || ldx > kMaxK) return Q4_ERR_SHAPE;
  if (!x || !w_codes || !w_scales || !w_zeros || !y) return Q4_ERR_NULL;
  if (!aligned(x, 16) || (ldx % 8) != 0 || !aligned(w_codes, 16) || !aligned(w_scales, 2) ||
      !aligned(w_zeros, 2) || !aligned(y, 16) || (ldy % 8) != 0)
    return Q4_ERR_ALIGN;
  if (M == 0 || N == 0) return Q4_OK;
  q4::EpilogueArgs ep{nullptr, nullptr, 0, bias, y, ldy, out == Q4_OUT_F32 ? 1 : 0};
  return launched(q4::launch_gemm_w4a16(x, ldx, w_codes, w_scales, w_zeros, M, N, K, ep,
                                        static_cast<hipStream_t>(stream)));
}

q4_status attention_fp8_quantize(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk,
                                 const uint16_t* v, int64_t ldv, int64_t batch, int64_t seq, int64_t heads,
                                 int64_t head_dim, uint8_t* q_codes, uint8_t* q_scales, uint8_t* k_codes,
                                 uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales, void* stream) {
  if (head_dim != 128 || batch < 0 || seq < 0 || heads < 0) return Q4_ERR_SHAPE;
  if (batch * seq * heads > kMaxAttnElems / 128) return Q4_ERR_SHAPE;
  const int64_t width = heads * 128;
  if (ldq < width || ldk < width || ldv < width || ldq > kMaxLdx || ldk > kMaxLdx || ldv > kMaxLdx)
    return Q4_ERR_SHAPE;
  if (batch == 0 || seq == 0 || heads == 0) return Q4_OK;   // empty: the pointers are not looked at
  if (!q || !k || !v || !q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales)
    return Q4_ERR_NULL;
  if (!aligned(q, 2) || !aligned(k, 2) || !aligned(v, 4) || (ldv % 2) != 0 || !aligned(q_codes, 16) ||
      !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scales, 4) || !aligned(k_scales, 4) ||
      !aligned(v_scales, 4))
    return Q4_ERR_ALIGN;
  return launched(q4::launch_attn_quantize(q, ldq, k, ldk, v, ldv, batch, seq, heads, q_codes, q_scales, k_codes,
                                           k_scales, v_codes, v_scales, static_cast<hipStream_t>(stream)));
}

q4_status attention_fp8(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                        const uint8_t* k_scales, const uint8_t* v_codes, const uint8_t* v_scales, int64_t batch,
                        int64_t seq, int64_t heads, int64_t head_dim, float softmax_scale, uint16_t* out,
                        int64_t ldo, void* stream) {
  if (head_dim != 128 || batch < 0 || seq < 0 || heads < 0) return Q4_ERR_SHAPE;
  if (batch * seq * heads > kMaxAttnElems / 128) return Q4_ERR_SHAPE;
  if (!(softmax_scale > 0.0f) || !(softmax_scale < 3.0e38f)) return Q4_ERR_SHAPE;
  if (ldo < heads * 128 || ldo > kMaxLdx) return Q4_ERR_SHAPE;
  if (batch == 0 || seq == 0 || heads == 0) return Q4_OK;   // empty: the pointers are not looked at
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales || !out) return Q4_ERR_NULL;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(q_scales, 4) ||
      !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(out, 8) || (ldo % 4) != 0)
    return Q4_ERR_ALIGN;
  return launched(q4::launch_attn_fp8(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, batch, seq, heads,
                                      softmax_scale, out, ldo, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
