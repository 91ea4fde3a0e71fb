/*
 * q4lin -- the 4-bit quantized linear layer of a diffusion transformer, for one
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The layer (SVDQuant Guide, aifetchly: "The Three Pillars of SVDQuant",
 * 1. Mathematical Outlier Factorization, forward-projection equation, and
 * "Step 2: The SVDQuant Dual-Branch Linear Layer") is
 *
 *     Y = deq(Q(X)) deq(Q(W))^T  +  (X L1) L2  +  bias
 *
 * with X [M, K] the activations (tokens x in-features, bf16), W^T [N, K] the
 * weight (out-features x in-features), Q a 4-bit block quantizer along K, and the
 * optional rank-r low-rank branch applied to the unquantized X, evaluated right to
 * left (down-projection L1 [K, r] first, then up-projection L2 [r, N]).  Y [M, N].
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer on the current HIP device, owned
 *     by the caller.  The library's one allocation is NVFP4's 4 KB scratch (see
 *     quantize_act); nothing else is allocated, and nothing is kept between calls.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - 4-bit codes are packed two per byte along K: element 2j in the low nibble,
 *     element 2j+1 in the high nibble; a row of K elements is K/2 bytes.  FP4 codes
 *     are E2M1 (sign in bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The 8-bit
 *     format (Q4_MXFP8) takes one E4M3FN byte per element.
 *   - Matrices are row-major.  Packed codes and scales are dense (row stride
 *     K/2 or K bytes, K/32 or K/16 bytes, K/64 elements).
 *   - `stream` is a hipStream_t (NULL: the default stream).  Work is queued on it
 *     and the call returns without synchronizing.
 *   - Arguments are checked on the host before anything is queued; a failed check
 *     returns its status and queues nothing.  Q4_ERR_LAUNCH reports a launch the
 *     HIP runtime refused.  Device-side faults are not reported here.
 *   - Inputs must be finite; results for NaN or infinite inputs are unspecified.
 *   - M = 0 or N = 0 is an empty problem: Q4_OK, nothing queued.
 *   - Calls are thread-safe; calls that write the same buffers must be ordered by
 *     the caller.
 */
#ifndef Q4LIN_H
#define Q4LIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define Q4_API __attribute__((visibility("default")))
#else
#define Q4_API
#endif

typedef enum q4_status {
  Q4_OK = 0,
  Q4_ERR_NULL = 1,    /* a required pointer is NULL                                  */
  Q4_ERR_SHAPE = 2,   /* negative size, K not a multiple of the block, bad rank/stride */
  Q4_ERR_ALIGN = 3,   /* a pointer or leading dimension breaks the stated alignment   */
  Q4_ERR_FORMAT = 4,  /* format not valid for this call                              */
  Q4_ERR_LAUNCH = 5,  /* the HIP runtime rejected a kernel launch                    */
  Q4_ERR_ALLOC = 6    /* the library's one scratch allocation (NVFP4, see below) failed */
} q4_status;

typedef enum q4_format {
  /* MXFP4: E2M1 elements, one E8M0 scale byte (2**(byte-127)) per 32 consecutive K
   * elements; OCP Microscaling Formats v1.0 conversion (shared exponent
   * floor(log2 amax) - 2, clamped to [-127, 127]; elements rounded to nearest
   * even, saturating at 6).  The pages name FP4 E2M1 in "Quantization for the
   * impatient" (bitsandbytes backend). */
  Q4_MXFP4 = 0,
  /* NVFP4-style: E2M1 elements, one FP8 E4M3 scale byte per 16 consecutive K
   * elements and one fp32 per-tensor scale s_t = amax/2688 (2688 = 6 * 448, 448
   * being the E4M3 limit the stability table of "Quantization for the impatient"
   * gives).  Block scale s_b = E4M3_RNE_SAT(amax_b / (6 s_t)), element
   * E2M1_RNE_SAT(x / (s_b s_t)), every step in fp32.  NVFP4 is named in the NVIDIA
   * Technical Blog summary (first optimization layer). */
  Q4_NVFP4 = 1,
  /* Weight-only asymmetric uint4 with a bf16 scale s and a bf16 (integer) zero
   * point z per 64 consecutive K elements: s = bf16(fp32(hi - lo)/15) over the
   * group range [lo, hi] widened to hold 0, z = clamp(RNE(-lo/s), 0, 15),
   * q = clamp(RNE(w/s) + z, 0, 15); the GEMM operand is bf16((q - z) s).  The
   * weight-only (W4A16) path the SVDQuant Guide contrasts with W4A4 in
   * "Why Standard Low-Bit Quantization Fails on DiTs". */
  Q4_INT4_G64 = 2,
  /* Signed int4, symmetric, one fp32 scale per row (per token / per output channel):
   * scale = max(fp32(amax / 7), 1e-8), q = clamp(round_half_even(x / scale), -8, 7)
   * -- the per-channel quantizer of the SVDQuant Guide's "Step 1".  Scales are
   * float [rows].  The GEMM runs on the INT8 MFMA (gfx950 has no 4-bit integer
   * matrix instruction): the comparison "Quantization for the impatient" draws
   * between native and emulated 4-bit matmul.  quantize_act (r = 0),
   * pack_weights and gemm_w4a4 only. */
  Q4_INT4_SYM = 3,
  /* MXFP8: FP8 E4M3FN elements (one byte each), one E8M0 scale byte per 32
   * consecutive K elements; the OCP MX conversion with emax(E4M3) = 8: shared
   * exponent floor(log2 amax) - 8 clamped to [-127, 127], elements rounded to
   * nearest even and saturated at 448, sign kept.  The 8-bit float the pages set
   * beside FP4 (the E4M3 range +-448 in "Quantization for the impatient",
   * stability section; the FP8 variants of the FLUX.2 [klein] model page).
   * Codes are uint8 [rows, K] (not K/2).  quantize_act (r = 0), pack_weights and
   * gemm_w4a4 only. */
  Q4_MXFP8 = 4
} q4_format;

typedef enum q4_out {
  Q4_OUT_BF16 = 0,   /* y is bf16, rounded to nearest even from the fp32 result */
  Q4_OUT_F32 = 1     /* y is fp32                                               */
} q4_out;

/*
 * quantize_act -- dynamic activation quantization, run on every call (outliers move
 * with the timestep: SVDQuant Guide, "Why Standard Low-Bit Quantization Fails on
 * DiTs"), fused with the low-rank down-projection t = X L1 of the same pass over X
 * (SVDQuant Guide, "3. The Nunchaku Fused Kernel Engine": one pass, no second read).
 *
 *   fmt           Q4_MXFP4, Q4_NVFP4, or Q4_INT4_SYM / Q4_MXFP8 (r = 0 only)
 *                 (else Q4_ERR_FORMAT).
 *   x             bf16 [M, K], row stride ldx elements.  16-byte aligned, ldx a
 *                 multiple of 8, ldx >= K.
 *   M, K          0 <= M <= 2^30; K >= 0 and a multiple of 32 (NVFP4 with r = 0:
 *                 of 16, its block).
 *   codes  (out)  uint8 [M, K/2] (MXFP8: [M, K]).  16-byte aligned.
 *   scales (out)  MXFP4, MXFP8: uint8 E8M0 [M, K/32]; NVFP4: uint8 E4M3 [M, K/16];
 *                 INT4_SYM: float [M] (passed through this pointer).
 *                 4-byte aligned.
 *   tensor_scale  NVFP4: float[1], written with s_t.  Other formats: ignored, may
 *                 be NULL.  NVFP4 runs two launches: the tensor amax as one partial
 *                 maximum per workgroup into a 4 KB scratch, then the encode pass
 *                 (with the fused t when r > 0), which reduces them first.  The
 *                 scratch is allocated once per (device, stream) on the first
 *                 NVFP4 call (this one or pack_weights) on that stream and kept
 *                 until the process ends; Q4_ERR_ALLOC if that fails.
 *   l1t           r > 0: bf16 L1^T [r, K] (the down-projection stored
 *                 in-features-contiguous, nn.Linear layout), 16-byte aligned.
 *                 r = 0: ignored.
 *   r             rank of the low-rank branch: 0, 16 or 32.
 *   t      (out)  r > 0: fp32 [M, r], 16-byte aligned, t = X L1 accumulated in fp32.
 */
Q4_API q4_status quantize_act(q4_format fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                       uint8_t* codes, uint8_t* scales, float* tensor_scale,
                       const uint16_t* l1t, int32_t r, float* t, void* stream);

/*
 * quantize_act_noalloc -- quantize_act for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results, checks and status codes are those of
 * quantize_act, and it allocates nothing.  The only scratch quantize_act uses --
 * NVFP4's 1024 per-workgroup partial maxima of the tensor amax, 4 KB -- lives
 * here in a static device array of that size on each GPU the library runs on,
 * held until the process ends; every input size fits it (the amax launch never
 * uses more workgroups than it has words), so no size is rejected for it.  Its
 * device address is looked up once per device on the first call there
 * (Q4_ERR_LAUNCH if that lookup fails).  All calls on one GPU share the array:
 * NVFP4 calls that overlap on one GPU (different streams, no ordering) race and
 * must be ordered by the caller.  MXFP4, INT4_SYM and MXFP8 use no scratch.
 */
Q4_API q4_status quantize_act_noalloc(q4_format fmt, const uint16_t* x, int64_t M, int64_t K,
                                      int64_t ldx, uint8_t* codes, uint8_t* scales,
                                      float* tensor_scale, const uint16_t* l1t, int32_t r, float* t,
                                      void* stream);

/*
 * quantize_act_smooth -- quantize_act with SmoothQuant pre-conditioning of the
 * activation: each element is divided by its channel's smoothing factor s_j
 * before quantization (SVDQuant Guide, "2. SmoothQuant Pre-Conditioning for DiTs":
 * X' = diag(s)^-1 X, W' = W diag(s)).  The division is a multiply by inv_s[j] =
 * 1/s_j: the element quantized is fp32(x_j * inv_s[j]) (fp32 multiply, round to
 * nearest even), then MXFP4 exactly as quantize_act does for a bf16 element.  The
 * low-rank product t = X L1 is computed from the unsmoothed X, so the caller folds
 * diag(s)^-1 into L1 offline (X' L1 = X (diag(s)^-1 L1)).
 *
 *   fmt       Q4_MXFP4 only (else Q4_ERR_FORMAT).
 *   inv_s     fp32 [K], positive and finite (not checked), 16-byte aligned; NULL is
 *             Q4_ERR_NULL.
 *   others    as quantize_act (tensor_scale is not used).
 */
Q4_API q4_status quantize_act_smooth(q4_format fmt, const uint16_t* x, int64_t M, int64_t K,
                              int64_t ldx, const float* inv_s, uint8_t* codes, uint8_t* scales,
                              const uint16_t* l1t, int32_t r, float* t, void* stream);

/*
 * pack_weights -- offline weight quantization and packing, once per model (the
 * SVDQuant Guide's "Step 1: Low-Rank Outlier Decomposition in PyTorch" quantizes
 * the residual weight once; "Quantization for the impatient" packs 4-bit weights
 * several to a word).  The same encoders as quantize_act, along K for every output
 * column n.
 *
 *   fmt               Q4_MXFP4, Q4_NVFP4, Q4_INT4_G64, Q4_INT4_SYM or Q4_MXFP8.
 *   w                 bf16, logical [K, N]: element (k, n) at w[k*stride_k + n*stride_n]
 *                     (stride_k = 1, stride_n = K for nn.Linear's [out, in] storage;
 *                     stride_k = N, stride_n = 1 for row-major [K, N]).  Strides >= 1.
 *                     w 2-byte aligned; with stride_k = 1, stride_n a multiple of 8
 *                     and w 16-byte aligned the rows are read 16 bytes at a time.
 *   K, N              K a multiple of 32 (MXFP4, INT4_SYM, MXFP8), 16 (NVFP4) or
 *                     64 (INT4_G64).
 *   codes  (out)      uint8 [N, K/2] (MXFP8: [N, K]), 16-byte aligned.
 *   scales (out)      MXFP4, MXFP8: uint8 [N, K/32]; NVFP4: uint8 E4M3 [N, K/16];
 *                     INT4_G64: bf16 [N, K/64]; INT4_SYM: float [N].  4-byte aligned.
 *   zeros  (out)      INT4_G64: bf16 [N, K/64] (integers 0..15); else ignored.
 *   tensor_scale(out) NVFP4: float[1] (s_t of the weight); else ignored.  NVFP4
 *                     uses the stream's 4 KB scratch, as quantize_act does.
 */
Q4_API q4_status pack_weights(q4_format fmt, const uint16_t* w, int64_t K, int64_t N,
                       int64_t stride_k, int64_t stride_n, uint8_t* codes, void* scales,
                       uint16_t* zeros, float* tensor_scale, void* stream);

/*
 * gemm_w4a4 -- Y = deq(A) deq(B)^T (+ bias), the 4-bit x 4-bit GEMM of the forward
 * equation (SVDQuant Guide, "1. Mathematical Outlier Factorization"; the 4-bit
 * branch carries about 95% of the compute per the decomposition figure).
 *
 *   fmt       Q4_MXFP4: block-scaled FP4 MFMA.  Q4_NVFP4: exact dequantization
 *             to fp16 (every E2M1 x E4M3 product is an fp16 normal or zero) and
 *             fp16 MFMA -- bf16 when K is not a multiple of 128; the two tensor
 *             scales multiply the fp32 result.
 *             Q4_INT4_SYM: int4 codes widened to int8 for the INT8 MFMA, int32
 *             sums, fp32 row scales (a_scales float [M], b_scales float [N])
 *             applied in the epilogue (gemm_w4a4 only).
 *             Q4_MXFP8: the same block-scaled MFMA with E4M3 operands (codes
 *             [rows, K]); half the FP4 rate (gemm_w4a4 only).
 *   a_*       activation codes [M, K/2] and scales (layout as quantize_act);
 *             a_tscale: NVFP4 float[1], else ignored.
 *   b_*       weight codes [N, K/2] and scales (layout as pack_weights).
 *             Codes 16-byte aligned, scales and tensor scales 4-byte aligned.
 *   M, N      0 .. 2^30.
 *   K         a multiple of 128, at most 2^22 (a tile's rows are addressed with
 *             32-bit offsets).
 *   bias      bf16 [N] or NULL.
 *   y   (out) [M, N] with row stride ldy >= N elements; bf16 or fp32 per `out`.
 *             16-byte aligned, ldy a multiple of 8.
 * Accumulation is fp32; |Y - Y_exact| stays within 1e-3 of the sum of the
 * magnitudes of the products that form each element (plus the bf16 store
 * rounding for Q4_OUT_BF16).
 */
Q4_API q4_status gemm_w4a4(q4_format fmt,
                    const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tscale,
                    const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                    int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                    void* y, int64_t ldy, q4_out out, void* stream);

/*
 * gemm_w4a4_lowrank -- gemm_w4a4 plus the low-rank up-projection t L2 fused into
 * the same kernel (SVDQuant Guide, "3. The Nunchaku Fused Kernel Engine": the 4-bit
 * GEMM and the 16-bit low-rank GEMM in one kernel).  t comes from quantize_act.
 *
 *   t     fp32 [M, r], 16-byte aligned.  It enters the bf16 MFMA as a pair of
 *         bf16 values (t = hi + lo), which keeps 16 significant bits.
 *   l2t   bf16 L2^T [N, r] (the up-projection stored rank-contiguous, nn.Linear
 *         layout), 16-byte aligned.
 *   r     16 or 32 (r = 0 is gemm_w4a4).
 * Other arguments as gemm_w4a4.
 */
Q4_API q4_status gemm_w4a4_lowrank(q4_format fmt,
                            const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tscale,
                            const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tscale,
                            int64_t M, int64_t N, int64_t K,
                            const float* t, const uint16_t* l2t, int32_t r,
                            const uint16_t* bias, void* y, int64_t ldy, q4_out out, void* stream);

/*
 * gemm_w4a4_lowrank_mxout -- the MXFP4 gemm_w4a4_lowrank whose epilogue emits the
 * next layer's activation in MXFP4 instead of (or besides) bf16: the output row's
 * bf16 values, exactly as they would be stored, are quantized in 32-column blocks
 * the way quantize_act quantizes a bf16 activation.  The next layer then needs no
 * separate quantizer pass over Y.  ("NVIDIA Technical Blog Details FLUX 3 Image
 * Klein ...", first optimization layer: 4-bit GEMMs whose epilogues carry the next
 * operation; handing the next layer its 4-bit input is that kind of fusion.)
 *
 *   a_*, b_*, M, N, K, t, l2t, r, bias   as gemm_w4a4_lowrank, MXFP4 operands; r may
 *             be 0 (no low-rank term).  N a multiple of 32.
 *   y   (out) bf16 [M, N] (row stride ldy), or NULL not to store it; when given,
 *             16-byte aligned, ldy a multiple of 8 and >= N.
 *   y_codes (out)  uint8 [M, N/2], row stride ldc bytes (>= N/2, a multiple of 4),
 *             4-byte aligned; low nibble = even column.
 *   y_scales (out) uint8 E8M0 [M, N/32], row stride lds bytes (>= N/32).
 */
Q4_API q4_status gemm_w4a4_lowrank_mxout(const uint8_t* a_codes, const uint8_t* a_scales,
                                  const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                  int64_t N, int64_t K, const float* t, const uint16_t* l2t,
                                  int32_t r, const uint16_t* bias, uint16_t* y, int64_t ldy,
                                  uint8_t* y_codes, int64_t ldc, uint8_t* y_scales, int64_t lds,
                                  void* stream);

/*
 * gemm_w4a4_lowrank_swiglu -- the MXFP4 gemm_w4a4_lowrank with a SwiGLU epilogue: the
 * GEMM computes the gate and up projections of an MLP together and stores only
 * silu(gate) * up, so the 2x wider intermediate never reaches HBM.  ("NVIDIA
 * Technical Blog Details FLUX 3 Image Klein ...", first optimization layer: GEMMs
 * with SwiGLU epilogues.  silu(z) = z / (1 + e^-z), applied to the gate, the plain
 * reading of SwiGLU, which the page names without defining.)
 *
 *   a_*, b_*, M, K, t, l2t, r, bias   as gemm_w4a4_lowrank, MXFP4 operands; r may be
 *             0.  The weight rows (and bias entries, and L2^T rows) come in groups
 *             of 64: rows 64 j .. 64 j + 31 are the gate and rows
 *             64 j + 32 .. 64 j + 63 the up projection of output columns
 *             32 j .. 32 j + 31.
 *   N         the number of weight rows: a multiple of 64; the output has N/2
 *             columns.
 *   y   (out) bf16 [M, N/2], row stride ldy >= N/2 (a multiple of 8), 16-byte
 *             aligned: silu(gate + b_gate) * (up + b_up), evaluated in fp32 from the
 *             fp32 accumulators and rounded to nearest even.
 */
Q4_API q4_status gemm_w4a4_lowrank_swiglu(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                   int64_t N, int64_t K, const float* t, const uint16_t* l2t,
                                   int32_t r, const uint16_t* bias, uint16_t* y, int64_t ldy,
                                   void* stream);

/*
 * gemm_w4a4_lowrank_qkv_rope -- the MXFP4 gemm_w4a4_lowrank of a fused QKV projection
 * whose epilogue splits Y into Q, K and V and applies the rotary position embedding
 * to Q and K, so the projection's output is written once, in place for attention.
 * ("NVIDIA Technical Blog Details FLUX 3 Image Klein ...", first optimization layer:
 * GEMMs with QKV-projection and RoPE epilogues.  The rotation of adjacent pairs by a
 * per-token angle table is the plain reading; the page defines neither.)
 *
 *   a_*, b_*, M, K, t, l2t, r, bias   as gemm_w4a4_lowrank, MXFP4 operands; r may be
 *             0.  Weight rows [0, D) are Q, [D, 2 D) K and [2 D, 3 D) V.
 *   N         3 D with D a multiple of 128.
 *   cs        float [M, head_dim/2, 2]: (cos, sin) of the angle of pair i for row m,
 *             8-byte aligned; or NULL for the split alone.  In Q and K, columns
 *             (2 i, 2 i + 1) of every head (counted inside the head) become
 *             (a c - b s, a s + b c), after the bias, in fp32.
 *   head_dim  even, at most 65536, dividing D (ignored when cs is NULL).
 *   yq, yk, yv (out)  bf16 [M, D] each, row stride ldy >= D (a multiple of 8),
 *             16-byte aligned.
 */
Q4_API q4_status gemm_w4a4_lowrank_qkv_rope(const uint8_t* a_codes, const uint8_t* a_scales,
                                     const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                     int64_t N, int64_t K, const float* t, const uint16_t* l2t,
                                     int32_t r, const uint16_t* bias, const float* cs,
                                     int32_t head_dim, uint16_t* yq, uint16_t* yk, uint16_t* yv,
                                     int64_t ldy, void* stream);

/*
 * gemm_w4a16 -- the weight-only comparison path: Y = X w_hat^T (+ bias) with
 * w_hat = bf16((q - z) s) dequantized tile by tile in LDS and a bf16 MFMA GEMM
 * (SVDQuant Guide, "Why Standard Low-Bit Quantization Fails on DiTs", third point,
 * and the dilemma figure: weights unpacked before every multiplication;
 * "Quantization for the impatient", "Why fewer bits != faster").
 *
 *   x         bf16 [M, K], row stride ldx (multiple of 8), 16-byte aligned.
 *   w_codes   uint8 [N, K/2]; w_scales, w_zeros bf16 [N, K/group] from pack_weights.
 *   group     64.
 *   K, ldx    K a multiple of 64; K and ldx at most 2^22.
 * Other arguments as gemm_w4a4.
 */
Q4_API q4_status gemm_w4a16(const uint16_t* x, int64_t ldx,
                     const uint8_t* w_codes, const uint16_t* w_scales, const uint16_t* w_zeros,
                     int64_t M, int64_t N, int64_t K, int32_t group,
                     const uint16_t* bias, void* y, int64_t ldy, q4_out out, void* stream);

/*
 * attention_fp8_quantize -- the first half of FP8 attention (NVIDIA Technical Blog
 * summary, second optimization layer: attention quantized to FP8): Q and K to
 * MXFP8 along head_dim, V to MXFP8 along the keys, transposed.
 *
 *   q, k, v   bf16 [batch * seq, heads * 128], row strides ldq, ldk, ldv (elements,
 *             at least heads * 128): token-major, head h in columns h*128 .. +128,
 *             as gemm_w4a4_lowrank_qkv_rope writes them.  v and ldv: 4-byte
 *             aligned / even.
 *   head_dim  128 (the only value supported).
 *   q_codes, k_codes    uint8 [batch * seq, heads * 128] E4M3 codes, 16-byte aligned.
 *   q_scales, k_scales  uint8 [batch * seq, heads * 4] E8M0 scale bytes (one per
 *                       32 channels), 4-byte aligned.
 *   v_codes   uint8 [batch, heads * 128, seq64], seq64 = seq rounded up to 64: row
 *             h*128 + d holds channel d of head h over the keys (zero past seq);
 *             16-byte aligned.
 *   v_scales  uint8 [batch, heads, seq64 / 64, 256]: for key block kb (keys
 *             64 kb .. +63), byte c*128 + (d % 32)*4 + d / 32 is the E8M0 scale of
 *             channel d over keys 64 kb + 32 c .. +31 (0 for keys past seq).
 * Element and scale rule as quantize_act with Q4_MXFP8: E = floor(log2 amax) - 8
 * clamped to [-127, 127], codes E4M3 round-to-nearest-even of x 2**-E saturated
 * at +-448.  batch, seq, heads >= 0; batch * seq * heads * 128 below 2^31.  An
 * empty problem (batch, seq or heads 0) returns Q4_OK without looking at the
 * pointers.
 */
Q4_API q4_status attention_fp8_quantize(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk,
                                        const uint16_t* v, int64_t ldv, int64_t batch, int64_t seq,
                                        int64_t heads, int64_t head_dim, uint8_t* q_codes,
                                        uint8_t* q_scales, uint8_t* k_codes, uint8_t* k_scales,
                                        uint8_t* v_codes, uint8_t* v_scales, void* stream);

/*
 * attention_fp8 -- the second half: softmax(c Q K^T) V per (batch item, head) on
 * the operands attention_fp8_quantize wrote, with the FP8 reading of the NVIDIA
 * Technical Blog summary's quantized attention:
 *   scores s = q^ . k^ on the block-scaled MFMA (fp32 accumulation);
 *   online softmax over blocks of 64 keys in key order: per block m' = max(m,
 *   max c s), p = exp(c s - m'), l' = l exp(m - m') + sum p;
 *   P quantized to MXFP8 along the keys per 32-key chunk (the rule above) and
 *   O' = O exp(m - m') + P^ V^ on the block-scaled MFMA;
 *   out = O / l, bf16 round-to-nearest-even.
 * Every query attends to the seq keys of its own batch item (no mask otherwise).
 *
 *   softmax_scale  c > 0, finite (1/sqrt(128) for standard attention).
 *   out            bf16 [batch * seq, heads * 128], row stride ldo (multiple of 4,
 *                  at least heads * 128), 8-byte aligned.
 * Other arguments as attention_fp8_quantize.  The repair budget the page gives
 * (rho = 0.005) is not applied: every query runs in FP8.
 */
Q4_API q4_status attention_fp8(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                               const uint8_t* k_scales, const uint8_t* v_codes, const uint8_t* v_scales,
                               int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                               float softmax_scale, uint16_t* out, int64_t ldo, void* stream);

/* Static, NUL-terminated name of a status ("Q4_OK", ...); "unknown" otherwise. */
Q4_API const char* q4_status_string(q4_status s);

#ifdef __cplusplus
}
#endif

#endif /* Q4LIN_H */
