"""Block quantizers of the oracle (test infrastructure only).

All three quantize each row of a [rows, K] bf16 matrix along K (the reduction
dimension of the GEMM), so they serve both the activation X [M, K] and the weight
stored output-major, W^T [N, K] (nn.Linear's [out, in] orientation, the one the
SVDQuant Guide's dual-branch layer registers for its 4-bit weight buffer).

Why activations are quantized at run time, on every call: the SVDQuant Guide, "Why
Standard Low-Bit Quantization Fails on DiTs", first two points (outliers exceed 100x
the median and move with the timestep).

Every quantizer divides by the scale and then rounds, the order of the per-channel
quantizer in the SVDQuant Guide, "Step 1: Low-Rank Outlier Decomposition in
PyTorch".  The scale rules are not on the pages; they are the readings below.
"""

import numpy as np

from .formats import (
    E2M1_EMAX, E4M3_MAX, E2M1_MAX, bf16_to_f32, bf16_to_f64, check_finite, e2m1_decode,
    e2m1_encode, e4m3_decode, e4m3_encode, f32_to_bf16_rne, floor_log2, pack_nibbles,
    unpack_nibbles)

MX_BLOCK = 32
NV_BLOCK = 16
INT4_GROUP = 64
NV_TENSOR_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)   # 6 * 448 = 2688


def _rows(bits, block):
    bits = np.asarray(bits, dtype=np.uint16)
    if bits.ndim != 2 or bits.shape[1] % block:
        raise ValueError(f"expected a [rows, K] matrix with K a multiple of {block}")
    return bits


# ----------------------------------------------------------------------------- MXFP4
def mx_quantize(bits):
    """MXFP4: E2M1 elements with one E8M0 scale per 32 consecutive K elements.

    OCP MX v1.0 conversion (section 6.3): for a block with largest magnitude amax,
    the shared exponent is E = floor(log2 amax) - emax(E2M1) = floor(log2 amax) - 2,
    clamped to the E8M0 range [-127, 127]; each element is encoded as
    E2M1_RNE_SAT(x * 2**-E).  A block of zeros gets E = -127 (byte 0x00).
    The scale byte is E + 127 (the E8M0 bias).

    Returns (codes uint8 [rows, K/2] low nibble = even k, scales uint8 [rows, K/32]).
    """
    bits = _rows(bits, MX_BLOCK)
    x = bf16_to_f64(bits)
    check_finite(x, "activation/weight")
    return _mx_quantize_values(x)


def _mx_quantize_values(x):
    """The MXFP4 steps of mx_quantize on real values x [rows, K] (fp64, each exactly
    a bf16 or fp32 number)."""
    rows, K = x.shape
    blocks = x.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    E = np.where(amax > 0, floor_log2(np.where(amax > 0, amax, 1.0)) - E2M1_EMAX, -127)
    E = np.clip(E, -127, 127)
    scaled = blocks * np.ldexp(1.0, -E)[..., None]          # exact: a power of two
    codes = e2m1_encode(scaled).reshape(rows, K)
    return pack_nibbles(codes), (E + 127).astype(np.uint8)


def mx_quantize_smoothed(bits, inv_s):
    """MXFP4 of the smoothed activation X' = X diag(s)^-1 (the SVDQuant Guide, "2.
    SmoothQuant Pre-Conditioning for DiTs").  The division by s_j is taken as a
    multiply by the fp32 factor inv_s[j] = 1/s_j, in fp32 with round to nearest even:
    v = fp32(x * inv_s[j]).  v is then quantized exactly as mx_quantize quantizes a
    bf16 element (every fp32 value is exact in fp64).

    inv_s: float32 [K], positive and finite.  Returns (codes, scales) as mx_quantize.
    """
    bits = _rows(bits, MX_BLOCK)
    inv_s = np.asarray(inv_s, dtype=np.float32)
    if inv_s.shape != (bits.shape[1],) or not np.all(np.isfinite(inv_s)) or np.any(~(inv_s > 0)):
        raise ValueError("inv_s must be a positive finite fp32 vector of length K")
    x = bf16_to_f32(bits)
    check_finite(x, "activation")
    v = (x * inv_s[None, :]).astype(np.float32)              # fp32 multiply, RNE
    check_finite(v, "smoothed activation")
    return _mx_quantize_values(v.astype(np.float64))


def mx_dequantize(codes, scales):
    """MXFP4 codes/scales -> fp64 [rows, K]: grid value * 2**(byte - 127)."""
    vals = e2m1_decode(unpack_nibbles(codes))
    rows, K = vals.shape
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != (rows, K // MX_BLOCK) or np.any(scales == 0xFF):
        raise ValueError("bad MX scale array (shape, or the NaN byte 0xFF)")
    E = scales.astype(np.int64) - 127
    return (vals.reshape(rows, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, E)[..., None]).reshape(rows, K)


# ----------------------------------------------------------------------------- NVFP4
def nv_tensor_scale(bits, amax_t=None):
    """Per-tensor fp32 scale s_t = fp32(amax_t / 2688), or 1 for an all-zero tensor.

    2688 = 6 * 448 maps the tensor's largest magnitude onto the largest E2M1 value
    times the largest E4M3 scale, so every block scale fits E4M3.  amax_t, when
    given, is the largest magnitude of the whole tensor that ``bits`` is a slice
    of (so a subset of rows can be quantized as part of the full tensor).
    """
    if amax_t is None:
        x = bf16_to_f32(bits)
        check_finite(x, "activation/weight")
        amax_t = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    amax_t = np.float32(amax_t)
    if amax_t == 0:
        return np.float32(1.0)
    return np.float32(amax_t / NV_TENSOR_DIVISOR)                    # fp32 division


def nv_quantize(bits, amax_t=None):
    """NVFP4-style: E2M1 elements, one E4M3 scale per 16 K elements, one fp32
    tensor scale, every step in fp32 with round to nearest even:

        s_t  = fp32(amax_t / 2688)                    (1 if amax_t = 0)
        s_b  = E4M3_RNE_SAT(fp32(amax_b / fp32(6 * s_t)))
        code = E2M1_RNE_SAT(fp32(x / fp32(s_b * s_t)))   if s_b != 0, else signed 0

    amax_t: the whole tensor's largest magnitude when ``bits`` holds only some of
    its rows (see ``nv_tensor_scale``).

    Returns (codes uint8 [rows, K/2], scales uint8 E4M3 [rows, K/16], s_t float32).
    """
    bits = _rows(bits, NV_BLOCK)
    rows, K = bits.shape
    s_t = nv_tensor_scale(bits, amax_t)
    x = bf16_to_f32(bits).reshape(rows, K // NV_BLOCK, NV_BLOCK)
    amax_b = np.abs(x).max(axis=-1)                                   # float32, exact
    ratio = amax_b / (np.float32(6.0) * s_t)                          # fp32 mul, fp32 div
    sb_codes = e4m3_encode(ratio.astype(np.float64))
    s_b = e4m3_decode(sb_codes).astype(np.float32)                    # exact in fp32
    denom = s_b * s_t                                                 # fp32 multiply
    with np.errstate(divide="ignore", invalid="ignore"):
        scaled = x / denom[..., None]                                 # fp32 division
    scaled = np.where((s_b == 0)[..., None], np.copysign(np.float32(0), x), scaled)
    codes = e2m1_encode(scaled.astype(np.float64)).reshape(rows, K)
    return pack_nibbles(codes), sb_codes, s_t


def nv_dequantize(codes, sb_codes, s_t):
    """NVFP4 codes/scales -> fp64 [rows, K]: grid value * s_b * s_t (exact)."""
    vals = e2m1_decode(unpack_nibbles(codes))
    rows, K = vals.shape
    s_b = e4m3_decode(np.asarray(sb_codes, dtype=np.uint8))
    if s_b.shape != (rows, K // NV_BLOCK):
        raise ValueError("bad NV scale array shape")
    out = vals.reshape(rows, K // NV_BLOCK, NV_BLOCK) * s_b[..., None] * float(np.float32(s_t))
    return out.reshape(rows, K)


# ----------------------------------------------------------------------------- int4 asym g64
def int4_g64_quantize(bits):
    """Asymmetric unsigned int4 with a bf16 scale and a bf16 (integer) zero point
    per 64 consecutive K elements, for the weight-only comparison path:

        lo = min(0, min w), hi = max(0, max w)                     (the range holds 0)
        s  = bf16_RNE(fp32(fp32(hi - lo) / 15)), s = 1 if that is 0
        z  = clamp(RNE(fp32(-lo / s)), 0, 15)                      (an integer)
        q  = clamp(RNE(fp32(w / s)) + z, 0, 15)

    RNE to an integer is half-to-even, the rounding torch.round performs in the
    SVDQuant Guide's per-channel quantizer.

    Returns (codes uint8 [rows, K/2], scales bf16 bits [rows, K/64], zeros bf16 bits).
    """
    bits = _rows(bits, INT4_GROUP)
    rows, K = bits.shape
    w = bf16_to_f32(bits).reshape(rows, K // INT4_GROUP, INT4_GROUP)
    check_finite(w, "weight")
    lo = np.minimum(w.min(axis=-1), np.float32(0))
    hi = np.maximum(w.max(axis=-1), np.float32(0))
    s = bf16_to_f32(f32_to_bf16_rne((hi - lo) / np.float32(15)))     # fp32 sub, div, bf16
    s = np.where(s == 0, np.float32(1), s)
    z = np.clip(np.rint(-lo / s), 0, 15)                              # fp32 div, RNE
    q = np.clip(np.rint(w / s[..., None]) + z[..., None], 0, 15)      # fp32 div, RNE
    codes = pack_nibbles(q.reshape(rows, K).astype(np.uint8))
    return codes, f32_to_bf16_rne(s), f32_to_bf16_rne(z.astype(np.float32) + np.float32(0))


def int4_g64_dequantize(codes, scales, zeros):
    """Weight-only operand: w_hat = bf16_RNE(fp32(q - z) * s), returned as fp64.

    (q - z) has at most 5 bits and s 8, so the fp32 product is exact and the single
    rounding is the one to bf16, the GEMM's operand type.
    """
    q = unpack_nibbles(codes).astype(np.float32)
    rows, K = q.shape
    s = bf16_to_f32(scales)
    z = bf16_to_f32(zeros)
    if s.shape != (rows, K // INT4_GROUP) or z.shape != s.shape:
        raise ValueError("bad int4 scale/zero shape")
    prod = (q.reshape(rows, K // INT4_GROUP, INT4_GROUP) - z[..., None]) * s[..., None]
    return bf16_to_f64(f32_to_bf16_rne(prod.reshape(rows, K)))


# ----------------------------------------------------------------------------- int4 symmetric
INT4_QMAX, INT4_QMIN = 7, -8
INT4_SCALE_FLOOR = np.float32(1e-8)


def _nearest_int_half_even(v):
    """Nearest integer to each fp32 value, ties to the even integer, written out from
    the definition: the integer below, plus one when the fraction is over a half or
    exactly a half above an odd integer.  fp32 values of magnitude 2**23 and more are
    integers already."""
    v = np.asarray(v, dtype=np.float64)                               # exact copy of fp32
    lo = np.floor(v)
    frac = v - lo                                                     # exact: |v| < 2**53
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(lo, 2.0) == 1.0))
    return lo + up


def int4_sym_quantize(bits):
    """Signed int4 with one fp32 step per row (the Q4_INT4_SYM format; the
    per-channel quantizer of the SVDQuant Guide, "Step 1: Low-Rank Outlier
    Decomposition in PyTorch", taken per row for both operands).

    A row is represented as q * step with integer codes q in [-8, 7].  The step
    maps the row's largest magnitude onto the largest positive code:
    step = fp32(amax / 7), and no smaller than 1e-8 (an all-zero row gets the floor).
    Each element's code is the integer nearest to the fp32 quotient fp32(x / step),
    ties to even, limited to the code range; since |x| <= amax = 7 step, only -7 ..
    7 occur.  Codes are stored as two's-complement nibbles, two per byte, even k in
    the low nibble.  Returns (codes uint8 [rows, K/2], steps float32 [rows]).
    """
    bits = _rows(bits, 2)
    x = bf16_to_f32(bits)
    check_finite(x, "activation/weight")
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    step = (amax / np.float32(INT4_QMAX)).astype(np.float32)          # fp32 division
    step = np.where(step < INT4_SCALE_FLOOR, INT4_SCALE_FLOOR, step).astype(np.float32)
    quot = (x / step[:, None]).astype(np.float32)                     # fp32 division
    q = _nearest_int_half_even(quot)
    q = np.minimum(np.maximum(q, INT4_QMIN), INT4_QMAX).astype(np.int64)
    return pack_nibbles((q & 0xF).astype(np.uint8)), step


def int4_sym_dequantize(codes, scales):
    """int4 codes (two's complement nibbles) and fp32 row scales -> fp64 q * scale."""
    n = unpack_nibbles(codes).astype(np.int64)
    q = np.where(n >= 8, n - 16, n)
    scales = np.asarray(scales, dtype=np.float32)
    if scales.shape != (q.shape[0],):
        raise ValueError("bad int4 scale vector shape")
    return q * scales.astype(np.float64)[:, None]


# ----------------------------------------------------------------------------- MXFP8 (E4M3)
E4M3_EMAX = 8                                                     # 448 = 1.75 * 2**8


def mxfp8_quantize(bits):
    """MXFP8: FP8 E4M3FN elements with one E8M0 scale per 32 consecutive K elements,
    by the OCP MX v1.0 conversion as for MXFP4 but with emax(E4M3) = 8: E =
    floor(log2 amax) - 8 clamped to [-127, 127] (-127 for a zero block), each element
    E4M3_RNE(x * 2**-E) saturated at +-448 (a block's largest values can reach
    2**9 * (1 - 2**-8) before saturation), sign kept (a negative value that rounds
    to zero gives 0x80).

    Returns (codes uint8 [rows, K], scales uint8 [rows, K/32]).
    """
    bits = _rows(bits, MX_BLOCK)
    rows, K = bits.shape
    x = bf16_to_f64(bits)
    check_finite(x, "activation/weight")
    blocks = x.reshape(rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    E = np.where(amax > 0, floor_log2(np.where(amax > 0, amax, 1.0)) - E4M3_EMAX, -127)
    E = np.clip(E, -127, 127)
    scaled = blocks * np.ldexp(1.0, -E)[..., None]              # exact: a power of two
    mag = np.minimum(np.abs(scaled), E4M3_MAX)
    codes = e4m3_encode(mag) | np.where(np.signbit(scaled), 0x80, 0).astype(np.uint8)
    return codes.reshape(rows, K).astype(np.uint8), (E + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales):
    """MXFP8 codes/scales -> fp64 [rows, K]: (-1)^s * E4M3 value * 2**(byte - 127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    mag = e4m3_decode(codes & 0x7F)
    vals = np.where(codes & 0x80, -mag, mag)
    E = np.asarray(scales, dtype=np.uint8).astype(np.int64) - 127
    if E.shape != (rows, K // MX_BLOCK):
        raise ValueError("bad MX scale array shape")
    return (vals.reshape(rows, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, E)[..., None]).reshape(rows, K)
