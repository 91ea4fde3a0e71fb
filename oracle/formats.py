"""Element and scale encoders of the oracle (test infrastructure only).

Every routine works on whole NumPy arrays but is written as the plain definition
of the format, with no blocking or reordering.  Inputs are finite; a non-finite
input raises ``ValueError`` (the layer's contract is finite activations and
weights).
"""

import numpy as np

# FP4 E2M1 magnitudes by 3-bit index (exponent bits e1 e0, mantissa bit m):
# 0 0 0 -> 0, 0 0 1 -> 0.5 (subnormal), then 1, 1.5, 2, 3, 4, 6.
# OCP Microscaling Formats (MX) v1.0, section 5.3.3 (FP4 E2M1 element type).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of the largest normal, 6 = 1.5 * 2**2

# FP8 E4M3FN: bias 7, 3 mantissa bits, no infinities, largest finite 448
# (the +-448 range given in "Quantization for the impatient", stability table).
E4M3_MAX = 448.0


def check_finite(x, what="input"):
    if not np.all(np.isfinite(x)):
        raise ValueError(f"{what} holds a non-finite value; the layer takes finite inputs only")


# ----------------------------------------------------------------------------- bf16
def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x):
    """fp32 values -> bf16 bit patterns, round to nearest, ties to even.

    The 16 discarded bits are rounded on the integer pattern: add 0x7FFF plus the
    lowest kept bit, then truncate.  Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float32)
    check_finite(x)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (fp64 array): 2**(floor(log2|v|) - 7),
    never below the subnormal spacing 2**-133."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.where(v > 0, floor_log2(np.where(v > 0, v, 1.0)), -126)
    return np.ldexp(1.0, np.maximum(e, -126) - 7)


# ----------------------------------------------------------------------------- log2
def floor_log2(v):
    """floor(log2 v) for positive finite fp64 v, read off the binary exponent.

    Every bf16 and fp32 value, subnormals included, is a normal fp64 number, so the
    11-bit exponent field minus the bias 1023 is exactly floor(log2 v).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~(v > 0)) or not np.all(np.isfinite(v)):
        raise ValueError("floor_log2 takes positive finite values")
    biased = (v.view(np.uint64) >> np.uint64(52)) & np.uint64(0x7FF)
    if np.any(biased == 0):
        raise ValueError("fp64 subnormal: outside the range of bf16/fp32 inputs")
    return biased.astype(np.int64) - 1023


# ----------------------------------------------------------------------------- E2M1
def e2m1_encode(v):
    """Real values (fp64) -> FP4 E2M1 codes (uint8, sign in bit 3).

    Round to the nearest point of {0, .5, 1, 1.5, 2, 3, 4, 6}; a value half way
    between two points goes to the one whose code has mantissa bit 0 (the even
    code); magnitudes above 6 saturate to 6 (FP4 has no infinity or NaN).  The sign
    bit is kept, so a negative value that rounds to zero gives code 0x8.

    Decision table on m = |v| (the midpoints and where their ties go):
        m <= 0.25 -> 0        (0.25 ties to 0)
        m <  0.75 -> 0.5
        m <= 1.25 -> 1        (0.75 and 1.25 tie to 1)
        m <  1.75 -> 1.5
        m <= 2.5  -> 2        (1.75 and 2.5 tie to 2)
        m <  3.5  -> 3
        m <= 5    -> 4        (3.5 and 5 tie to 4)
        otherwise -> 6
    """
    v = np.asarray(v, dtype=np.float64)
    check_finite(v)
    m = np.abs(v)
    idx = np.full(m.shape, 7, dtype=np.uint8)
    idx[m <= 5.0] = 6
    idx[m < 3.5] = 5
    idx[m <= 2.5] = 4
    idx[m < 1.75] = 3
    idx[m <= 1.25] = 2
    idx[m < 0.75] = 1
    idx[m <= 0.25] = 0
    return (np.signbit(v).astype(np.uint8) << 3) | idx


def e2m1_decode(codes):
    """FP4 E2M1 codes -> fp64 values (code 0x8 decodes to -0.0)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[codes & 7]
    return np.where(codes & 8, -mag, mag)


# ----------------------------------------------------------------------------- E4M3
def e4m3_encode(v):
    """Non-negative real values (fp64) -> FP8 E4M3FN codes (uint8), round to
    nearest even, saturating at 448, with subnormals (spacing 2**-9 below 2**-6).

    With e = max(floor(log2 v), -6), the representable values in [2**e, 2**(e+1))
    are q * 2**(e-3) for q = 8..15, so q = RNE(v / 2**(e-3)) and the code is
    (e + 7) * 8 + (q - 8); q = 16 carries into the next binade with the same formula,
    and e = -6 with q < 8 gives the subnormal codes 0..7.
    """
    v = np.asarray(v, dtype=np.float64)
    check_finite(v)
    if np.any(v < 0):
        raise ValueError("e4m3_encode is used for non-negative scales only")
    safe = np.where(v > 0, v, 1.0)
    e = np.maximum(np.where(v > 0, floor_log2(safe), -6), -6)
    q = np.rint(v / np.ldexp(1.0, e - 3))          # exact division by a power of two
    code = 8 * e + 48 + q
    code = np.where(v >= E4M3_MAX, 0x7E, code)    # saturate at 448 (code 0x7E)
    return code.astype(np.uint8)


def e4m3_decode(codes):
    """FP8 E4M3FN codes (sign bit clear) -> fp64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    if np.any(codes & 0x80) or np.any((codes & 0x7F) == 0x7F):
        raise ValueError("scale codes are non-negative and never NaN")
    e = (codes >> 3).astype(np.int64)
    m = (codes & 7).astype(np.float64)
    return np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.ldexp(1.0, e - 10))


# ----------------------------------------------------------------------------- nibbles
def pack_nibbles(codes):
    """[rows, K] 4-bit codes -> [rows, K/2] bytes; element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)


def unpack_nibbles(packed):
    """[rows, K/2] bytes -> [rows, K] 4-bit codes (inverse of ``pack_nibbles``)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out
