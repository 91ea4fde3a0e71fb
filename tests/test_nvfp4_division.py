"""The NVFP4 encoders divide every element by its block's scale product den, the
symmetric INT4 quantizer by its row scale and the asymmetric INT4 packer by its
group scale, in fp32 (IEEE division, round to nearest even).  The kernels form that quotient from
one correctly rounded reciprocal per block, y = RN(1/den), as RN(q + r y) with
q = RN(x y) and r = RN(x - den q) (Markstein's correction, two fmas).  This checks
on the CPU, with exact rational arithmetic for the final fma, that the result
equals the IEEE quotient for bf16 numerators over the whole range of quotients
that decide an E2M1 code, and for denominators with every kind of significand.
The NVFP4 encoders also take each block scale's quotient amax / (6 s_t) this way when
6 s_t lies in [2^-80, 2^100]; the second test covers the quotients that decide a
nonzero E4M3 code (2^-10 to 448)."""

from fractions import Fraction

import numpy as np


def rn32(v):
    """A rational rounded to the nearest fp32 (ties to even), normal range."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scale = Fraction(2) ** (23 - e)
    m = a * scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl) / scale)


def _check_quotients(mags, exp_lo, exp_hi, seed):
    rng = np.random.default_rng(seed)
    f32 = np.float32
    checked = 0
    for trial in range(40):
        if trial % 4 == 0:        # significands all ones, and exact powers of two
            den = f32(np.ldexp(f32(2.0) - f32(2.0 ** -23) * (trial % 8 // 4), int(rng.integers(exp_lo, exp_hi))))
        else:
            den = f32(np.exp2(rng.uniform(exp_lo, exp_hi)) * rng.uniform(1, 2))
        y = f32(1) / den                                             # IEEE: correctly rounded
        xs = (mags * den).astype(np.float32)
        xs = (xs.view(np.uint32) & 0xFFFF0000).view(np.float32)      # bf16 numerators
        xs = np.concatenate([xs, -xs])
        ieee = xs / den
        q = (xs * y).astype(np.float32)
        # x - den q is exact in fp64 (48-bit product, heavy cancellation): one rounding
        r = (xs.astype(np.float64) - np.float64(den) * q.astype(np.float64)).astype(np.float32)
        for qi, ri, ref in zip(q, r, ieee):
            got = rn32(Fraction(float(qi)) + Fraction(float(ri)) * Fraction(float(y)))
            assert got == float(ref)
            checked += 1
    return checked


def test_reciprocal_quotient_is_the_ieee_quotient():
    mags = (np.arange(0x3E00, 0x4184, 3, dtype=np.uint32) << 16).view(np.float32)   # 0.125 .. 16.5
    assert _check_quotients(mags, -60, 60, 7) > 10000


def test_block_scale_quotient_is_the_ieee_quotient():
    """amax / d6 with d6 = 6 s_t: quotients from 2^-10 (half the smallest E4M3
    subnormal; below it every code is 0) to 448, d6 over [2^-79, 2^99]."""
    mags = (np.arange(0x3A80, 0x43E1, 7, dtype=np.uint32) << 16).view(np.float32)   # 2^-10 .. 448
    assert _check_quotients(mags, -79, 99, 11) > 10000
