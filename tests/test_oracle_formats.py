"""Pins of the oracle's element and scale encoders against things other than the
oracle itself: exact brute force in rational arithmetic, the bit-level definition
of each format, and library casts (torch's bf16 and float8_e4m3fn conversions,
math.frexp)."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


# ------------------------------------------------------------------ E2M1 decode
def test_e2m1_decode_matches_bit_level_definition():
    # FP4 E2M1: sign s, exponent e (2 bits, bias 1), mantissa m (1 bit);
    # e = 0 is subnormal: m * 2**(1-1) * 0.5; else 2**(e-1) * (1 + m/2).
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
        want = -mag if s else mag
        got = F.e2m1_decode(np.array([code], np.uint8))[0]
        assert Fraction(got) == want, code
        assert math.copysign(1.0, got) == (-1.0 if s else 1.0)


# ------------------------------------------------------------------ E2M1 encode
def _brute_e2m1(v: Fraction, neg: bool):
    """argmin over the 8 magnitudes in exact arithmetic; ties -> even code
    (mantissa bit 0); beyond 6 saturate."""
    m = abs(v)
    grid = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    if m >= 6:
        idx = 7
    else:
        d = [abs(m - g) for g in grid]
        best = min(d)
        cands = [i for i in range(8) if d[i] == best]
        idx = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
    return (8 if neg else 0) | idx


def test_e2m1_encode_exhaustive_8bit_significands():
    # Every value with an 8-bit significand (all bf16 significands) in binades
    # 2**-14 .. 2**3, both signs, plus zeros and large magnitudes.  Any x * 2**-E
    # the MX quantizer forms is such a value.
    vals = [0.0, -0.0, 8.0, 100.0, 2.0 ** 40, -7.0, -1e30]
    for e in range(-14, 4):
        for sig in range(128, 256):
            v = sig * 2.0 ** (e - 7)
            vals += [v, -v]
    vals = np.array(vals)
    got = F.e2m1_encode(vals)
    for v, g in zip(vals, got):
        assert g == _brute_e2m1(Fraction(float(v)), math.copysign(1.0, v) < 0), v


def test_e2m1_encode_midpoints_tie_to_even():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0, 2, 2, 4, 4, 6, 6])            # 0, 1, 1, 2, 2, 4, 4
    assert np.array_equal(F.e2m1_encode(mids), want)
    assert np.array_equal(F.e2m1_encode(-mids), want | 8)


def test_e2m1_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([np.nan]))
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([np.inf]))


# ------------------------------------------------------------------ floor(log2)
def test_floor_log2_all_positive_bf16_against_frexp():
    bits = _all_finite_bf16()
    v = F.bf16_to_f64(bits)
    v = v[v > 0]
    got = F.floor_log2(v)
    want = np.array([math.frexp(float(x))[1] - 1 for x in v])
    assert np.array_equal(got, want)
    assert got.min() == -133 and got.max() == 127


# ------------------------------------------------------------------ bf16
def test_bf16_decode_against_torch():
    bits = _all_finite_bf16()
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_to_f64(bits), t)


def test_bf16_rne_against_torch_cast():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # force ties (low 16 bits exactly 0x8000) and near-ties on a third of them
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000
    u[1::7] = (u[1::7] & 0xFFFF0000) | 0x7FFF
    x = u.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16_rne(x), want)


def test_bf16_ulp_closed_form():
    assert F.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert F.bf16_ulp(np.array([1.99]))[0] == 2.0 ** -7
    assert F.bf16_ulp(np.array([-3.0]))[0] == 2.0 ** -6
    assert F.bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133
    assert F.bf16_ulp(np.array([2.0 ** -130]))[0] == 2.0 ** -133


# ------------------------------------------------------------------ E4M3
def _torch_e4m3(v):
    t = torch.from_numpy(np.asarray(v, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_against_torch():
    codes = np.arange(0x7F, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.e4m3_decode(codes), want)
    assert F.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert F.e4m3_decode(np.array([0x01], np.uint8))[0] == 2.0 ** -9


def test_e4m3_encode_dense_sweep_against_torch_cast():
    # all non-negative finite bf16 values (as fp32), every E4M3 value, every
    # midpoint between neighbours, and one fp32 ulp either side of each midpoint
    bits = _all_finite_bf16()
    v = F.bf16_to_f64(bits)
    v = np.abs(v[(v >= 0) & (v < 1e6)]).astype(np.float32)   # block maxima are never -0
    vals = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    sweep = np.concatenate([v, vals, mids, up, dn, np.float32([448, 460, 464, 480, 1e5])])
    got = F.e4m3_encode(sweep.astype(np.float64))
    assert np.array_equal(got, _torch_e4m3(sweep))


def test_e4m3_encode_saturates_not_nan():
    got = F.e4m3_encode(np.array([447.9, 448.0, 463.9, 464.0, 479.0, 1e9]))
    assert np.all(got == 0x7E)


# ------------------------------------------------------------------ nibbles
def test_nibble_pack_order_and_roundtrip():
    codes = np.arange(32, dtype=np.uint8).reshape(2, 16) % 16
    packed = F.pack_nibbles(codes)
    assert packed[0, 0] == (codes[0, 0] | (codes[0, 1] << 4))     # even k in the low nibble
    assert np.array_equal(F.unpack_nibbles(packed), codes)
