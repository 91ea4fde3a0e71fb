"""Pins of the oracle's block quantizers: exact round trips of representable
values, the scale rules' defining inequalities checked against brute force, the
outlier-collapse behaviour the SVDQuant Guide describes, an independent torch
re-derivation of the fp32 NVFP4 steps, and brute-force int4 rounding."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from bit_quantized_gemm_quantize_amd import synth
from oracle import formats as F
from oracle import quant as Q


def bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


# ------------------------------------------------------------------ MXFP4
def test_mx_scale_rule_brute_force_all_bf16_amax():
    # For a block whose largest magnitude is A, the OCP MX shared exponent is the
    # one that puts A / 2**E in [4, 8) (E2M1's largest binade is [4, 8)), unless
    # that E falls outside E8M0's [-127, 127].  Checked for every positive bf16 A,
    # by searching E rather than computing it.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits < 0x7F80) & (bits > 0)]          # positive finite bf16
    block = np.zeros((bits.size, 32), dtype=np.uint16)
    block[:, 5] = bits                      # the maximum sits anywhere in the block
    _, scales = Q.mx_quantize(block)
    for b, s in zip(bits, scales[:, 0]):
        a = Fraction(float(F.bf16_to_f64(np.array([b]))[0]))
        E = next(e for e in range(-140, 140) if Fraction(4) <= a / Fraction(2) ** e < 8)
        assert int(s) == max(-127, min(127, E)) + 127


def test_mx_zero_block_and_negative_zero():
    codes, scales = Q.mx_quantize(np.array([[0x8000] * 16 + [0x0000] * 16], np.uint16))
    assert scales[0, 0] == 0
    un = F.unpack_nibbles(codes)[0]
    assert np.all(un[:16] == 8) and np.all(un[16:] == 0)


def test_mx_round_trip_every_code_and_exponent():
    # A block [6 * 2**E, g_1 * 2**E, ...] with grid values g_i must come back with
    # scale byte E + 127 and exactly the same codes, for every E the bf16 input
    # can reach and every one of the 16 codes.
    rng = np.random.default_rng(3)
    rows = []
    want_codes = []
    Es = list(range(-127, 126))
    for E in Es:
        codes = rng.integers(0, 16, size=32).astype(np.uint8)
        codes[0] = 7                                     # +6: fixes the block max
        codes[1:17] = np.arange(16)                      # all codes present
        vals = F.e2m1_decode(codes) * 2.0 ** E
        rows.append(bf16(vals))
        want_codes.append(codes)
    rows = np.array(rows)
    assert np.array_equal(F.bf16_to_f64(rows), np.array([F.e2m1_decode(c) * 2.0 ** E for c, E in zip(want_codes, Es)]))
    codes, scales = Q.mx_quantize(rows)
    assert np.array_equal(scales[:, 0], np.array(Es) + 127)
    assert np.array_equal(F.unpack_nibbles(codes), np.array(want_codes))
    # and dequantization gives the input back exactly
    assert np.array_equal(Q.mx_dequantize(codes, scales), F.bf16_to_f64(rows))


def test_mx_dequant_error_bound():
    # Round to nearest on the grid: for every unsaturated element the error is at
    # most half the grid spacing at that point, times the block scale.
    x = synth.activations(64, 512, seed=11, dist="student_t3")[0]
    codes, scales = Q.mx_quantize(x)
    xd = Q.mx_dequantize(codes, scales)
    xv = F.bf16_to_f64(x)
    scale = np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    m = np.abs(xv) / scale
    half_gap = np.select([m < 2, m < 4, m <= 6], [0.25, 0.5, 1.0], m - 6)   # beyond 6: clipped
    assert np.all(np.abs(xv - xd) <= half_gap * scale)
    assert np.all(m < 8)     # the scale rule never leaves an element beyond 8 * 2**E


def test_mx_outlier_collapse_described_on_the_pages():
    # The SVDQuant Guide ("Why Standard Low-Bit Quantization Fails on DiTs"): one
    # large channel inflates the shared scale so that normal values collapse into
    # one bin.  With block maximum A, every |x| <= 2**(floor(log2 A) - 4) becomes
    # +-0 (it lands at or below 0.25 on the E2M1 grid).
    d = synth.tiny_layer(seed=0)
    x = F.bf16_to_f64(d["x"])
    codes, scales = Q.mx_quantize(d["x"])
    vals = F.e2m1_decode(F.unpack_nibbles(codes))
    ch = d["outlier_channels"]
    obs_out = n_out = obs_norm = n_norm = 0
    expect = var = 0.0
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            blk = x[r, b * 32:(b + 1) * 32]
            A = np.abs(blk).max()
            thr = 2.0 ** (math.floor(math.log2(A)) - 4)
            assert np.all(vals[r, b * 32:(b + 1) * 32][np.abs(blk) <= thr] == 0)
            zero = vals[r, b * 32:(b + 1) * 32] == 0
            inside = ch[(ch >= b * 32) & (ch < (b + 1) * 32)] - b * 32
            if inside.size:
                normal = np.setdiff1d(np.arange(32), inside)
                obs_out += zero[normal].sum()
                n_out += normal.size
                # closed form for the N(0,1) normals: P(|z| <= thr) = erf(thr / sqrt 2)
                p = math.erf(thr / math.sqrt(2.0))
                expect += normal.size * p
                var += normal.size * p * (1 - p)
            else:
                obs_norm += zero.sum()
                n_norm += 32
    assert var > 0
    # the observed collapse in outlier blocks matches the closed form (5 sigma) ...
    assert abs(obs_out - expect) < 5 * math.sqrt(var) + 1
    # ... and is far above the zero rate of ordinary blocks
    assert n_out > 0 and n_norm > 0
    assert obs_out / n_out > 0.5 > 0.2 > obs_norm / n_norm


# ------------------------------------------------------------------ NVFP4
def test_nv_round_trip_representable_tensor():
    # amax_t = 2688 * 2**j makes s_t = 2**j exactly; a block whose largest
    # magnitude is 6 * s_b * s_t reproduces s_b, and grid * s_b * s_t reproduces
    # every code.
    rng = np.random.default_rng(5)
    j = -3
    s_t = 2.0 ** j
    sb_all = F.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    rows, want_sb, want_codes = [], [], []
    for i in range(0, sb_all.size, 2):
        sb_codes = np.array([i + 1, min(i + 2, 0x7E)], np.uint8)
        sbs = F.e4m3_decode(sb_codes)
        codes = rng.integers(0, 16, size=32).astype(np.uint8)
        codes[0] = 7
        codes[16] = 15
        vals = F.e2m1_decode(codes) * np.repeat(sbs, 16) * s_t
        rows.append(vals)
        want_sb.append(sb_codes)
        want_codes.append(codes)
    rows = np.array(rows)
    rows[0, 1] = 2688 * s_t                         # the tensor maximum
    want_codes[0][1] = 7
    want_sb[0][0] = 0x7E
    rows[0, :16] = F.e2m1_decode(want_codes[0][:16]) * 448 * s_t
    bits = bf16(rows)
    assert np.array_equal(F.bf16_to_f64(bits), rows)         # all exactly bf16
    codes, sb, st = Q.nv_quantize(bits)
    assert st == np.float32(s_t)
    assert np.array_equal(sb, np.array(want_sb))
    assert np.array_equal(F.unpack_nibbles(codes), np.array(want_codes))
    assert np.array_equal(Q.nv_dequantize(codes, sb, st), rows)


def test_nv_fp32_steps_against_torch_rederivation():
    # The same definition computed with torch float32 ops and torch's own E4M3
    # cast; E2M1 by nearest-grid argmin with the even tie-break.
    x = synth.activations(48, 256, seed=9, outliers=3)[0]
    codes, sb, st = Q.nv_quantize(x)
    xt = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).float()
    amax = xt.abs().max()
    s_t = amax / torch.tensor(2688.0)
    assert s_t.item() == float(st)
    blocks = xt.reshape(48, 16, 16)
    ratio = blocks.abs().amax(-1) / (torch.tensor(6.0) * s_t)
    sb_t = ratio.clamp(max=448.0).to(torch.float8_e4m3fn)
    assert np.array_equal(sb_t.view(torch.uint8).numpy(), sb)
    den = sb_t.float() * s_t
    v = (blocks / den[..., None]).double().numpy().reshape(48, 256)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    m = np.minimum(np.abs(v), 6.0)
    d = np.abs(m[..., None] - grid)
    best = d.min(-1, keepdims=True)
    tie_even = np.where(d == best, np.arange(8) % 2, 9)     # among the nearest, prefer even
    idx = np.where((d == best).sum(-1) > 1, np.argmin(tie_even, -1), np.argmin(d, -1))
    want = (np.signbit(v).astype(np.uint8) << 3) | idx.astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(codes), want)


def test_nv_block_scale_never_exceeds_e4m3_and_max_block_saturates():
    x = synth.activations(32, 512, seed=2, outliers=5)[0]
    codes, sb, st = Q.nv_quantize(x)
    assert sb.max() <= 0x7E
    xv = np.abs(F.bf16_to_f64(x)).reshape(32, 32, 16)
    r, b = np.unravel_index(np.argmax(xv.max(-1)), (32, 32))
    assert sb[r, b] == 0x7E                     # the block holding amax_t uses 448


def test_nv_zero_tensor():
    codes, sb, st = Q.nv_quantize(np.zeros((2, 32), np.uint16))
    assert st == 1.0 and np.all(sb == 0) and np.all(codes == 0)


# ------------------------------------------------------------------ int4 g64
def test_int4_round_trip_representable_groups():
    # groups holding (0 - z) * s and (15 - z) * s fix s and z exactly; choose s with
    # few significant bits so every (q - z) * s is a bf16 value
    rng = np.random.default_rng(8)
    rows, want_q, want_s, want_z = [], [], [], []
    for s in [2.0 ** -6, 1.5 * 2.0 ** -5, 0.25, 1.0, 1.5 * 2.0 ** 3]:
        for z in range(16):
            q = rng.integers(0, 16, size=64)
            q[3], q[40] = 0, 15
            rows.append((q - z) * s)
            want_q.append(q)
            want_s.append(s)
            want_z.append(z)
    rows = np.array(rows)
    bits = bf16(rows)
    assert np.array_equal(F.bf16_to_f64(bits), rows)
    codes, sc, zc = Q.int4_g64_quantize(bits)
    assert np.array_equal(F.bf16_to_f64(sc)[:, 0], np.array(want_s))
    assert np.array_equal(F.bf16_to_f64(zc)[:, 0], np.array(want_z))
    assert np.array_equal(F.unpack_nibbles(codes), np.array(want_q))
    assert np.array_equal(Q.int4_g64_dequantize(codes, sc, zc), rows)


def test_int4_code_is_brute_force_nearest_level():
    # q minimises |fp32(w / s) - (q - z)| over q in [0, 15]; an exact tie goes to
    # even (q - z), the half-to-even rounding of the page's torch.round.
    w = synth.weights(16, 256, seed=4)
    codes, sc, zc = Q.int4_g64_quantize(w)
    q = F.unpack_nibbles(codes).reshape(16, 4, 64).astype(np.int64)
    s = F.bf16_to_f32(sc)
    z = F.bf16_to_f64(zc).astype(np.int64)
    wv = F.bf16_to_f32(w).reshape(16, 4, 64)
    for r in range(16):
        for g in range(4):
            assert 0 <= z[r, g] <= 15
            for k in range(64):
                v = Fraction(float(np.float32(wv[r, g, k] / s[r, g])))
                d = [abs(v - (qq - z[r, g])) for qq in range(16)]
                best = min(d)
                c = [qq for qq in range(16) if d[qq] == best]
                want = c[0] if len(c) == 1 else [qq for qq in c if (qq - z[r, g]) % 2 == 0][0]
                assert q[r, g, k] == want


def test_int4_scale_and_zero_definition_brute_force():
    w = synth.weights(8, 128, seed=6)
    codes, sc, zc = Q.int4_g64_quantize(w)
    wv = F.bf16_to_f32(w).reshape(8, 2, 64)
    for r in range(8):
        for g in range(2):
            lo = min(0.0, float(wv[r, g].min()))
            hi = max(0.0, float(wv[r, g].max()))
            s32 = np.float32(np.float32(np.float32(hi) - np.float32(lo)) / np.float32(15))
            s_t = torch.tensor(float(s32), dtype=torch.float32).to(torch.bfloat16).float().item()
            assert F.bf16_to_f64(sc[r:r + 1, g])[0] == s_t
            z = np.float32(-np.float32(lo) / np.float32(s_t))
            assert F.bf16_to_f64(zc[r:r + 1, g])[0] == min(15, max(0, round(float(z))))


# ----------------------------------------------------------------------------- int4 symmetric
def test_int4_sym_against_brute_force():
    """Per row: scale = fp32(amax / 7) (struct-rounded Python float division), each
    element rounded half-to-even with Python's round() on the fp32 quotient."""
    import struct

    def f32(v):
        return struct.unpack("<f", struct.pack("<f", v))[0]

    rng = np.random.default_rng(21)
    x = synth.to_bf16_bits(rng.standard_normal((6, 64)) * np.exp(rng.uniform(-6, 6, (6, 1))))
    x[5] = 0                                                   # an all-zero row: scale 1e-8, codes 0
    codes, scales = Q.int4_sym_quantize(x)
    xf = F.bf16_to_f64(x)
    n = F.unpack_nibbles(codes).astype(int)
    q = np.where(n >= 8, n - 16, n)
    for r in range(6):
        amax = float(np.abs(xf[r]).max())
        s = max(f32(amax / 7.0), f32(1e-8))
        assert scales[r] == np.float32(s)
        for k in range(64):
            want = max(-8, min(7, round(f32(float(xf[r, k]) / s))))
            assert q[r, k] == want, (r, k)


def test_int4_sym_closed_forms():
    # the row maximum maps to +-7; multiples of the scale map to themselves; exact
    # halves round to even (so -8 is never produced: |x| <= amax = 7 scale)
    s = 0.5
    vals = np.array([3.5, -3.5, 1.0, -1.0, 0.25, 0.75, -0.25, -0.75, 1.25, -1.25] + [0.0] * 22)
    x = synth.to_bf16_bits(vals[None, :])
    codes, scales = Q.int4_sym_quantize(x)
    assert scales[0] == np.float32(3.5 / 7)
    deq = Q.int4_sym_dequantize(codes, scales)[0]
    assert list(deq[:10] / s) == [7, -7, 2, -2, 0, 2, 0, -2, 2, -2]


# ----------------------------------------------------------------------------- MXFP8
def _e4m3_values():
    """Every non-negative finite E4M3FN value, from the format's definition (exponent
    bias 7, 3 mantissa bits, subnormals, 0x7F is NaN)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


def test_mxfp8_against_brute_force():
    """Blocks over a wide range: the scale from math.frexp, each element the nearest
    E4M3 value (ties to the even code) of x * 2**-E by exhaustive search, saturating at
    448, sign kept."""
    import math
    vals = _e4m3_values()
    rng = np.random.default_rng(31)
    x = synth.to_bf16_bits(rng.standard_normal((3, 64)) * np.exp(rng.uniform(-20, 20, (3, 64))))
    x[2, :32] = synth.to_bf16_bits(np.linspace(-500, 500, 32)[None, :])[0]
    codes, scales = Q.mxfp8_quantize(x)
    xf = F.bf16_to_f64(x)
    for r in range(3):
        for b in range(2):
            blk = xf[r, 32 * b:32 * b + 32]
            amax = float(np.abs(blk).max())
            E = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
            assert scales[r, b] == E + 127
            for j in range(32):
                v = Fraction(float(blk[j])) / Fraction(2) ** E
                m = min(abs(v), Fraction(448))
                best = min(range(0x7F), key=lambda c: (abs(vals[c] - m), c & 1))
                want = best | (0x80 if math.copysign(1.0, float(blk[j])) < 0 else 0)
                assert codes[r, 32 * b + j] == want, (r, b, j)


def test_mxfp8_round_trip_and_saturation():
    # grid values times 2**E with 448 * 2**E present come back exactly; values between
    # 448 and 512 (times 2**E) saturate to 448
    grid = np.array([float(v) for v in _e4m3_values()])
    rng = np.random.default_rng(32)
    blk = rng.choice(grid, 32) * rng.choice([-1, 1], 32)
    blk[0] = 448.0 * 1.0                      # floor(log2 448) = 8 -> E = 0
    x = synth.to_bf16_bits((blk * 2.0 ** 5)[None, :])
    codes, scales = Q.mxfp8_quantize(x)
    assert scales[0, 0] == 127 + 5
    assert np.array_equal(Q.mxfp8_dequantize(codes, scales)[0], blk * 2.0 ** 5)
    y = synth.to_bf16_bits(np.array([[480.0, -496.0, 256.0] + [0.0] * 29]))
    c2, s2 = Q.mxfp8_quantize(y)
    assert s2[0, 0] == 127 and list(Q.mxfp8_dequantize(c2, s2)[0, :3]) == [448.0, -448.0, 256.0]
