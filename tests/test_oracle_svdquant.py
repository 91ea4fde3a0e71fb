"""SVDQuant pre-conditioning, CPU only: the oracle's smoothed MXFP4 quantizer and
the offline preparation (smoothing factors, activation-weighted low-rank split,
residual), each pinned to something other than itself."""

import math
import struct
from fractions import Fraction

import numpy as np

import oracle
from bit_quantized_gemm_quantize_amd import synth, weight_prep

F, Q = oracle.formats, oracle.quant
GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def f32(v):
    """Round a Python float (fp64) to fp32, nearest even, through struct."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def encode_brute(v):
    """E2M1 code of a real value: nearest grid point by exhaustive search, ties to
    the even code, saturating, sign kept (argmin written out independently)."""
    m = Fraction(abs(v))
    best = min(range(8), key=lambda i: (abs(GRID[i] - m), i & 1))
    if m > 6:
        best = 7
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_smoothing_by_one_is_plain_mx():
    x, _, _ = synth.activations(16, 128, seed=1, outliers=3)
    assert all(np.array_equal(a, b) for a, b in
               zip(Q.mx_quantize(x), Q.mx_quantize_smoothed(x, np.ones(128, np.float32))))


def test_smoothing_by_powers_of_two_shifts_the_scales():
    # v = x * 2^k is exact, so the codes are unchanged and every scale byte moves by k
    x, _, _ = synth.activations(16, 128, seed=2, outliers=3)
    c0, s0 = Q.mx_quantize(x)
    k = np.repeat(np.array([-3, 2, 0, 5]), 32)
    c1, s1 = Q.mx_quantize_smoothed(x, np.ldexp(1.0, k).astype(np.float32))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(int), s0.astype(int) + k[::32][None, :])


def test_smoothed_quantizer_against_brute_force():
    rng = np.random.default_rng(5)
    rows, K = 4, 64
    x = synth.to_bf16_bits(rng.standard_normal((rows, K)) * np.exp(rng.uniform(-4, 4, (rows, K))))
    inv = rng.uniform(0.01, 3.0, K).astype(np.float32)
    codes, scales = Q.mx_quantize_smoothed(x, inv)
    codes = F.unpack_nibbles(codes)
    xf = F.bf16_to_f64(x)
    for r in range(rows):
        for b in range(K // 32):
            v = [f32(float(xf[r, 32 * b + j]) * float(inv[32 * b + j])) for j in range(32)]
            amax = max(abs(t) for t in v)
            E = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 2))
            assert scales[r, b] == E + 127
            for j in range(32):
                assert codes[r, 32 * b + j] == encode_brute(math.ldexp(v[j], -E)), (r, b, j)


def test_smoothing_factors_closed_form():
    x, ch, _ = synth.activations(64, 96, seed=3, outliers=2)
    wt = synth.weights(40, 96, seed=3)
    wt = wt.copy()
    wt[:, 5] = 0                                            # a zero weight channel -> s = 1
    inv, s = weight_prep.smoothing_factors(x, wt)
    xa = np.abs(F.bf16_to_f64(x)).max(axis=0)
    wa = np.abs(F.bf16_to_f64(wt)).max(axis=0)
    want = np.sqrt(xa / np.where(wa > 0, wa, 1.0))
    want[5] = 1.0
    assert np.allclose(s, want, rtol=2 ** -23)
    assert np.array_equal(inv, (1.0 / want).astype(np.float32))
    assert np.all(np.abs(s * inv.astype(np.float64) - 1.0) <= 2.0 ** -52)   # s = 1 / inv
    assert np.all(s[ch] > 4 * np.median(s))   # outlier channels (gain >= 30): about sqrt(gain) x


def test_weighted_lowrank_identity_is_truncated_svd():
    rng = np.random.default_rng(7)
    w = rng.standard_normal((48, 40))
    l1, l2, sv = weight_prep.weighted_lowrank(w, np.eye(48), 6, ridge=0.0)
    u, s, vh = np.linalg.svd(w, full_matrices=False)
    assert np.allclose(l1 @ l2, (u[:, :6] * s[:6]) @ vh[:6], atol=1e-10)
    assert np.allclose(sv, s)


def test_weighted_lowrank_error_closed_form_and_optimality():
    rng = np.random.default_rng(8)
    K, N, r = 40, 30, 5
    a = rng.standard_normal((200, K)) * np.exp(rng.uniform(-2, 2, K))[None, :]
    c = np.cov(a.T)
    w = rng.standard_normal((K, N))
    l1, l2, sv = weight_prep.weighted_lowrank(w, c, r, ridge=0.0)
    lam, q = np.linalg.eigh(0.5 * (c + c.T))
    root = (q * np.sqrt(lam)[None, :]) @ q.T
    err = np.linalg.norm(root @ (w - l1 @ l2))
    assert math.isclose(err, math.sqrt(np.sum(sv[r:] ** 2)), rel_tol=1e-9)   # Eckart-Young
    u, s, vh = np.linalg.svd(w, full_matrices=False)
    plain = (u[:, :r] * s[:r]) @ vh[:r]
    assert err < np.linalg.norm(root @ (w - plain))


def test_svdquant_split_reconstructs_the_smoothed_weight():
    d = weight_prep.attn_proj_svdquant(seed=4, M=64, K=256, N=192, rank=16, calib=256)
    s = 1.0 / d["inv_s"].astype(np.float64)
    w = F.bf16_to_f64(d["wt"]).T * s[:, None]                      # W' [K, N]
    approx = (F.bf16_to_f64(d["l1"]) * s[:, None]) @ F.bf16_to_f64(d["l2"])
    r = F.bf16_to_f64(d["rt"]).T
    # R' is bf16(W' - approx): within half a bf16 ulp of the exact difference
    assert np.all(np.abs(approx + r - w) <= np.abs(w - approx) * 2.0 ** -8 + 1e-30)
    # the smoothed weight's big rows (the outlier channels) go to the low-rank part
    ch = d["outlier_channels"]
    assert np.abs(r[ch]).max() < 0.2 * np.abs(w[ch]).max()


def test_svdquant_lowers_the_layer_error():
    """Quality, against the unquantized bf16 product in fp64: smoothing plus the
    weighted low-rank branch beats plain W4A4 and the unsmoothed SVD split by a wide
    margin on activations with 1% outlier channels."""
    M, K, N, r = 256, 512, 512, 32
    d = weight_prep.attn_proj_svdquant(seed=3, M=M, K=K, N=N, rank=r, calib=512)
    x = F.bf16_to_f64(d["x"])
    y = x @ F.bf16_to_f64(d["wt"]).T
    rel = lambda yq: np.linalg.norm(yq - y) / np.linalg.norm(y)
    A = Q.mx_dequantize(*Q.mx_quantize(d["x"]))
    plain = rel(A @ Q.mx_dequantize(*Q.mx_quantize(d["wt"])).T)
    l1, l2, rt = weight_prep.lowrank_split(d["wt"], r, 3)
    split = rel(A @ Q.mx_dequantize(*Q.mx_quantize(rt)).T + (x @ F.bf16_to_f64(l1)) @ F.bf16_to_f64(l2))
    As = Q.mx_dequantize(*Q.mx_quantize_smoothed(d["x"], d["inv_s"]))
    svdq = rel(As @ Q.mx_dequantize(*Q.mx_quantize(d["rt"])).T
               + (x @ F.bf16_to_f64(d["l1"])) @ F.bf16_to_f64(d["l2"]))
    assert svdq < 0.3 * plain and svdq < 0.3 * split, (plain, split, svdq)


def test_int4_channel_estimate_against_brute_force():
    """The Guide's per-channel INT4 estimate: every entry is the nearest of the 16
    grid points q * step (q = -8 .. 7, step = row amax / 7 floored at 1e-8), ties
    to the even q, found by exhaustive search in exact arithmetic."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((6, 40)) * np.exp(rng.uniform(-3, 3, (6, 1)))
    w[2] = 0.0                                   # an all-zero channel: step 1e-8, all zeros
    w[3, :8] = np.array([0.5, 1.5, -0.5, -2.5, 3.5, 7.0, -7.0, 2.0]) * (7.0 / 7.0)   # ties at step 1
    w[3, 8:] = 0.0
    est = weight_prep.int4_channel_estimate(w)
    for n in range(w.shape[0]):
        step = max(Fraction(float(np.abs(w[n]).max())) / 7, Fraction(1e-8))
        for k in range(w.shape[1]):
            v = Fraction(float(w[n, k]))
            q = min(range(-8, 8), key=lambda c: (abs(c * step - v), c & 1))
            assert Fraction(float(est[n, k])) == Fraction(float(q * step)) or \
                abs(Fraction(float(est[n, k])) - q * step) <= step * Fraction(2) ** -50, (n, k)


def test_guide_step1_factors_pins():
    """The Guide's literal Step-1 factors: (1) a weight already on its INT4 grid has
    no error to factor; (2) with an identity covariance the factors are the best
    rank-r approximation of the error (Eckart-Young: the residual norm is the
    discarded singular values, and beats another rank-r candidate); (3) scaling the
    covariance by a scales the factors' product by a (the product carries the
    covariance's units, which is why the page's residual W - L1 L2 is not an
    approximation of the quantization error)."""
    rng = np.random.default_rng(12)
    N, K, r = 24, 32, 4
    step = np.exp(rng.uniform(-2, 1, (N, 1)))
    q = rng.integers(-7, 8, (N, K)).astype(np.float64)   # |q| <= 7: the row amax is 7 steps
    q[:, 0] = 7.0                                 # the row amax is 7 steps: the grid is exact
    left, right, s = weight_prep.guide_step1_factors(q * step, np.eye(K), r)
    # only the rounding of amax / 7 separates the weight from its grid
    assert s[0] <= 1e-13 * np.abs(q * step).max() and np.abs(left @ right).max() <= 1e-13 * np.abs(q * step).max()
    w = rng.standard_normal((N, K))
    dw = w - weight_prep.int4_channel_estimate(w)
    left, right, s = weight_prep.guide_step1_factors(w, np.eye(K), r)
    err = np.linalg.norm(dw - left @ right)
    assert math.isclose(err, math.sqrt(np.sum(s[r:] ** 2)), rel_tol=1e-9)
    other = dw.copy()
    other[:, r:] = 0.0                            # a different rank-r matrix
    assert err < np.linalg.norm(dw - other)
    l3, r3, _ = weight_prep.guide_step1_factors(w, 3.0 * np.eye(K), r)
    assert np.allclose(l3 @ r3, 3.0 * (left @ right), rtol=1e-9, atol=1e-12)


def test_guide_step1_split_reconstructs_the_weight():
    d = weight_prep.attn_proj_calibrated(seed=5, M=32, K=128, N=96, calib=256)
    g = weight_prep.guide_step1_split(d["x_cal"], d["wt"], 8)
    w = F.bf16_to_f64(d["wt"])                                        # [N, K]
    left, right, _ = weight_prep.guide_step1_factors(w, np.cov(F.bf16_to_f64(d["x_cal"]).T), 8)
    exact = w - left @ right
    r = F.bf16_to_f64(g["rt"])
    assert np.all(np.abs(r - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)   # bf16 rounding only
    assert np.array_equal(g["l1"], synth.to_bf16_bits(right.T))
    assert np.array_equal(g["l2"], synth.to_bf16_bits(left.T))
